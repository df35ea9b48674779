"""Builds libgemm_f32.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m dense_fp32_gemm_amd.build [--verbose] [--poison-lds]

hipcc compiles for gfx950 only.  Packed-FP32 instruction selection is turned
off for device code (-Xclang -target-feature -Xclang -packed-fp32-ops); the
host pass prints a harmless "not a recognized feature" warning for it.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "gemm_f32.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgemm_f32.so")
ARCH = "gfx950"

HIPFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-command-line-argument",
]


# Debug build: -DGEMM_F32_POISON_LDS makes the kernels set every LDS slot to
# NaN before it is refilled or first written (see kPoisonLds in the source),
# so a stale LDS read shows up as NaN in C.  gemm_f32_describe() then ends
# with " lds=poisoned".
POISON_LDS = "-DGEMM_F32_POISON_LDS"


def command(out: str, extra: list[str] | None = None, poison_lds: bool = False) -> list[str]:
    """The hipcc command line that builds the library into `out`."""
    flags = [*HIPFLAGS, *([POISON_LDS] if poison_lds else []), *(extra or [])]
    return ["hipcc", *flags, "-I", INCLUDE, *SOURCES, "-o", out]


def build(verbose: bool = False, extra: list[str] | None = None, poison_lds: bool = False) -> str:
    """Compile the library; returns its path.  Always recompiles."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = command(tmp, extra, poison_lds)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, poison_lds="--poison-lds" in sys.argv)
    print(LIBRARY)
