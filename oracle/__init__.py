"""Dense FP32 GEMM oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path
(``dense_fp32_gemm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, built with the host compiler):
the double-accumulating triple loop that the UIUC ECE408 Lecture 12 final
project page uses as its golden reference (project_template.cu, section 3),
generalised to row-major leading dimensions.  This module only marshals numpy
arrays into it.

Parity pins: both entry points are pinned by ``tests/test_oracle.py``
(identity, permutation, all-ones, rank-1, exact-integer, exact-rational,
brute force, and a float64 library cross-check), and planted mistakes in
``oracle.c`` are shown to fail those pins, so nothing here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

# The oracle must not be re-associated or contracted: -O2 without fast-math,
# and FMA contraction off.  OpenMP parallelises over output rows only.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SOURCE, out: str = LIBRARY, verbose: bool = False) -> str:
    """Compile ``src`` into the shared library ``out`` with gcc."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data if a.size else 0


def _row_stride(x: np.ndarray, rows: int, cols: int, name: str) -> int:
    """Row stride (elements) of a float32 row-major view of shape rows x cols."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.shape != (rows, cols):
        raise ValueError(f"{name} has shape {x.shape}, expected {(rows, cols)}")
    if rows and cols:
        if x.strides[1] != 4 or x.strides[0] % 4 or x.strides[0] < 0:
            raise ValueError(f"{name} must be row-major with unit column stride")
        return max(x.strides[0] // 4, cols)
    return max(cols, 1)


class Oracle:
    """numpy-facing wrapper of one build of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64 = ctypes.c_int64
        fp = ctypes.c_void_p
        lib.oracle_gemm_f32.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        fp, i64, fp, i64, fp, i64]
        lib.oracle_gemm_f32.restype = ctypes.c_int
        lib.oracle_gemm_f32_at.argtypes = [ctypes.c_int, fp, i64, fp, i64,
                                           i64, fp, fp, fp]
        lib.oracle_gemm_f32_at.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        self._lib = lib
        self.path = path

    def gemm(self, A: np.ndarray, B: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
        """C = A @ B by the double-accumulating definition; returns float32 C.

        A is M x K and B is K x N, float32, row-major; row strides may exceed
        the row length.  If ``out`` is given it must be an M x N float32
        row-major view; only that window is written.
        """
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        lda = _row_stride(A, M, K, "A")
        ldb = _row_stride(B, K, N, "B")
        if out is None:
            out = np.empty((M, N), dtype=np.float32)
        ldc = _row_stride(out, M, N, "out")
        rc = self._lib.oracle_gemm_f32(M, N, K, _ptr(A), lda, _ptr(B), ldb,
                                       _ptr(out), ldc)
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
        return out

    def gemm_at(self, A: np.ndarray, B: np.ndarray, rows, cols) -> np.ndarray:
        """The elements C(rows[t], cols[t]) of A @ B, each by the definition."""
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        lda = _row_stride(A, M, K, "A")
        ldb = _row_stride(B, K, N, "B")
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape or r.ndim != 1:
            raise ValueError("rows and cols must be 1-D and of equal length")
        if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
            raise IndexError("sample position outside the M x N output")
        out = np.empty(r.size, dtype=np.float32)
        self._lib.oracle_gemm_f32_at(K, _ptr(A), lda, _ptr(B), ldb, r.size,
                                     _ptr(r), _ptr(c), _ptr(out))
        return out

    def threads(self) -> int:
        """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
        return self._lib.oracle_threads()

    def set_threads(self, n: int) -> None:
        """Use n OpenMP threads from now on (the results do not depend on it)."""
        self._lib.oracle_set_threads(int(n))


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def gemm(A, B, out=None):
    return load().gemm(A, B, out)


def gemm_at(A, B, rows, cols):
    return load().gemm_at(A, B, rows, cols)


def threads() -> int:
    return load().threads()


def set_threads(n: int) -> None:
    load().set_threads(n)
