"""Scaling and roofline report for square FP32 GEMMs.

    python -m dense_fp32_gemm_amd.report [--max-n 8192] [--min-n 128]
                                         [--steps 20] [--warmup 10] [--csv out.csv]

For n = min_n, 2*min_n, ..., max_n this times C = A . B at n x n x n with the
configuration gemm_f32 selects, and prints one row per size:

  kernel, n, us (mean), TFLOP/s, % of the FP32 matrix peak,
  compulsory GB 4(3 n^2) / 1e9, arithmetic intensity FLOP/B,
  compulsory GB/s, roofline bound min(peak, AI * HBM bandwidth),
  fraction of that bound, workgroups per CU (occupancy), check.

The check column runs the same size on quarter-step operands, where the
product is exact in binary32 and so independent of the summation order, and
compares it bit for bit with the vector-FMA configuration, an independently
written kernel (the library itself never calls the CPU oracle).  The rows'
correctness is pinned separately: tests/test_parity.py runs gemm_f32 at
every size of the default report (n = 128 ... 8192) on the same quarter-step
operands and compares the whole of C bit for bit with the CPU oracle.  This
is the Lecture 12 final-project page's report_data.cu flow (sizes doubling,
a CSV row per size with FLOP rate, bytes, intensity, bandwidth and a check).
"""
from __future__ import annotations

import argparse
import csv
import sys
import time

import numpy as np

from . import binding as gb
from . import inputs

PEAK_TFLOPS = 157.3      # MI355X dense FP32 matrix peak
HBM_GBS = 8000.0         # MI355X HBM3E bandwidth
VALU_CONFIG = 0          # the vector-FMA kernel


def _gemm(config, A, B, C, stream):
    n = A.shape[0]
    return gb.gemm_f32_with_config(config, n, n, n, A.data_ptr(), n, B.data_ptr(), n,
                                   C.data_ptr(), n, stream.cuda_stream)


def row_for(torch, n, steps, warmup):
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    qa, qb = inputs.quarter_step(n, n, n)
    A = torch.from_numpy(qa).to(dev)
    B = torch.from_numpy(qb).to(dev)
    C = torch.empty((n, n), dtype=torch.float32, device=dev)
    R = torch.empty((n, n), dtype=torch.float32, device=dev)
    rc = _gemm(-1, A, B, C, stream) or _gemm(VALU_CONFIG, A, B, R, stream)
    if rc:
        raise gb.GemmError(rc)
    torch.cuda.synchronize()
    check = "bit-exact" if torch.equal(C, R) else "MISMATCH"     # against the vector-FMA kernel
    del qa, qb
    ua, ub = inputs.uniform(n, n, n)
    A.copy_(torch.from_numpy(ua))
    B.copy_(torch.from_numpy(ub))
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < 0.2:
        _gemm(-1, A, B, C, stream)
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        _gemm(-1, A, B, C, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    _, desc = gb.gemm_f32_describe(-1, n, n, n, A.data_ptr(), n, B.data_ptr(), n, C.data_ptr(), n)
    name = desc.split()[0]
    cfg = gb.config_names().index(name)
    occ = gb.gemm_f32_config_info(cfg, occupancy=True)["blocks_per_cu"]
    flop = 2.0 * n ** 3
    nbytes = 4.0 * 3 * n * n
    tflops = flop / (ms * 1e-3) / 1e12
    ai = flop / nbytes
    roof = min(PEAK_TFLOPS, ai * HBM_GBS / 1e3)
    return dict(kernel=name, n=n, us=ms * 1e3, tflops=tflops, pct_peak=100 * tflops / PEAK_TFLOPS,
                gb=nbytes / 1e9, ai=ai, gbs=nbytes / (ms * 1e-3) / 1e9, roof_tflops=roof,
                frac_of_roof=tflops / roof, blocks_per_cu=occ, check=check)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--min-n", type=int, default=128)
    ap.add_argument("--max-n", type=int, default=8192)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--csv", default=None)
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("the report needs a GPU", file=sys.stderr)
        return 1
    keys = ["kernel", "n", "us", "tflops", "pct_peak", "gb", "ai", "gbs", "roof_tflops",
            "frac_of_roof", "blocks_per_cu", "check"]
    print(" ".join(f"{k:>14}" for k in keys), flush=True)
    rows = []
    n = args.min_n
    while n <= args.max_n:
        r = row_for(torch, n, args.steps, args.warmup)
        rows.append(r)
        print(" ".join(f"{r[k]:>14.4g}" if isinstance(r[k], float) else f"{r[k]:>14}" for k in keys),
              flush=True)
        torch.cuda.empty_cache()
        n *= 2
    if args.csv:
        with open(args.csv, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=keys)
            w.writeheader()
            w.writerows(rows)
    return 0 if all(r["check"] == "bit-exact" for r in rows) else 2


if __name__ == "__main__":
    sys.exit(main())
