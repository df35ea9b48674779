"""Kernel-configuration sweep: correctness first, then speed, per shape.

    python -m dense_fp32_gemm_amd.sweep [--shapes M,N,K ...] [--configs 1,2,...]
                                        [--steps 10] [--warmup 3] [--csv out.csv]

For every shape, every configuration (all of them unless --configs names
some) first runs on quarter-step operands, whose product is exact in binary32
and therefore identical bit for bit whatever the summation order: each
configuration's C must equal, bit for bit, the C of a fixed reference kernel
(the vector-FMA configuration, written independently of the matrix-core
kernels), otherwise it is reported as failing and not timed.  (The parity
tests tie the vector-FMA kernel itself to the CPU oracle.)  Configurations that pass are then timed
on uniform[-1,1) operands (hipEvents around each call, after at least
--warmup calls and 0.2 s of warm-up) and ranked by mean time.  The plan the
shape rule makes (config -1) is checked and timed as one more candidate,
named auto:<configuration>, since it can differ from every forced
configuration (a remainder strip).  This is how the shape -> configuration table in
gemm_f32.hip is chosen; the Lecture 12 final-project page's sweep.cu follows
the same "correct first, then fast" order for its block/tile/coarsening
search.
"""
from __future__ import annotations

import argparse
import csv
import sys
import time

import numpy as np

from . import binding as gb
from . import inputs

DEFAULT_SHAPES = [(512, 512, 512), (1025, 1023, 1000), (1000, 1000, 1000),
                  (2048, 2048, 2048), (8192, 8192, 8192), (8192, 8192, 128),
                  (16384, 64, 4096), (64, 16384, 4096), (4096, 4096, 16384)]


REFERENCE_CONFIG = 0       # valu_64x64: the vector-FMA kernel


def _run(torch, config, A, B, C, stream):
    M, K = A.shape
    N = B.shape[1]
    return gb.gemm_f32_with_config(config, M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                   C.data_ptr(), N, stream.cuda_stream)


def sweep_shape(torch, shape, configs, steps, warmup, log=print):
    M, N, K = shape
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    qa, qb = inputs.quarter_step(M, N, K)
    A = torch.from_numpy(qa).to(dev)
    B = torch.from_numpy(qb).to(dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    ref = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    rc = _run(torch, REFERENCE_CONFIG, A, B, ref, stream)
    torch.cuda.synchronize()
    if rc != gb.GEMM_F32_OK or not bool(torch.isfinite(ref).all()):
        raise RuntimeError(f"reference kernel failed on {shape}: {gb.gemm_f32_status_string(rc)}")
    # The automatic plan (config -1) runs as a candidate of its own: it can
    # differ from every forced configuration (a remainder strip).  It is
    # checked and timed first, so that no slow forced configuration runs
    # just before it.
    _, plan = gb.gemm_f32_describe(-1, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N)
    strip = [w for w in plan.split() if w.startswith("strip_")]
    names = {c: gb.gemm_f32_config_name(c) for c in configs}
    names[-1] = "auto:" + (plan.split() or ["?"])[0] + "".join(" " + w for w in strip)
    passed = []
    for c in [-1] + list(configs):
        C.fill_(float("nan"))
        rc = _run(torch, c, A, B, C, stream)
        torch.cuda.synchronize()
        if rc != gb.GEMM_F32_OK:
            rows.append(dict(M=M, N=N, K=K, config=names[c], ok=False, auto=c == -1,
                             note=gb.gemm_f32_status_string(rc)))
            continue
        ok = bool(torch.equal(C, ref))
        if ok:
            passed.append(c)
        else:
            rows.append(dict(M=M, N=N, K=K, config=names[c], ok=False, auto=c == -1,
                             note="differs on quarter-step operands"))
    del A, B, qa, qb, ref
    ua, ub = inputs.uniform(M, N, K)
    A = torch.from_numpy(ua).to(dev)
    B = torch.from_numpy(ub).to(dev)
    del ua, ub
    flop = 2.0 * M * N * K
    nbytes = 4.0 * (M * K + K * N + M * N)
    for c in passed:
        # At least `warmup` calls and 0.2 s of them: short kernels must not be
        # timed while the clock is still ramping up.
        t0 = time.perf_counter()
        done = 0
        while done < warmup or time.perf_counter() - t0 < 0.2:
            for _ in range(1 if done < warmup else 10):
                _run(torch, c, A, B, C, stream)
                done += 1
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            _run(torch, c, A, B, C, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        row = dict(M=M, N=N, K=K, config=names[c], ok=True, note="", auto=c == -1,
                   ms_mean=float(ms.mean()), ms_median=float(np.median(ms)), ms_min=float(ms.min()),
                   tflops=flop / (ms.mean() * 1e-3) / 1e12, gbs=nbytes / (ms.mean() * 1e-3) / 1e9)
        rows.append(row)
    timed = sorted((r for r in rows if r["ok"]), key=lambda r: r["ms_mean"])
    for rank, r in enumerate(timed):
        r["rank"] = rank + 1
        log(f"{M:>6} {N:>6} {K:>6}  #{rank + 1:<2} {r['config']:<20} {r['ms_mean'] * 1e3:10.1f} us "
            f"{r['tflops']:8.2f} TFLOPS {r['gbs']:8.1f} GB/s{'  <- auto' if r['auto'] else ''}")
    for r in rows:
        if not r["ok"]:
            log(f"{M:>6} {N:>6} {K:>6}  FAIL {r['config']:<20} {r['note']}")
    del A, B, C
    torch.cuda.empty_cache()
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", nargs="*", default=None, help="M,N,K triples")
    ap.add_argument("--configs", default=None, help="comma-separated configuration indices")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--csv", default=None)
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 1
    shapes = ([tuple(int(x) for x in s.split(",")) for s in args.shapes] if args.shapes
              else DEFAULT_SHAPES)
    configs = ([int(c) for c in args.configs.split(",")] if args.configs
               else list(range(gb.gemm_f32_num_configs())))
    print("configs:", ", ".join(f"{c}={gb.gemm_f32_config_name(c)}" for c in configs), flush=True)
    all_rows = []
    for shp in shapes:
        all_rows += sweep_shape(torch, shp, configs, args.steps, args.warmup,
                                log=lambda s: print(s, flush=True))
    if args.csv:
        keys = ["M", "N", "K", "config", "ok", "rank", "auto", "ms_mean", "ms_median", "ms_min",
                "tflops", "gbs", "note"]
        with open(args.csv, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=keys, extrasaction="ignore")
            w.writeheader()
            for r in all_rows:
                w.writerow(r)
    return 0


if __name__ == "__main__":
    sys.exit(main())
