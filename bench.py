#!/usr/bin/env python3
"""Benchmark of the tile-signaled GEMM paths on one MI355X.

Default workload: AllGather + GEMM at one rank's TP=8 share of a Llama-style
MLP up-projection (A 8192x4096 bf16 gathered from 8 row chunks of 1024, one
local and seven written by the concurrent copy kernel; B 4096x1792 bf16;
fp32 accumulate, bf16 out).  One step = one gemm_ag_overlap call in overlap
mode with its inputs already resident in HBM.  The same kernels are also timed
serialized (copy, then GEMM), GEMM-only and copy-only, for the speedup, the
"within 10% of GEMM-only" ratio and the overlap ratio.

Prints one JSON line (see --help for options).  Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "overlapped TFLOP/s, % bf16 MFMA peak, speedup vs serialized copy+GEMM"


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama_ag", choices=["llama_ag"])
    p.add_argument("--aux-cus", type=int, default=0, help="copy-kernel CUs (0 = default, -1 = shared)")
    p.add_argument("--tile", type=int, default=0)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--sweep", action="store_true", help="also print per-configuration timings to stderr")
    return p.parse_args()


def _cpu_baseline(inp, M, N, K, R):
    """The oracle as it stands, on this host's cores: full AG + GEMM in float64."""
    import numpy as np
    import oracle
    from synth.gen import split_chunks
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    loc, peers = split_chunks(inp["a"], R, 0)
    times = []
    t_end = time.perf_counter() + 20.0
    while len(times) < 3 and (not times or time.perf_counter() < t_end):
        t0 = time.perf_counter()
        oracle.ag_gemm(loc, peers, inp["b"], R, 0)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": 2.0 * M * N * K / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the full workload (AllGather + {M}x{N}x{K} GEMM, float64 numpy), "
                      f"median of {len(times)} runs, {t:.2f} s each"}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(peers are stood in for by buffers in local HBM).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tile_level_communication_signaled_amd as tsg
    from synth import CONFIGS, ag_inputs
    from synth.gen import split_chunks

    cfg = CONFIGS[args.workload]
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    rank = 0
    flops = 2.0 * M * N * K

    # Two resident input sets, used alternately, so that back-to-back steps do
    # not find their operands in the 256 MB Infinity Cache.
    sets = []
    host_inp = None
    for s in range(2):
        inp = ag_inputs(M, K, N, R, rank=rank, seed=cfg["seed"] + 100 * s)
        if s == 0:
            host_inp = inp
        loc, peers = split_chunks(inp["a"], R, rank)
        d = {
            "loc": torch.from_numpy(loc.view(np.int16)).cuda(),
            "peers": torch.from_numpy(peers.view(np.int16)).cuda(),
            "b": torch.from_numpy(inp["b"].view(np.int16)).cuda(),
            "full": torch.empty((M, K), dtype=torch.int16, device="cuda"),
            "c": torch.empty((M, N), dtype=torch.int16, device="cuda"),
        }
        sets.append(d)
    torch.cuda.synchronize()

    ctx = tsg.Context(0)
    opts = tsg.Opts(aux_cus=args.aux_cus, tile=args.tile)

    def call(i, mode):
        d = sets[i % 2]
        tsg.gemm_ag_overlap(ctx, d["loc"], d["peers"], d["full"], d["b"], d["c"], tsg.BF16, M, N, K, R, rank,
                            opts=opts, mode=mode)

    def timed(mode, steps, warmup, kernel=None):
        for i in range(warmup):
            call(i, mode)
        if ctx.check() != tsg.OK:
            raise RuntimeError(ctx.last_error())
        ctx.enable_kernel_timing(kernel is not None)
        kms = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            call(i, mode)
            if kernel is not None:
                kms.append(ctx.kernel_ms(kernel))   # waits for this step's kernel event
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        ctx.enable_kernel_timing(False)
        st = ctx.check()
        if st != tsg.OK:
            raise RuntimeError(ctx.last_error())
        return dt * 1e3, (float(np.mean(kms)) if kms else None)

    # Timed region of the headline number: K overlap steps, nothing else.
    for i in range(args.warmup):
        call(i, tsg.OVERLAP)
    if ctx.check() != tsg.OK:
        raise RuntimeError(ctx.last_error())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i, tsg.OVERLAP)
    torch.cuda.synchronize()
    ms_overlap = (time.perf_counter() - t0) / args.steps * 1e3
    if ctx.check() != tsg.OK:
        raise RuntimeError(ctx.last_error())

    # Reference modes and per-kernel durations (HIP events on the kernels' own streams).
    _, gemm_ms_in_overlap = timed(tsg.OVERLAP, args.steps, 2, kernel=0)
    ms_serial, _ = timed(tsg.SERIAL, args.steps, 2)
    ms_compute, gemm_ms_alone = timed(tsg.COMPUTE_ONLY, args.steps, 2, kernel=0)
    ms_comm, copy_ms = timed(tsg.COMM_ONLY, args.steps, 2, kernel=1)

    tflops = flops / (ms_overlap * 1e-3) / 1e12
    achieved = flops / (gemm_ms_in_overlap * 1e-3) / 1e12
    copy_bytes = 2 * (M * K * 2)   # every chunk (local included) read once and written once
    gemm_bytes = M * K * 2 + K * N * 2 + M * N * 2
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_overlap, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/64 bf16 operands, two resident input sets used alternately)",
        "config": {"workload": f"{args.workload}: AllGather+GEMM, A {M}x{K} bf16 in {R} row chunks of {M // R} "
                               f"(rank {rank} local, {R - 1} copied in by the concurrent copy kernel), "
                               f"B {K}x{N} bf16, fp32 accumulate, bf16 out",
                   "M": M, "N": N, "K": K, "R": R, "aux_cus": args.aux_cus, "tile": args.tile},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "speedup_vs_serial": round(ms_serial / ms_overlap, 4),
        "overlap_vs_compute_only": round(ms_overlap / ms_compute, 4),
        "overlap_ratio": round((ms_compute + ms_comm - ms_overlap) / ms_comm, 4),
        "ms": {"overlap": round(ms_overlap, 5), "serial": round(ms_serial, 5),
               "compute_only": round(ms_compute, 5), "comm_only": round(ms_comm, 5),
               "gemm_kernel_in_overlap": round(gemm_ms_in_overlap, 5),
               "gemm_kernel_alone": round(gemm_ms_alone, 5), "copy_kernel": round(copy_ms, 5)},
        "copy_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "ag_gemm_kernel", "algorithmic_bytes": gemm_bytes},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(host_inp, M, N, K, R)
    print(json.dumps(out), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
