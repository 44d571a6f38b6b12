#!/usr/bin/env python3
"""Benchmark of the tile-signaled GEMM paths on one MI355X.

Headline workload (the JSON line's `value`): AllGather + GEMM at one rank's
TP=8 share of a Llama-style MLP up-projection -- A 8192x4096 bf16 gathered
from 8 row chunks of 1024 (the local one and seven written by the concurrent
copy kernel), B 4096x1792 bf16, fp32 accumulate, bf16 out.  One step = one
gemm_ag_overlap call in overlap mode with every input already resident in
HBM; K steps are timed with the wall clock between two device
synchronisations.  The same kernels are also timed serialized (copy, then
GEMM), GEMM-only and copy-only, giving the speedup over serial, the ratio to
GEMM-only and the overlap ratio (comp + comm - overlap) / comm.

`paths` also holds the AllGather + GEMM with the copy paced at seven xGMI
links' rate (arrival_gbps), and reports the same four modes for every path at its full-size
workload: AG+GEMM, GEMM+RS (8192x1792 @ 1792x4096, 7 fp32 peer partials),
the CTA-pipelined MLP (2048x8192 @ 8192x4096, GELU, @ 4096x8192) and MoE
(4096 tokens, hidden 4096, 8 experts of 4096x1408 / 1408x4096, top-2 Zipf),
the latter also with its y staging in bf16.

Prints one JSON line.  Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "overlapped TFLOP/s, % bf16 MFMA peak, speedup vs serialized copy+GEMM"
XGMI_GBPS = 1071            # arrival pacing of the xGMI-paced AG line: 7 links x ~153 GB/s
CSRC = os.path.join(ROOT, "tile_level_communication_signaled_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--aux-cus", type=int, default=0, help="copy-kernel CUs of the headline (0 = default, -1 = shared)")
    p.add_argument("--tile", type=int, default=0)
    p.add_argument("--paths", default="all", choices=["all", "ag"], help="also time the other three paths")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--headline-only", action="store_true",
                   help="time only the headline overlap steps (for kernel traces)")
    p.add_argument("--trace-path", choices=["gemm_rs", "mlp2", "moe", "moe_bf16_staging", "moe_ag", "ag_kv_attention",
                                            "ag_copy_engine"],
                   help="time only this path's overlap steps (for kernel traces of that path), print one "
                        "JSON line and exit")
    p.add_argument("--counters", action="store_true",
                   help="counter-collection run: the profiler serialises kernels, so every path runs in "
                        "compute-only mode and in comm-only mode (K steps each) instead of overlapped, then "
                        "one plain 1 GiB device copy of known size calibrates the byte counters; prints "
                        "nothing")
    p.add_argument("--timeline", action="store_true",
                   help="print each path's device timeline of one overlapped call (units active and "
                        "waiting per time bin) as markdown, and exit")
    p.add_argument("--library-gemms", action="store_true",
                   help="time torch.matmul (hipBLASLt) on the plain GEMMs of the AllGather, ReduceScatter and "
                        "MLP paths, and torch's scaled_dot_product_attention (flash and memory-efficient "
                        "backends only) on the attention workload, beside this library's compute-only calls of "
                        "those paths; print a markdown table and exit (a comparison only: no path calls them)")
    p.add_argument("--summarize-mfma", metavar="CSV",
                   help="no GPU: turn the counter_collection.csv of a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                        "GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES SQ_LDS_BANK_CONFLICT "
                        "SQ_LDS_IDX_ACTIVE run of --counters into a markdown table per kernel and exit")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: turn the counter_collection.csv files of two rocprofv3 --pmc runs of "
                        "--counters (FETCH_SIZE, then WRITE_SIZE) into the traffic record and exit")
    return p.parse_args()


# Sources the AllGather + GEMM kernels are compiled from: a traffic record
# measured on other code does not apply.
AG_SOURCES = ("ag.hip", "tsg_gemm.hpp", "tsg_device.hpp", "tsg_copy.hpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in AG_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters, or
    None when the record is missing or older than the current sources."""
    try:
        rec = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["bytes_per_launch"])


CALIB_BYTES = 1 << 30   # the plain device copy that --counters runs: 1 GiB read, 1 GiB written


KERNELS = ("ag_gemm_kernel", "ag_copy_kernel", "rs_gemm_kernel", "rs_reduce_kernel", "mlp_gemm1_kernel",
           "mlp_gemm2_kernel", "mlp_fused_kernel", "moe_count_kernel", "moe_place_kernel", "moe_producer_kernel",
           "moe_combine_kernel", "moe_rb_order_kernel", "moe_ag_kernel", "ag_attn_kernel", "ag_attn_copy_kernel")


def summarize_counters(fetch_csv: str, write_csv: str, out_path: str = TRAFFIC) -> dict:
    """Per-launch HBM bytes of the library's kernels from two rocprofv3 --pmc
    runs of --counters.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch and averaged per
    kernel.  Each counter is scaled by the factor that makes it read exactly
    1 GiB on the plain 1 GiB device copy (the largest __amd_rocclr_copyBuffer
    dispatch) of the same run."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    rec = {"source_hash": source_hash(), "calibration_bytes": CALIB_BYTES, "kernels": {}}
    totals = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        acc = per_kernel(path, name)
        calib = max(v for k, vs in acc.items() if k.startswith("__amd_rocclr_copyBuffer") for v in vs)
        scale = CALIB_BYTES / (calib * 1024.0)
        rec[name + "_scale"] = round(scale, 5)
        for short in KERNELS:
            vs = [v for k, lst in acc.items() if short in k for v in lst]
            if vs:
                totals.setdefault(short, {})[name] = sum(vs) / len(vs) * 1024.0 * scale
                totals[short]["launches_" + name] = len(vs)
    for short, t in totals.items():
        rec["kernels"][short] = {"fetch_bytes": int(t["FETCH_SIZE"]), "write_bytes": int(t["WRITE_SIZE"]),
                                 "bytes_per_launch": int(t["FETCH_SIZE"] + t["WRITE_SIZE"]),
                                 "launches": t["launches_FETCH_SIZE"]}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def summarize_mfma(csv_path: str) -> str:
    """Markdown table per kernel from one rocprofv3 --pmc run of --counters:
    active cycles = GRBM_GUI_ACTIVE summed over the 8 XCDs / 8 (the
    dispatch's duration in GPU clocks), MFMA utilisation =
    SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs), MFMA GFLOP =
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, LDS conflict % = SQ_LDS_BANK_CONFLICT
    / SQ_LDS_IDX_ACTIVE; means over each kernel's dispatches."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        short = next((k for k in KERNELS if k in r["Kernel_Name"]), None)
        if short is None:
            continue
        d = per.setdefault(short, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["| kernel | launches | active cycles | MFMA busy cycles | MFMA util % | MFMA GFLOP | LDS conflict % |",
             "|---|---|---|---|---|---|---|"]
    for short in KERNELS:
        if short not in per:
            continue
        ds = list(per[short].values())
        mean = lambda key: sum(d.get(key, 0.0) for d in ds) / len(ds)
        active = mean("GRBM_GUI_ACTIVE") / 8
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
        util = 100.0 * busy / (active * 1024) if active else 0.0
        gflop = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / 1e9
        lds = mean("SQ_LDS_IDX_ACTIVE")
        conf = 100.0 * mean("SQ_LDS_BANK_CONFLICT") / lds if lds else 0.0
        lines.append(f"| {short} | {len(ds)} | {active:,.0f} | {busy:,.0f} | {util:.1f} | {gflop:.2f} | {conf:.2f} |")
    return "\n".join(lines)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 0) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _time_host(fn, budget_s: float, min_runs: int = 3):
    """Median seconds of fn() over repeated runs: at least min_runs, and more
    until about budget_s seconds have passed."""
    import numpy as np
    times = []
    t_end = time.perf_counter() + budget_s
    while len(times) < min_runs or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def _cpu_baselines(ag_host, budget_s: float = 8.0) -> dict:
    """The oracle as it stands, timed on this host's cores for every workload
    (float64 numpy, the BLAS's own threads), in the unit of each path's GPU
    line; the tiny AllGather+GEMM also on one thread.  Bounded samples: every
    entry runs the whole workload, repeated for about its time budget."""
    import oracle
    from synth import CONFIGS, ag_inputs, mlp2_inputs, moe_inputs, rs_inputs
    from synth.gen import split_chunks
    cores, model = _blas_threads(), _cpu_model()
    out = {}

    def entry(flops, t, runs, what, threads=cores):
        return {"value": round(flops / t / 1e12, 4), "unit": "TFLOP/s", "ms": round(t * 1e3, 3),
                "cores": int(threads), "cpu": model, "kind": "oracle",
                "sample": f"{what}, float64 numpy on the host, median of {runs} runs"}

    c1 = CONFIGS["tiny_ag"]
    M, N, K, R = c1["M"], c1["N"], c1["K"], c1["R"]
    inp = ag_inputs(M, K, N, R, rank=0, seed=c1["seed"], dist="uniform")
    loc, peers = split_chunks(inp["a"], R, 0)
    f1 = lambda: oracle.ag_gemm(loc, peers, inp["b"], R, 0)
    t, n = _time_host(f1, 2.0)
    out["tiny_ag"] = entry(2.0 * M * N * K, t, n, f"AllGather + {M}x{N}x{K} GEMM, R={R}")
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t, n = _time_host(f1, 2.0)
        out["tiny_ag_1thread"] = entry(2.0 * M * N * K, t, n, f"AllGather + {M}x{N}x{K} GEMM, R={R}", 1)
    except Exception:  # pragma: no cover
        pass

    c2 = CONFIGS["llama_ag"]
    M, N, K, R = c2["M"], c2["N"], c2["K"], c2["R"]
    loc, peers = split_chunks(ag_host["a"], R, 0)
    t, n = _time_host(lambda: oracle.ag_gemm(loc, peers, ag_host["b"], R, 0), budget_s)
    out["llama_ag"] = entry(2.0 * M * N * K, t, n, f"the full workload (AllGather + {M}x{N}x{K} GEMM, R={R})")

    c3 = CONFIGS["gemm_rs"]
    M, N, K, R = c3["M"], c3["N"], c3["K"], c3["R"]
    inp = rs_inputs(M, K, N, R, rank=0, seed=c3["seed"])
    t, n = _time_host(lambda: oracle.gemm_rs(inp["x"], inp["w"], inp["peer_partials"], R, 0), budget_s / 2, 2)
    out["gemm_rs"] = entry(2.0 * M * N * K, t, n, f"the full workload ({M}x{N}x{K} GEMM + reduce of {R} chunks)")

    c4 = CONFIGS["mlp2"]
    M, K1, N1, N2 = c4["M"], c4["K1"], c4["N1"], c4["N2"]
    inp = mlp2_inputs(M, K1, N1, N2, seed=c4["seed"])
    t, n = _time_host(lambda: oracle.mlp2(inp["x"], inp["w1"], inp["w2"]), budget_s / 2, 2)
    out["mlp2"] = entry(2.0 * M * N1 * K1 + 2.0 * M * N2 * N1, t, n,
                        f"the full workload ({M}x{K1} @ {K1}x{N1}, GELU, @ {N1}x{N2})")

    c5 = CONFIGS["moe"]
    T, Hh, I, E, k = c5["T"], c5["H"], c5["I"], c5["E"], c5["k"]
    inp = moe_inputs(T, Hh, I, E, k=k, seed=c5["seed"], zipf=c5["zipf"])
    t, n = _time_host(lambda: oracle.moe_expert_combine(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_up"],
                                                        inp["w_down"]), budget_s / 2, 2)
    out["moe"] = entry(4.0 * T * k * Hh * I, t, n,
                       f"the full workload ({T} tokens, top-{k} of {E} experts {Hh}x{I} / {I}x{Hh}, combine)")

    # the gather side of the same layer: 4096 tokens from 8 ranks, gather,
    # up projection, SiLU
    R6 = 8
    loc6, peers6 = split_chunks(inp["x"], R6, 0)
    t, n = _time_host(lambda: oracle.moe_ag_up(loc6, peers6, R6, 0, inp["topk_ids"], inp["w_up"]), budget_s / 2, 2)
    out["moe_ag"] = entry(2.0 * T * k * Hh * I, t, n,
                          f"the full workload (AllGather of {T} tokens from {R6} ranks, gather, "
                          f"top-{k} of {E} experts {Hh}x{I}, SiLU)")

    # AllGather KV + attention: 2048 queries over the 16384-token context;
    # the sample is 4 of the 32 heads (the oracle's cost is per head), with
    # the rate scaled to the sample's own FLOPs
    import numpy as np
    from synth import f32_to_bf16_bits
    S7, R7, D7, h7 = 16384, 8, 128, 4
    sl7 = S7 // R7
    rng = np.random.default_rng(7)
    mk = lambda shape: f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    q7, kf7, vf7 = mk((sl7, h7, D7)), mk((S7, h7, D7)), mk((S7, h7, D7))
    kl7, kp7 = split_chunks(kf7, R7, 0)
    vl7, vp7 = split_chunks(vf7, R7, 0)
    t, n = _time_host(lambda: oracle.ag_kv_attention(q7, kl7, kp7, vl7, vp7, R7, 0), budget_s / 2, 2)
    out["ag_kv_attention"] = entry(4.0 * sl7 * S7 * D7 * h7, t, n,
                                   f"{h7} of the 32 heads ({sl7} queries over the gathered {S7}-token context, "
                                   f"D={D7}, {R7} ranks)")
    return out


class Timer:
    """Times calls of one path in each mode: milliseconds per call over
    back-to-back calls (stream-ordered throughput, as in the headline), plus
    the main/aux kernel durations that the library measures with events on
    the kernels' own streams."""

    def __init__(self, torch, tsg, ctx, fn):
        self.torch, self.tsg, self.ctx, self.fn = torch, tsg, ctx, fn

    def _check(self):
        if self.ctx.check() != self.tsg.OK:
            raise RuntimeError(self.ctx.last_error())

    def modes(self, modes, n, rounds=3, warmup=3):
        """ms per call for each mode: the modes are interleaved over `rounds`
        rounds of n back-to-back calls each (so a clock change between modes
        does not bias one of them) and the median round is kept."""
        torch = self.torch
        for m in modes:
            for i in range(warmup):
                self.fn(i, m)
        self._check()
        got = {m: [] for m in modes}
        for _ in range(rounds):
            for m in modes:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i in range(n):
                    self.fn(i, m)
                torch.cuda.synchronize()
                got[m].append((time.perf_counter() - t0) / n * 1e3)
        self._check()
        return {m: sorted(v)[len(v) // 2] for m, v in got.items()}

    def per_call(self, modes, n, warmup=3):
        """Per-call device time of each mode from events recorded on the
        caller's stream around each call (fork to join), n calls back to
        back: {mode: (p10, p50, p90) in ms}."""
        torch = self.torch
        out = {}
        for m in modes:
            for i in range(warmup):
                self.fn(i, m)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(evs):
                a.record()
                self.fn(i, m)
                b.record()
            torch.cuda.synchronize()
            v = sorted(a.elapsed_time(b) for a, b in evs)
            out[m] = (v[len(v) // 10], v[len(v) // 2], v[(9 * len(v)) // 10])
        self._check()
        return out

    def kernels(self, mode, n, which, spread=None):
        """Median kernel ms (library events) over n calls, per kernel slot;
        with a dict `spread`, also its p10 and p90 per slot."""
        torch, ctx = self.torch, self.ctx
        kms = {k: [] for k in which}
        ctx.enable_kernel_timing(True)
        for i in range(n):
            self.fn(i, mode)
            for k in which:
                kms[k].append(ctx.kernel_ms(k))
        torch.cuda.synchronize()
        ctx.enable_kernel_timing(False)
        self._check()
        if spread is not None:
            for k, v in kms.items():
                v = sorted(v)
                spread[k] = (v[len(v) // 10], v[(9 * len(v)) // 10])
        return {k: sorted(v)[len(v) // 2] for k, v in kms.items()}


def _summary(flops, hbm_bytes, t):
    """t: dict mode -> ms per call, back to back (None when the mode does not apply)."""
    ov, se, co, cm = t["overlap"], t["serial"], t["compute_only"], t.get("comm_only")
    out = {
        "ms": {k: (None if v is None else round(v, 5)) for k, v in t.items()},
        "tflops": round(flops / (ov * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100.0 * flops / (ov * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "hbm_GBps_algorithmic": round(hbm_bytes / (ov * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * hbm_bytes / (ov * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "speedup_vs_serial": round(se / ov, 4),
        "overlap_vs_compute_only": round(ov / co, 4),
        "flops": int(flops),
        "hbm_bytes_algorithmic": int(hbm_bytes),
    }
    if cm:
        out["overlap_ratio"] = round((co + cm - ov) / cm, 4)
    return out


def _path_line(tsg, timer, flops, nbytes, modes, n):
    """One path's line: back-to-back ms per call of each mode (median of
    interleaved rounds), the rates and ratios of _summary, and the per-call
    p10 / p50 / p90 of each mode."""
    names = {tsg.OVERLAP: "overlap", tsg.SERIAL: "serial", tsg.COMPUTE_ONLY: "compute_only",
             tsg.COMM_ONLY: "comm_only"}
    tm = timer.modes(modes, n)
    pc = timer.per_call(modes, max(n, 20))
    t = {"overlap": tm.get(tsg.OVERLAP), "serial": tm.get(tsg.SERIAL),
         "compute_only": tm.get(tsg.COMPUTE_ONLY), "comm_only": tm.get(tsg.COMM_ONLY)}
    if t["serial"] is None or t["compute_only"] is None:
        ov = t["overlap"]
        out = {"ms": {k: round(v, 5) for k, v in t.items() if v is not None},
               "tflops": round(flops / (ov * 1e-3) / 1e12, 2),
               "pct_bf16_peak": round(100.0 * flops / (ov * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
               "hbm_GBps_algorithmic": round(nbytes / (ov * 1e-3) / 1e9, 1)}
    else:
        out = _summary(flops, nbytes, t)
    out["ms_per_call_p10_p50_p90"] = {names[m]: [round(x, 5) for x in pc[m]] for m in modes}
    return out


def _path_ag(torch, tsg, ctx, cfg, n, opts, seed_sets=2):
    import numpy as np
    from synth import ag_inputs
    from synth.gen import split_chunks
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    sets, host = [], None
    for s in range(seed_sets):
        inp = ag_inputs(M, K, N, R, rank=0, seed=cfg["seed"] + 100 * s)
        host = host or inp
        loc, peers = split_chunks(inp["a"], R, 0)
        sets.append({"loc": torch.from_numpy(loc.view(np.int16)).cuda(),
                     "peers": torch.from_numpy(peers.view(np.int16)).cuda(),
                     "b": torch.from_numpy(inp["b"].view(np.int16)).cuda(),
                     "full": torch.empty((M, K), dtype=torch.int16, device="cuda"),
                     "c": torch.empty((M, N), dtype=torch.int16, device="cuda")})

    def fn(i, mode, o=None):
        d = sets[i % len(sets)]
        tsg.gemm_ag_overlap(ctx, d["loc"], d["peers"], d["full"], d["b"], d["c"], tsg.BF16, M, N, K, R, 0,
                            opts=o if o is not None else opts, mode=mode)
    flops = 2.0 * M * N * K
    gemm_bytes = M * K * 2 + K * N * 2 + M * N * 2
    copy_bytes = 2 * M * K * 2
    return fn, flops, gemm_bytes, copy_bytes, host


def _moe_remote_first(torch, tsg, ctx, fn, flops, nbytes, n, ep_ranks=8, ep_rank=7):
    """The MoE expert compute + combine with remote-critical tiles first
    (tokens from 8 source ranks, this rank 7) beside the plain order: the
    overlapped time of each, and from one call's device timeline of each, when
    the last down tile of a remote-critical row block published its ready
    signal (from then on every remote-bound output could be on its way), the
    mean of those tiles' ready times, and when the last tile of all was
    ready, in microseconds from the call's first record.
    The blocks are classed by the source-rank masks the call left in the
    workspace."""
    import numpy as np
    ws, dims = fn.workspace
    lay = tsg.moe_workspace_layout(dims)
    prio = tsg.Opts(ep_ranks=ep_ranks, ep_rank=ep_rank)
    out = {"ep_ranks": ep_ranks, "ep_rank": ep_rank}
    for label, opts in (("plain", tsg.Opts()), ("remote_first", prio)):
        line = _path_line(tsg, Timer(torch, tsg, ctx, lambda i, mode, o_=None, o=opts: fn(i, mode, o)), flops,
                          nbytes, (tsg.OVERLAP,), n)
        tl = tsg.Opts(timeline=1, ep_ranks=opts.ep_ranks, ep_rank=opts.ep_rank)
        fn(0, tsg.OVERLAP, tl)
        if ctx.check() != tsg.OK:
            raise RuntimeError(ctx.last_error())
        recs = np.array(ctx.timeline(), dtype=np.uint64)
        if label == "plain":
            # the masks: one more call with the order on, timeline off
            fn(0, tsg.OVERLAP, prio)
            if ctx.check() != tsg.OK:
                raise RuntimeError(ctx.last_error())
        w = ws.cpu().numpy()
        n_rb = int(w[lay["meta"]:lay["meta"] + 4].view(np.int32)[0])
        mask = w[lay["rb_mask"]:lay["rb_mask"] + 4 * n_rb].view(np.uint32)
        remote = (mask & ~np.uint32(1 << ep_rank)) != 0
        kind = (recs[:, 0] >> np.uint64(56)).astype(np.int64)
        rb = ((recs[:, 0] & np.uint64(0xFFFFFFFF)) >> np.uint64(16)).astype(np.int64)
        t0 = recs[:, 1].astype(np.int64).min()
        end = recs[:, 3].astype(np.int64)
        down = kind == 8
        rem = down & np.isin(rb, np.nonzero(remote)[0])
        # device wall clock: 100 ticks per microsecond
        line["remote_tiles_ready_us"] = round(float(end[rem].max() - t0) / 100.0, 2)
        line["remote_tiles_mean_ready_us"] = round(float((end[rem] - t0).mean()) / 100.0, 2)
        line["all_tiles_ready_us"] = round(float(end[down].max() - t0) / 100.0, 2)
        line["call_us"] = round(float(end.max() - t0) / 100.0, 2)
        out["remote_blocks"], out["blocks"] = int(remote.sum()), n_rb
        out[label] = line
    return out


def _other_paths(torch, tsg, ctx):
    """The GEMM+RS, MLP and MoE paths at full size: name -> (fn(i, mode,
    opts=None), flops, algorithmic HBM bytes, modes the path has)."""
    import numpy as np
    from synth import CONFIGS, mlp2_inputs, moe_inputs, rs_inputs
    dv = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    out = {}

    c3 = CONFIGS["gemm_rs"]
    M, N, K, R = c3["M"], c3["N"], c3["K"], c3["R"]
    inp = rs_inputs(M, K, N, R, rank=0, seed=c3["seed"])
    x, w, pp = dv(inp["x"]), dv(inp["w"]), dv(inp["peer_partials"])
    P = torch.empty((M, N), dtype=torch.float32, device="cuda")
    o = torch.empty((M // R, N), dtype=torch.float32, device="cuda")
    rs_fn = lambda i, mode, opts=None: tsg.gemm_rs_overlap(ctx, x, w, P, pp, o, M, N, K, R, 0, opts=opts, mode=mode)
    mr = M // R
    rs_bytes = M * K * 2 + K * N * 2 + M * N * 4 + (R - 1) * mr * N * 4 + 2 * mr * N * 4
    out["gemm_rs"] = (rs_fn, 2.0 * M * N * K, rs_bytes,
                      (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY))

    c4 = CONFIGS["mlp2"]
    M4, K1, N1, N2 = c4["M"], c4["K1"], c4["N1"], c4["N2"]
    inp = mlp2_inputs(M4, K1, N1, N2, seed=c4["seed"])
    dx, d1, d2 = dv(inp["x"]), dv(inp["w1"]), dv(inp["w2"])
    h = torch.empty((M4, N1), dtype=torch.int16, device="cuda")
    y = torch.empty((M4, N2), dtype=torch.float32, device="cuda")
    mlp_fn = lambda i, mode, opts=None: tsg.mlp2_pipelined(ctx, dx, d1, h, d2, y, M4, K1, N1, N2, opts=opts,
                                                          mode=mode)
    mlp_flops = 2.0 * M4 * N1 * K1 + 2.0 * M4 * N2 * N1
    mlp_bytes = M4 * K1 * 2 + K1 * N1 * 2 + 2 * M4 * N1 * 2 + N1 * N2 * 2 + M4 * N2 * 4
    out["mlp2"] = (mlp_fn, mlp_flops, mlp_bytes, (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY))

    c5 = CONFIGS["moe"]
    T, Hh, I, E, k = c5["T"], c5["H"], c5["I"], c5["E"], c5["k"]
    inp = moe_inputs(T, Hh, I, E, k=k, seed=c5["seed"], zipf=c5["zipf"])
    mx, ids, g, wu, wd = dv(inp["x"]), dv(inp["topk_ids"]), dv(inp["topk_w"]), dv(inp["w_up"]), dv(inp["w_down"])
    mo = torch.empty((T, Hh), dtype=torch.float32, device="cuda")
    cnt = torch.empty((E,), dtype=torch.int32, device="cuda")
    srt = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    wsb = tsg.workspace_bytes(tsg.OP_MOE, [T, Hh, I, E, k])
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    def moe_fn(i, mode, opts=None):
        tsg.moe_expert_combine(ctx, mx, ids, g, wu, wd, mo, cnt, srt, ws, wsb, T, Hh, I, E, k, opts=opts, mode=mode)
    moe_fn.workspace = (ws, [T, Hh, I, E, k])   # read back by the remote-critical line
    moe_flops = 4.0 * T * k * Hh * I
    moe_bytes = T * k * Hh * 2 + 2 * E * Hh * I * 2 + 2 * T * k * I * 2 + 2 * T * k * Hh * 4 + T * Hh * 4
    out["moe"] = (moe_fn, moe_flops, moe_bytes, (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY))

    # the gather side of the same MoE layer at tensor parallelism 8: the
    # 4096 tokens gathered from 8 ranks of 512, then gathered per expert and
    # multiplied by this rank's up-projection shards, SiLU, h in pair order
    from synth.gen import split_chunks
    R6 = 8
    loc6, peers6 = split_chunks(inp["x"], R6, 0)
    dl6, dp6 = dv(loc6), dv(peers6)
    full6 = torch.empty((T, Hh), dtype=torch.int16, device="cuda")
    h6 = torch.empty((T * k, I), dtype=torch.int16, device="cuda")
    wsb6 = tsg.workspace_bytes(tsg.OP_MOE_AG, [T, Hh, I, E, k])
    ws6 = torch.empty((wsb6,), dtype=torch.uint8, device="cuda")
    moe_ag_fn = lambda i, mode, opts=None: tsg.moe_ag_group_gemm(ctx, dl6, dp6, full6, ids, wu, h6, cnt, srt, ws6,
                                                                 wsb6, T, Hh, I, E, k, R6, 0, opts=opts, mode=mode)
    moe_ag_flops = 2.0 * T * k * Hh * I
    moe_ag_bytes = 3 * T * Hh * 2 + E * Hh * I * 2 + T * k * I * 2
    out["moe_ag"] = (moe_ag_fn, moe_ag_flops, moe_ag_bytes,
                     (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY))

    # sequence-parallel self-attention with the KV context gathered: 16k
    # tokens, 32 heads of 128, one rank's share of 8 (2048 queries)
    S7, heads7, R7 = 16384, 32, 8
    sl7 = S7 // R7
    rng7 = np.random.default_rng(7)
    mk7 = lambda shape: torch.from_numpy(rng7.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16).cuda()
    q7 = mk7((sl7, heads7, 128))
    kl7, vl7 = mk7((sl7, heads7, 128)), mk7((sl7, heads7, 128))
    kp7, vp7 = mk7((R7 - 1, sl7, heads7, 128)), mk7((R7 - 1, sl7, heads7, 128))
    kf7 = torch.empty((S7, heads7, 128), dtype=torch.bfloat16, device="cuda")
    vf7 = torch.empty_like(kf7)
    o7 = torch.empty_like(q7)
    attn_fn = lambda i, mode, opts=None: tsg.ag_kv_attention(ctx, q7, kl7, kp7, vl7, vp7, kf7, vf7, o7, S7, heads7,
                                                             128, R7, 0, opts=opts, mode=mode)
    attn_flops = 4.0 * sl7 * S7 * 128 * heads7
    attn_bytes = 4 * S7 * heads7 * 128 * 2 + 2 * sl7 * heads7 * 128 * 2
    out["ag_kv_attention"] = (attn_fn, attn_flops, attn_bytes,
                              (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY))

    # the same MoE workload with the y staging in bf16 (stage_dtype): the
    # staging round trip moves half the bytes
    def moe_bf16_fn(i, mode, opts=None):
        o = tsg.Opts(stage_dtype=tsg.BF16) if opts is None else opts
        o.stage_dtype = tsg.BF16
        return moe_fn(i, mode, o)
    moe_bf16_bytes = moe_bytes - T * k * Hh * 4
    out["moe_bf16_staging"] = (moe_bf16_fn, moe_flops, moe_bf16_bytes,
                               (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY))
    return out


def _tiny_line(torch, tsg, ctx, n):
    """The tiny AllGather + GEMM (4 ranks, 256x128x256, fp32 out): a latency
    line in microseconds per call for each mode, with per-call p10 / p50 /
    p90; TFLOP/s is nominal at this size."""
    import numpy as np
    from synth import CONFIGS, ag_inputs
    from synth.gen import split_chunks
    c = CONFIGS["tiny_ag"]
    M, N, K, R = c["M"], c["N"], c["K"], c["R"]
    inp = ag_inputs(M, K, N, R, rank=0, seed=c["seed"], dist="uniform")
    loc, peers = split_chunks(inp["a"], R, 0)
    dl = torch.from_numpy(loc.view(np.int16)).cuda()
    dp = torch.from_numpy(peers.view(np.int16)).cuda()
    db = torch.from_numpy(inp["b"].view(np.int16)).cuda()
    full = torch.empty((M, K), dtype=torch.int16, device="cuda")
    cc = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fn = lambda i, mode, o=None: tsg.gemm_ag_overlap(ctx, dl, dp, full, db, cc, tsg.F32, M, N, K, R, 0, mode=mode)
    line = _path_line(tsg, Timer(torch, tsg, ctx, fn), 2.0 * M * N * K, 2 * (M * K + K * N) + 4 * M * N,
                      (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY), max(n, 50))
    line["us"] = {k: (None if v is None else round(v * 1e3, 2)) for k, v in line.pop("ms").items()}
    line["us_per_call_p10_p50_p90"] = {k: [round(x * 1e3, 2) for x in v]
                                       for k, v in line.pop("ms_per_call_p10_p50_p90").items()}
    line["workload"] = f"AllGather+GEMM, A {M}x{K} bf16 in {R} row chunks, B {K}x{N} bf16, fp32 out"
    return line


# Timeline record kinds (tsg_timeline): producer / consumer units of each path.
TL_KINDS = {"ag_gemm": ((1, "copy units"), (2, "GEMM tiles")),
            "gemm_rs": ((3, "GEMM tiles"), (4, "reduce units")),
            "mlp2": ((5, "GEMM1 tiles"), (6, "GEMM2 tiles")),
            "moe": ((7, "up tiles"), (8, "down tiles"), (9, "combine units")),
            "moe_ag": ((1, "copy units"), (10, "up tiles")),
            "ag_kv_attention": ((1, "copy units"), (11, "attention tiles")),
            "moe_bf16_staging": ((7, "up tiles"), (8, "down tiles"), (9, "combine units"))}


def _timeline_text(name, recs, bins=24):
    """Markdown table of one overlapped call's device timeline: per time bin,
    the units of each kind that are active, and how many of them are waiting
    for a signal (records: {kind<<56 | where<<32 | id, start, start + wait,
    end}, 100 MHz wall clock)."""
    kinds = TL_KINDS[name]
    rows = [(int(r[0]) >> 56, r[1], r[2], r[3]) for r in recs]
    t0 = min(r[1] for r in rows)
    t1 = max(r[3] for r in rows)
    span = max(1, t1 - t0)
    head = f"**{name}**: one call, span {span / 100:.1f} us.  Per bin of {span / bins / 100:.1f} us: " \
           "units active (of which waiting for a signal)."
    lines = [head, "", "| t (us) | " + " | ".join(k[1] for k in kinds) + " |",
             "|---|" + "---|" * len(kinds)]
    for b in range(bins):
        lo, hi = t0 + span * b / bins, t0 + span * (b + 1) / bins
        cells = []
        for kind, _ in kinds:
            act = sum(1 for r in rows if r[0] == kind and r[1] < hi and r[3] >= lo)
            wt = sum(1 for r in rows if r[0] == kind and r[1] < hi and r[2] >= lo and r[2] > r[1])
            cells.append(f"{act} ({wt})" if wt else f"{act}")
        lines.append(f"| {(lo - t0) / 100:.1f} | " + " | ".join(cells) + " |")
    # per kind: when its units ran, how long they waited for signals and how
    # long they ran once their data was there
    import numpy as np
    lines += ["", "| units | count | start (us) | wait median / max (us) | run after the wait, median / p90 (us) "
                  "| end (us) |", "|---|---|---|---|---|---|"]
    for kind, label in kinds:
        rr = [r for r in rows if r[0] == kind]
        if not rr:
            continue
        st = np.array([(r[1] - t0) / 100 for r in rr])
        wt = np.array([(r[2] - r[1]) / 100 for r in rr])
        ru = np.array([(r[3] - r[2]) / 100 for r in rr])
        en = np.array([(r[3] - t0) / 100 for r in rr])
        lines.append(f"| {label} | {len(rr)} | {st.min():.1f}-{st.max():.1f} | {np.median(wt):.1f} / {wt.max():.1f} "
                     f"| {np.median(ru):.1f} / {np.percentile(ru, 90):.1f} | {en.min():.1f}-{en.max():.1f} |")
    if name == "ag_gemm":
        # copy units carry (chunk << 24 | slab << 12 | piece): when each of the
        # first column slabs was complete in every chunk
        done = {}
        for r0 in recs:
            if int(r0[0]) >> 56 == 1:
                sl = (int(r0[0]) >> 12) & 0xfff
                done[sl] = max(done.get(sl, 0), (r0[3] - t0) / 100)
        if done:
            lines += ["", "Column slab complete in every chunk (us): " +
                      ", ".join(f"slab {k}: {v:.1f}" for k, v in sorted(done.items())[:8]) + "."]
    return "\n".join(lines)


def _library_gemms(torch, tsg, ctx, ag_fn):
    """hipBLASLt (torch.matmul, bf16 operands) on the same GEMM shapes as the
    AG, RS and MLP paths, beside this library's compute-only calls of those
    paths (the same GEMMs; the MLP call also applies GELU between them).
    Each figure is the best of 3 rounds of 100 back-to-back calls."""
    from synth import CONFIGS
    other = _other_paths(torch, tsg, ctx)

    def best(fn, n=100):
        ts = []
        for _ in range(3):
            for i in range(20):
                fn(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
            ts.append((time.perf_counter() - t0) / n * 1e3)
        return min(ts)

    def lib(M, N, K, out32):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
        if out32:
            return best(lambda i: torch.mm(a, b, out_dtype=torch.float32))
        return best(lambda i: torch.matmul(a, b))

    ag, rs, mlp = CONFIGS["llama_ag"], CONFIGS["gemm_rs"], CONFIGS["mlp2"]
    rows = []
    t_ag = best(lambda i: ag_fn(i, tsg.COMPUTE_ONLY))
    l_ag = lib(ag["M"], ag["N"], ag["K"], False)
    rows.append(("AG GEMM %dx%dx%d, bf16 out" % (ag["M"], ag["N"], ag["K"]), 2.0 * ag["M"] * ag["N"] * ag["K"],
                 l_ag, t_ag))
    t_rs = best(lambda i: other["gemm_rs"][0](i, tsg.COMPUTE_ONLY))
    l_rs = lib(rs["M"], rs["N"], rs["K"], True)
    rows.append(("RS GEMM %dx%dx%d, fp32 out" % (rs["M"], rs["N"], rs["K"]), 2.0 * rs["M"] * rs["N"] * rs["K"],
                 l_rs, t_rs))
    M, K1, N1, N2 = mlp["M"], mlp["K1"], mlp["N1"], mlp["N2"]
    t_mlp = best(lambda i: other["mlp2"][0](i, tsg.COMPUTE_ONLY))
    l_mlp = lib(M, N1, K1, False) + lib(M, N2, N1, True)
    rows.append(("MLP %dx%d -> %d -> %d (two GEMMs; bf16 H, fp32 Y)" % (M, K1, N1, N2),
                 2.0 * M * N1 * K1 + 2.0 * M * N2 * N1, l_mlp, t_mlp))
    # attention: 2048 queries (one rank's share) over 16384 keys, 32 heads of
    # 128, bf16; torch's fused backends only (its math path is never used)
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    S, Hh, D, sl = 16384, 32, 128, 2048
    q = torch.randn(1, Hh, sl, D, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, Hh, S, D, device="cuda", dtype=torch.bfloat16)
    v = torch.randn(1, Hh, S, D, device="cuda", dtype=torch.bfloat16)
    t_at = best(lambda i: other["ag_kv_attention"][0](i, tsg.COMPUTE_ONLY), 30)
    l_at = None
    for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([be]):
                t = best(lambda i: F.scaled_dot_product_attention(q, k, v), 30)
            l_at = t if l_at is None else min(l_at, t)
        except RuntimeError:
            pass
    out = ["| operation | library ms | TFLOP/s | this library, compute only, ms | TFLOP/s |", "|---|---|---|---|---|"]
    for name, fl, lt, tt in rows:
        out.append(f"| {name}: hipBLASLt | {lt:.4f} | {fl / lt / 1e9:.0f} | {tt:.4f} | {fl / tt / 1e9:.0f} |")
    fl_at = 4.0 * sl * S * D * Hh
    if l_at is not None:
        out.append(f"| attention {sl} queries x {S} keys x {Hh} heads of {D}: torch SDPA (flash / memory-efficient) "
                   f"| {l_at:.4f} | {fl_at / l_at / 1e9:.0f} | {t_at:.4f} | {fl_at / t_at / 1e9:.0f} |")
    return "\n".join(out)


def main():
    args = _parse()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters)))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(peers are stood in for by buffers in local HBM).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tile_level_communication_signaled_amd as tsg
    from synth import CONFIGS, mlp2_inputs, moe_inputs, rs_inputs

    ctx = tsg.Context(0)
    # All work on one dedicated stream (events, library calls, copies): the
    # library's kernels are then ordered after it without the legacy default
    # stream's implicit synchronisation.
    torch.cuda.set_stream(torch.cuda.Stream())
    hopts = tsg.Opts(aux_cus=args.aux_cus, tile=args.tile)
    cfg = CONFIGS["llama_ag"]
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    ag_fn, ag_flops, ag_gemm_bytes, ag_copy_bytes, ag_host = _path_ag(torch, tsg, ctx, cfg, args.steps, hopts)

    if args.timeline:
        # One overlapped call per path with device timestamps (after warm-up);
        # AG also serialized, for comparison.
        out = ["Device timelines (`python3 bench.py --timeline`), one call each.", ""]
        runs = [("ag_gemm", ag_fn, tsg.OVERLAP), ("ag_gemm", ag_fn, tsg.SERIAL), ("ag_gemm", ag_fn, tsg.COMPUTE_ONLY)]
        if args.paths == "all":
            for name, (fn, *_rest) in _other_paths(torch, tsg, ctx).items():
                runs.append((name, fn, tsg.OVERLAP))
        for name, fn, mode in runs:
            for i in range(200):
                fn(i, mode)
            torch.cuda.synchronize()
            # the recorded call follows another call on the stream without a
            # host synchronisation, as in the timed loops
            fn(1, mode)
            fn(0, mode, tsg.Opts(aux_cus=args.aux_cus, tile=args.tile, timeline=1))
            torch.cuda.synchronize()
            if ctx.check() != tsg.OK:
                raise RuntimeError(ctx.last_error())
            label = {tsg.OVERLAP: "overlap", tsg.SERIAL: "serial", tsg.COMPUTE_ONLY: "compute only"}[mode]
            out += [f"### {name}, {label}", "", _timeline_text(name, ctx.timeline()), ""]
        print("\n".join(out), flush=True)
        ctx.close()
        return

    if args.library_gemms:
        print(_library_gemms(torch, tsg, ctx, ag_fn), flush=True)
        ctx.close()
        return

    if args.trace_path:
        if args.trace_path == "ag_copy_engine":
            dma = tsg.Opts(aux_cus=args.aux_cus, tile=args.tile, copy_engine=1)
            fn, flops = (lambda i, mode, o=None: ag_fn(i, mode, dma)), ag_flops
        else:
            fn, flops, _nbytes, _modes = _other_paths(torch, tsg, ctx)[args.trace_path]
        for i in range(args.warmup):
            fn(i, tsg.OVERLAP)
        if ctx.check() != tsg.OK:
            raise RuntimeError(ctx.last_error())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i, tsg.OVERLAP)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        if ctx.check() != tsg.OK:
            raise RuntimeError(ctx.last_error())
        print(json.dumps({"path": args.trace_path, "mode": "overlap", "ms_per_step": round(ms, 5),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "steps": args.steps}), flush=True)
        ctx.close()
        return

    if args.counters:
        for i in range(args.steps):
            ag_fn(i, tsg.COMPUTE_ONLY)
        for i in range(args.steps):
            ag_fn(i, tsg.COMM_ONLY)
        if args.paths == "all":
            for name, (fn, _f, _b, modes) in _other_paths(torch, tsg, ctx).items():
                if name == "moe_bf16_staging":   # same kernel names: keep the record to one variant
                    continue
                for mode in (tsg.COMPUTE_ONLY, tsg.COMM_ONLY):
                    # the gather-side and attention kernels run their copy
                    # alone under their own names: compute-only launches only
                    if mode == tsg.COMM_ONLY and name in ("moe_ag", "ag_kv_attention"):
                        continue
                    if mode in modes:
                        for i in range(args.steps):
                            fn(i, mode)
        torch.cuda.synchronize()
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        if ctx.check() != tsg.OK:
            raise RuntimeError(ctx.last_error())
        ctx.close()
        return

    # ---- headline: K overlap steps between two synchronisations, nothing else
    for i in range(args.warmup):
        ag_fn(i, tsg.OVERLAP)
    if ctx.check() != tsg.OK:
        raise RuntimeError(ctx.last_error())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ag_fn(i, tsg.OVERLAP)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    if ctx.check() != tsg.OK:
        raise RuntimeError(ctx.last_error())

    if args.headline_only:
        print(json.dumps({"metric": METRIC, "value": round(ag_flops / (ms_step * 1e-3) / 1e12, 2),
                          "unit": "TFLOP/s", "ms_per_step": round(ms_step, 5), "steps": args.steps}), flush=True)
        ctx.close()
        return

    timer = Timer(torch, tsg, ctx, ag_fn)
    n = max(5, min(args.steps, 30))
    ALL = (tsg.OVERLAP, tsg.SERIAL, tsg.COMPUTE_ONLY, tsg.COMM_ONLY)
    ag = _path_line(tsg, timer, ag_flops, ag_gemm_bytes + ag_copy_bytes, ALL, n)
    k_spread = {}
    k_ov = timer.kernels(tsg.OVERLAP, max(n, 50), (0, 1), k_spread)
    k_co = timer.kernels(tsg.COMPUTE_ONLY, n, (0,))
    k_cm = timer.kernels(tsg.COMM_ONLY, n, (1,))
    ag["kernel_ms_p10_p90"] = {"gemm_in_overlap": [round(x, 5) for x in k_spread[0]],
                               "copy_in_overlap": [round(x, 5) for x in k_spread[1]]}
    ag["kernel_ms"] = {"gemm_in_overlap": round(k_ov[0], 5), "copy_in_overlap": round(k_ov[1], 5),
                       "gemm_alone": round(k_co[0], 5), "copy_alone": round(k_cm[1], 5)}
    paths = {"ag_gemm": ag}
    if args.paths == "all":
        # the tiny AllGather + GEMM: a latency line, in microseconds
        paths["tiny_ag"] = _tiny_line(torch, tsg, ctx, n)
        # the same AllGather + GEMM with the arrival paced at seven peers'
        # xGMI links (about 153 GB/s each), as a multi-GPU rank would see it
        paced = tsg.Opts(aux_cus=args.aux_cus, tile=args.tile, arrival_gbps=XGMI_GBPS)
        paths["ag_gemm_xgmi_paced"] = _path_line(
            tsg, Timer(torch, tsg, ctx, lambda i, mode, o=None: ag_fn(i, mode, paced)), ag_flops,
            ag_gemm_bytes + ag_copy_bytes, ALL, n)
        paths["ag_gemm_xgmi_paced"]["arrival_gbps"] = XGMI_GBPS
        # the same AllGather + GEMM with the chunks moved by the DMA copy
        # engines (one stream per peer chunk)
        dma = tsg.Opts(aux_cus=args.aux_cus, tile=args.tile, copy_engine=1)
        paths["ag_gemm_copy_engine"] = _path_line(
            tsg, Timer(torch, tsg, ctx, lambda i, mode, o=None: ag_fn(i, mode, dma)), ag_flops,
            ag_gemm_bytes + ag_copy_bytes, ALL, n)

    if args.paths == "all":
        other = _other_paths(torch, tsg, ctx)
        for name, (fn, flops, nbytes, modes) in other.items():
            paths[name] = _path_line(tsg, Timer(torch, tsg, ctx, fn), flops, nbytes, modes, n)
        # The CU splits the configurations name, beside the shared-CU
        # defaults: the two-GEMM MLP with GEMM1 / GEMM2 on 128/128 ... 224/32
        # CUs, and the MoE combine as a persistent consumer on 16 CUs.
        fn, flops, nbytes, _m = other["mlp2"]
        sweep = {}
        for q in (128, 96, 64, 32):
            o = tsg.Opts(aux_cus=q)
            sweep[f"{256 - q}/{q}"] = _path_line(
                tsg, Timer(torch, tsg, ctx, lambda i, mode, o_=None, o=o: fn(i, mode, o)), flops, nbytes,
                (tsg.OVERLAP,), n)
        og = tsg.Opts(order=1)
        sweep["shared, grouped order"] = _path_line(
            tsg, Timer(torch, tsg, ctx, lambda i, mode, o_=None: fn(i, mode, og)), flops, nbytes, (tsg.OVERLAP,), n)
        paths["mlp2_cu_splits"] = sweep
        # the GEMM+RS eight-wave tile (16x16x32 fragments): faster alone, but
        # its workgroups fill their CUs, so overlap runs back to back
        fn, flops, nbytes, _m = other["gemm_rs"]
        o6 = tsg.Opts(tile=6)
        paths["gemm_rs_tile6"] = _path_line(
            tsg, Timer(torch, tsg, ctx, lambda i, mode, o_=None: fn(i, mode, o6)), flops, nbytes,
            (tsg.OVERLAP, tsg.COMPUTE_ONLY), n)
        fn, flops, nbytes, _m = other["moe"]
        o16 = tsg.Opts(aux_cus=16)
        paths["moe_combine_16cu"] = _path_line(
            tsg, Timer(torch, tsg, ctx, lambda i, mode, o_=None: fn(i, mode, o16)), flops, nbytes, (tsg.OVERLAP,), n)
        paths["moe_remote_first"] = _moe_remote_first(torch, tsg, ctx, fn, flops, nbytes, n)

    tflops = ag_flops / (ms_step * 1e-3) / 1e12
    achieved = ag_flops / (k_ov[0] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/64 bf16 operands; two resident input sets used alternately)",
        "config": {"workload": f"AllGather+GEMM, A {M}x{K} bf16 in {R} row chunks of {M // R} "
                               f"(rank 0 local, {R - 1} copied in by the concurrent copy kernel), "
                               f"B {K}x{N} bf16, fp32 accumulate, bf16 out",
                   "M": M, "N": N, "K": K, "R": R, "aux_cus": args.aux_cus, "tile": args.tile},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "speedup_vs_serial": ag["speedup_vs_serial"],
        "overlap_vs_compute_only": ag["overlap_vs_compute_only"],
        "overlap_ratio": ag.get("overlap_ratio"),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic("ag_gemm_kernel"), "kernel": "ag_gemm_kernel (in overlap mode)",
                     "algorithmic_bytes": ag_gemm_bytes, "source_hash": source_hash()},
        "paths": paths,
    }
    if not args.no_cpu:
        cb = _cpu_baselines(ag_host)
        head = dict(cb["llama_ag"])
        head.pop("ms", None)
        out["cpu_baseline"] = head
        out["cpu_baselines"] = cb
    print(json.dumps(out), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
