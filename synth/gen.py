"""Seeded input generators.

Every tensor is drawn from its own PCG64 stream, obtained by spawning
``numpy.random.SeedSequence(seed)`` in a fixed order per workload, drawn in
float64, scaled, cast to float32 and, for bf16 operands, rounded to bf16 by
round-to-nearest-even.  bf16 tensors are returned as ``uint16`` bit patterns so
that the oracle and the device path consume the very same bytes.

Workload shapes follow the five configurations this library is measured on:
a tiny AllGather+GEMM, the AllGather+GEMM of one rank's TP=8 share of a
Llama-style MLP up-projection, a GEMM+ReduceScatter producer/consumer, a
two-GEMM MLP pipelined at 128-row-block granularity, and a top-2 MoE expert
compute with gate-weighted combine.
"""
from __future__ import annotations

import numpy as np

# name -> parameters.  The first entry is the small case the oracle checks
# exhaustively; the others are the full-size workloads.
CONFIGS = {
    "tiny_ag": dict(kind="ag", M=256, K=256, N=128, R=4, dist="uniform", seed=0, out="f32"),
    "llama_ag": dict(kind="ag", M=8192, K=4096, N=1792, R=8, dist="normal", seed=1, out="bf16"),
    "gemm_rs": dict(kind="rs", M=8192, K=1792, N=4096, R=8, seed=2),
    "mlp2": dict(kind="mlp2", M=2048, K1=8192, N1=4096, N2=8192, seed=3),
    "moe": dict(kind="moe", T=4096, H=4096, I=1408, E=8, k=2, zipf=1.2, seed=4),
}


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in generated input")
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_bf16(rng, shape, scale: float) -> np.ndarray:
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _uniform_bf16(rng, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.uniform(-1.0, 1.0, shape).astype(np.float32))


def split_chunks(a: np.ndarray, R: int, rank: int):
    """Row-chunk view of a gathered operand: chunk c (rows [c*M/R, (c+1)*M/R))
    belongs to rank c.  Returns (local chunk, peer chunks stacked in ascending
    rank order, skipping ``rank``)."""
    M = a.shape[0]
    if M % R:
        raise ValueError("M must be divisible by R")
    mr = M // R
    local = a[rank * mr:(rank + 1) * mr].copy()
    peers = np.stack([a[c * mr:(c + 1) * mr] for c in range(R) if c != rank]) if R > 1 else \
        np.zeros((0, mr) + a.shape[1:], dtype=a.dtype)
    return local, np.ascontiguousarray(peers)


def ag_inputs(M, K, N, R, rank=0, seed=0, dist="normal", a_scale=None, b_scale=None):
    """AllGather+GEMM operands.  A [M x K] is drawn whole (so the logical A does
    not depend on the local rank) and then split into the local chunk and the
    peers' chunks; B [K x N] is the local weight shard, row-major."""
    ra, rb = _streams(seed, 2)
    if dist == "uniform":
        a = _uniform_bf16(ra, (M, K))
        b = _uniform_bf16(rb, (K, N))
    elif dist == "normal":
        a = _normal_bf16(ra, (M, K), (1.0 / np.sqrt(K)) if a_scale is None else a_scale)
        b = _normal_bf16(rb, (K, N), (1.0 / np.sqrt(K)) if b_scale is None else b_scale)
    else:
        raise ValueError(dist)
    a_local, a_peers = split_chunks(a, R, rank)
    return dict(a=a, a_local=a_local, a_peers=a_peers, b=b)


def rs_inputs(M, K, N, R, rank=0, seed=2):
    """GEMM+ReduceScatter operands: X [M x K] ~ N(0,1), W [K x N] ~ N(0,1)/sqrt(K),
    and the R-1 peers' partial sums for the local chunk, fp32 N(0,1),
    [(R-1) x M/R x N] in ascending peer-rank order skipping ``rank``."""
    if M % R:
        raise ValueError("M must be divisible by R")
    rx, rw, rp = _streams(seed, 3)
    x = _normal_bf16(rx, (M, K), 1.0)
    w = _normal_bf16(rw, (K, N), 1.0 / np.sqrt(K))
    peers = rp.standard_normal((R - 1, M // R, N)).astype(np.float32)
    return dict(x=x, w=w, peer_partials=peers)


def mlp2_inputs(M, K1, N1, N2, seed=3):
    """Two-layer MLP operands: X [M x K1] ~ N(0,1), W1 [K1 x N1] ~ N(0,1)/sqrt(K1),
    W2 [N1 x N2] ~ N(0,1)/sqrt(N1)."""
    rx, r1, r2 = _streams(seed, 3)
    x = _normal_bf16(rx, (M, K1), 1.0)
    w1 = _normal_bf16(r1, (K1, N1), 1.0 / np.sqrt(K1))
    w2 = _normal_bf16(r2, (N1, N2), 1.0 / np.sqrt(N1))
    return dict(x=x, w1=w1, w2=w2)


def zipf_probs(E: int, s: float) -> np.ndarray:
    """Zipf(s) truncated to E experts: P(e) proportional to (e+1)^-s."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def moe_inputs(T, H, I, E, k=2, seed=4, zipf=1.2):
    """MoE operands.  Routing: each token draws k distinct experts one after
    another, without replacement, from Zipf(zipf) over the E experts (slot order
    = draw order), realised with the Gumbel-top-k construction, which has that
    distribution.  Gates are the softmax, over the k chosen experts in slot
    order, of per-(token, expert) logits ~ N(0,1).  X ~ N(0,1),
    W_up[e] [H x I] ~ N(0,1)/sqrt(H), W_down[e] [I x H] ~ N(0,1)/sqrt(I)."""
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    rx, rg, rl, ru, rd = _streams(seed, 5)
    x = _normal_bf16(rx, (T, H), 1.0)
    keys = np.log(zipf_probs(E, zipf))[None, :] + rg.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    logits = rl.standard_normal((T, E))
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    g = np.exp(sel)
    g = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    w_up = _normal_bf16(ru, (E, H, I), 1.0 / np.sqrt(H))
    w_down = _normal_bf16(rd, (E, I, H), 1.0 / np.sqrt(I))
    return dict(x=x, topk_ids=np.ascontiguousarray(ids), topk_w=np.ascontiguousarray(g),
                w_up=w_up, w_down=w_down)
