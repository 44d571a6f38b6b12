"""What each tile-signaled path computes, written out plainly in float64.

Citations use the keys defined in the package docstring ([TL], [TD], [DG]).
bf16 operands arrive as uint16 bit patterns and are decoded exactly.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64, f64_to_bf16_bits, gelu_erf, silu


# ---------------------------------------------------------------------------
# Static tile-centric mapping ([TL] section 4.1, static-mapping equations)
# ---------------------------------------------------------------------------
def static_map_ag(tile_id: int, Tm: int, M: int, R: int, C: int = 1):
    """Shape, rank and channel of AllGather producer tile ``tile_id`` when the
    gathered operand is sharded along M over R ranks with C channels (signals)
    per rank and the producer moves Tm rows per tile:

      M_per_rank = ceil(M / R),  M_per_channel = ceil(M / (R*C)),
      range_M    = [tile_id*Tm, tile_id*Tm + Tm),
      src_rank   = floor(tile_id / floor(M_per_rank / Tm)),
      channel    = floor(tile_id / floor(M_per_channel / Tm)).

    Returns (row_lo, row_hi, src_rank, channel).  The pages' equations assume
    Tm divides the per-channel row count; a ValueError is raised otherwise."""
    m_rank = -(-M // R)
    m_chan = -(-M // (R * C))
    if Tm <= 0 or m_chan % Tm:
        raise ValueError("Tm must divide the rows per channel")
    lo = tile_id * Tm
    return lo, lo + Tm, tile_id // (m_rank // Tm), tile_id // (m_chan // Tm)


# ---------------------------------------------------------------------------
# AllGather + GEMM
# ---------------------------------------------------------------------------
def ag_gather(a_local, a_peers, R: int, rank: int) -> np.ndarray:
    """Pull-mode intra-node AllGather ([TD] section 3.2, Algorithm 2): the
    local shard is copied into slot ``rank`` of the gathered buffer, then for
    every other rank r the shard held by r is copied into slot r.  Shards are
    row chunks of M/R rows; ``a_peers`` lists the R-1 peer shards in ascending
    rank order, skipping ``rank``.  Pure data movement, so bit patterns are
    returned unchanged."""
    a_local = np.asarray(a_local)
    a_peers = np.asarray(a_peers)
    mr = a_local.shape[0]
    if a_peers.shape[0] != R - 1 or (R > 1 and a_peers.shape[1:] != a_local.shape):
        raise ValueError("a_peers must hold R-1 shards shaped like a_local")
    out = np.empty((R * mr,) + a_local.shape[1:], dtype=a_local.dtype)
    out[rank * mr:(rank + 1) * mr] = a_local
    for r in range(R):
        if r != rank:
            out[r * mr:(r + 1) * mr] = a_peers[r if r < rank else r - 1]
    return out


def gemm(a_bits, b_bits) -> np.ndarray:
    """C[i, j] = sum_k A[i, k] * B[k, j] over the exact values of bf16 A [M x K]
    and B [K x N] (both row-major), in float64."""
    return bf16_to_f64(a_bits) @ bf16_to_f64(b_bits)


def gemm_abs(a_bits, b_bits) -> np.ndarray:
    """S[i, j] = sum_k |A[i, k] * B[k, j]|: the scale of the per-element error
    bound |gpu - ref| <= 1e-3 * S + 1e-5 used for every GEMM result."""
    return np.abs(bf16_to_f64(a_bits)) @ np.abs(bf16_to_f64(b_bits))


def ag_gemm(a_local, a_peers, b_bits, R: int, rank: int):
    """AllGather + GEMM of a tensor-parallel FFN's first part ([TL] section
    2.1 and Figure 1): the activation is gathered along M from all ranks, then
    multiplied by the local weight shard.  Returns (A_full bits, C float64)."""
    a_full = ag_gather(a_local, a_peers, R, rank)
    return a_full, gemm(a_full, b_bits)


# ---------------------------------------------------------------------------
# GEMM + ReduceScatter
# ---------------------------------------------------------------------------
def rs_reduce(p_local_chunk, peer_partials, R: int, rank: int) -> np.ndarray:
    """Reduction half of the one-sided ReduceScatter ([TD] section 3.3,
    Algorithm 3, second stream): R accumulates the chunk contributed by every
    rank r = 0 .. R-1 in ascending order.  The initial value of R is not
    printed; it is read as zero.  Rank ``rank`` contributes its own partial
    chunk; every other rank's contribution is taken from ``peer_partials``
    (ascending rank order, skipping ``rank``)."""
    p = np.asarray(p_local_chunk, dtype=np.float64)
    peers = np.asarray(peer_partials, dtype=np.float64)
    if peers.shape[0] != R - 1:
        raise ValueError("need R-1 peer partials")
    acc = np.zeros_like(p)
    for r in range(R):
        acc = acc + (p if r == rank else peers[r if r < rank else r - 1])
    return acc


def gemm_rs(x_bits, w_bits, peer_partials, R: int, rank: int):
    """GEMM + ReduceScatter of a tensor-parallel FFN's second part ([TL]
    section 2.1; [TD] Algorithm 3): the producer GEMM computes the full partial
    P = X W [M x N]; row chunk c (M/R rows) of P is the contribution destined
    for rank c.  The local rank's output is the sum over ranks of their chunk
    ``rank`` contributions.  Returns (P float64, out float64 [M/R x N])."""
    P = gemm(x_bits, w_bits)
    M = P.shape[0]
    if M % R:
        raise ValueError("M must be divisible by R")
    mr = M // R
    return P, rs_reduce(P[rank * mr:(rank + 1) * mr], peer_partials, R, rank)


# ---------------------------------------------------------------------------
# Two-GEMM MLP (CTA-pipelined on the device)
# ---------------------------------------------------------------------------
def mlp2(x_bits, w1_bits, w2_bits):
    """Two-layer GEMM MLP ([DG] CTA-pipelining abstract: a 2-layer GEMM
    representing the MLP; [TL] section 7.2: an activation between the two
    GEMMs).  Z = X W1; H = bf16(GELU(Z)), H being the bf16 operand of the
    second GEMM; Y = H W2.  Returns (Z float64, H bits, Y float64)."""
    z = gemm(x_bits, w1_bits)
    h = f64_to_bf16_bits(gelu_erf(z))
    return z, h, gemm(h, w2_bits)


# ---------------------------------------------------------------------------
# MoE: routing bookkeeping, expert compute, gate-weighted combine
# ---------------------------------------------------------------------------
def moe_route(topk_ids, E: int):
    """Dynamic-mapping tables of the MoE path ([TL] section 4.1, dynamic
    mapping; section 5, AllGather + MoE driven by topk_ids).

    Pair p = t*k + s is token t's s-th routing choice, expert topk_ids[t, s].
    counts[e] = number of pairs routed to e; offsets = exclusive prefix sum of
    counts (length E+1); sorted_ids lists the pair ids ordered by (expert, t,
    s), i.e. a stable sort of the pairs by expert.  Raises on ids outside
    [0, E)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_ids = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, sorted_ids


def moe_tile_table(counts, BM: int):
    """Row tiles of the grouped GEMM: every expert's rows (in sorted order)
    are padded up to a multiple of BM, and each BM-row tile maps to one expert
    (the lookup tables f_S_low / f_S_high / f_R of [TL] section 4.1 with the
    expert in the role of the source).  Returns (padded_offsets [E+1], list of
    (expert, padded_row_lo, n_valid_rows))."""
    counts = np.asarray(counts, dtype=np.int64)
    padded = -(-counts // BM) * BM
    poff = np.zeros(len(counts) + 1, dtype=np.int64)
    poff[1:] = np.cumsum(padded)
    tiles = []
    for e, c in enumerate(counts):
        for lo in range(0, int(padded[e]), BM):
            tiles.append((e, int(poff[e] + lo), int(min(BM, c - lo))))
    return poff, tiles


def moe_expert_combine(x_bits, topk_ids, topk_w, w_up_bits, w_down_bits):
    """Expert compute followed by the gate-weighted combine ([DG] MoE
    tile-signaling abstract: expert outputs return to token order; [TL]
    section 7.2: GroupGEMM + Scatter + Topk-Reduce).

    For every pair (t, s) with e = topk_ids[t, s]:
        u = x_t W_up[e];  h = bf16(SiLU(u));  y = h W_down[e];
    and out[t] = sum_s topk_w[t, s] * y_(t, s).  No residual, no gate
    renormalisation.  Returns dict(out [T x H], h bits [T*k x I] and y
    [T*k x H] in pair order, scale [T x H] = sum_s g_s * sum_k |h_k W_down_kj|
    for the error bound)."""
    x = bf16_to_f64(x_bits)
    ids = np.asarray(topk_ids, dtype=np.int64)
    g = np.asarray(topk_w, dtype=np.float64)
    T, k = ids.shape
    E = w_up_bits.shape[0]
    I = w_up_bits.shape[2]
    H = w_down_bits.shape[2]
    counts, offsets, sorted_ids = moe_route(ids, E)
    h_bits = np.zeros((T * k, I), dtype=np.uint16)
    y = np.zeros((T * k, H), dtype=np.float64)
    s_abs = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        pairs = sorted_ids[offsets[e]:offsets[e + 1]].astype(np.int64)
        if pairs.size == 0:
            continue
        toks = pairs // k
        u = x[toks] @ bf16_to_f64(w_up_bits[e])
        he = f64_to_bf16_bits(silu(u))
        wd = bf16_to_f64(w_down_bits[e])
        hv = bf16_to_f64(he)
        h_bits[pairs] = he
        y[pairs] = hv @ wd
        s_abs[pairs] = np.abs(hv) @ np.abs(wd)
    gp = g.reshape(-1)[:, None]
    out = (gp * y).reshape(T, k, H).sum(axis=1)
    scale = (gp * s_abs).reshape(T, k, H).sum(axis=1)
    return dict(out=out, h=h_bits, y=y, scale=scale, counts=counts, sorted_ids=sorted_ids)


def moe_ag_up(a_local, a_peers, R: int, rank: int, topk_ids, w_up_bits):
    """Gather side of a tensor-parallel MoE layer ([TL] section 5, AllGather
    + MoE; [TL] section 7.2, the MoE layer's first part, AG + Gather +
    GroupGEMM).  The token chunks of all R ranks are gathered along the token
    dimension (ag_gather, [TD] Algorithm 2); then every routed pair p = t*k +
    s with e = topk_ids[t, s] takes

        h[p] = bf16(SiLU(x_t W_up[e])),

    the gathered token's row times this rank's shard of the expert's up
    projection, rounded once to bf16.  Returns dict(x_full bits, h bits
    [T*k x I] in pair order, scale [T*k x I] = sum_k |x_tk W_up[e]_kj| for the
    error bound, counts, sorted_ids)."""
    x_full = ag_gather(a_local, a_peers, R, rank)
    x = bf16_to_f64(x_full)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    E, _, I = w_up_bits.shape
    counts, offsets, sorted_ids = moe_route(ids, E)
    h = np.zeros((T * k, I), dtype=np.uint16)
    scale = np.zeros((T * k, I), dtype=np.float64)
    for e in range(E):
        pairs = sorted_ids[offsets[e]:offsets[e + 1]].astype(np.int64)
        if pairs.size == 0:
            continue
        xe = x[pairs // k]
        we = bf16_to_f64(w_up_bits[e])
        h[pairs] = f64_to_bf16_bits(silu(xe @ we))
        scale[pairs] = np.abs(xe) @ np.abs(we)
    return dict(x_full=x_full, h=h, scale=scale, counts=counts, sorted_ids=sorted_ids)


def attention(q_bits, k_bits, v_bits):
    """Self-attention of queries q [Sq x heads x D] over keys and values
    [S x heads x D] (bf16 bits), per head, with no mask ([TL] section 7.2: two
    batched GEMMs and a softmax): out[i, h] = sum_j P_ij V[j, h] with
    P_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij) and
    s_ij = q[i, h] . K[j, h] / sqrt(D).  Returns dict(out float64
    [Sq x heads x D], pv_abs = sum_j P_ij |V[j, h]| for the error bound,
    qk_abs_max = max_j sum_d |q[i, h, d] K[j, h, d]| per (i, h))."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    Sq, H, D = q.shape
    out = np.empty((Sq, H, D))
    pv_abs = np.empty((Sq, H, D))
    qk_abs_max = np.empty((Sq, H))
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) / np.sqrt(D)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
        pv_abs[:, h, :] = p @ np.abs(v[:, h, :])
        qk_abs_max[:, h] = (np.abs(q[:, h, :]) @ np.abs(k[:, h, :]).T).max(axis=1)
    return dict(out=out, pv_abs=pv_abs, qk_abs_max=qk_abs_max)


def ag_kv_attention(q_bits, k_local, k_peers, v_local, v_peers, R: int, rank: int):
    """Sequence-parallel self-attention of one rank ([TL] section 2.1; [TL]
    section 5, AllGather KV + self-attention): the key and value shards of
    all R ranks are gathered along the sequence (ag_gather, [TD] Algorithm
    2), then this rank's queries attend over the whole gathered context.
    Returns dict(k_full, v_full bits, and attention()'s fields)."""
    k_full = ag_gather(k_local, k_peers, R, rank)
    v_full = ag_gather(v_local, v_peers, R, rank)
    res = attention(q_bits, k_full, v_full)
    res.update(k_full=k_full, v_full=v_full)
    return res


def overlap_ratio(comp_only: float, comm_only: float, overlap: float) -> float:
    """Fraction of communication time hidden by overlap ([TL] section 7.2):
    (comp_only + comm_only - overlap) / comm_only."""
    return (comp_only + comm_only - overlap) / comm_only
