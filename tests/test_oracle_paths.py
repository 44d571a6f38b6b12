"""Pins for the oracle's path functions: brute force on tiny inputs, exact
integer cases, closed forms and invariants."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import bf16_to_f64
from synth import ag_inputs, f32_to_bf16_bits, moe_inputs, mlp2_inputs, rs_inputs
from synth.gen import split_chunks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _fsum_dot(a_row, b_col):
    # products of two bf16 values are exact in float64; fsum rounds the sum once
    return math.fsum(float(p) * float(q) for p, q in zip(a_row, b_col))


# --------------------------------------------------------------------------
def test_static_mapping_hand_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "static_mapping.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) >= 9
    for r in rows:
        M, R, C, Tm, tid, lo, hi, rank, ch = map(int, r)
        assert oracle.static_map_ag(tid, Tm, M, R, C) == (lo, hi, rank, ch)


@pytest.mark.parametrize("M,R,C,Tm", [(8192, 8, 1, 128), (8192, 8, 4, 64), (256, 4, 1, 64), (768, 3, 2, 32)])
def test_static_mapping_against_row_owner(M, R, C, Tm):
    per_rank, per_chan = M // R, M // (R * C)
    for tid in range(M // Tm):
        lo, hi, rank, ch = oracle.static_map_ag(tid, Tm, M, R, C)
        owners = {m // per_rank for m in range(lo, hi)}
        chans = {m // per_chan for m in range(lo, hi)}
        assert owners == {rank} and chans == {ch}


# --------------------------------------------------------------------------
@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_ag_gather_restores_every_rank_view(R):
    inp = ag_inputs(M=16 * R, K=24, N=8, R=R, seed=3)
    for rank in range(R):
        loc, peers = split_chunks(inp["a"], R, rank)
        got = oracle.ag_gather(loc, peers, R, rank)
        assert got.dtype == np.uint16 and np.array_equal(got, inp["a"])


def test_ag_gather_slot_order_brute_force():
    # distinct constant rows per chunk make any slot mix-up visible
    R, mr, K = 5, 3, 4
    for rank in range(R):
        loc = np.full((mr, K), 100 + rank, dtype=np.uint16)
        peers = np.stack([np.full((mr, K), 100 + r, dtype=np.uint16) for r in range(R) if r != rank])
        out = oracle.ag_gather(loc, peers, R, rank)
        for r in range(R):
            assert np.all(out[r * mr:(r + 1) * mr] == 100 + r)


# --------------------------------------------------------------------------
def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(1)
    a = _bits(rng.uniform(-1, 1, (7, 13)))
    b = _bits(rng.uniform(-1, 1, (13, 5)))
    c = oracle.gemm(a, b)
    s = oracle.gemm_abs(a, b)
    av, bv = bf16_to_f64(a), bf16_to_f64(b)
    assert c.shape == (7, 5)
    for i in range(7):
        for j in range(5):
            ref = _fsum_dot(av[i], bv[:, j])
            assert abs(c[i, j] - ref) <= 1e-14 * s[i, j]
            assert abs(s[i, j] - math.fsum(abs(float(p) * float(q)) for p, q in zip(av[i], bv[:, j]))) <= 1e-14 * s[i, j]


def test_gemm_integer_exact_and_identity():
    rng = np.random.default_rng(2)
    a = _bits(rng.integers(-2, 3, (33, 64)))
    b = _bits(rng.integers(-2, 3, (64, 17)))
    c = oracle.gemm(a, b)
    want = bf16_to_f64(a).astype(np.int64) @ bf16_to_f64(b).astype(np.int64)
    assert np.array_equal(c, want.astype(np.float64))
    eye = _bits(np.eye(64))
    assert np.array_equal(oracle.gemm(a, eye), bf16_to_f64(a))


def test_ag_gemm_invariant_to_rank():
    inp = ag_inputs(M=64, K=32, N=16, R=4, seed=5, dist="uniform")
    ref = oracle.gemm(inp["a"], inp["b"])
    for rank in range(4):
        loc, peers = split_chunks(inp["a"], 4, rank)
        a_full, c = oracle.ag_gemm(loc, peers, inp["b"], 4, rank)
        assert np.array_equal(a_full, inp["a"]) and np.array_equal(c, ref)


# --------------------------------------------------------------------------
def test_rs_reduce_brute_force_and_special_cases():
    R, mr, N = 4, 3, 5
    rng = np.random.default_rng(4)
    for rank in range(R):
        p = rng.standard_normal((mr, N))
        peers = rng.standard_normal((R - 1, mr, N))
        out = oracle.rs_reduce(p, peers, R, rank)
        contrib = [p if r == rank else peers[r if r < rank else r - 1] for r in range(R)]
        for i in range(mr):
            for j in range(N):
                acc = 0.0
                for r in range(R):
                    acc = acc + contrib[r][i, j]
                assert out[i, j] == acc
        assert np.array_equal(oracle.rs_reduce(p, np.zeros_like(peers), R, rank), p)


def test_gemm_rs_chunks_and_zero_input():
    R = 4
    inp = rs_inputs(M=32, K=16, N=8, R=R, rank=1, seed=9)
    P, out = oracle.gemm_rs(inp["x"], inp["w"], inp["peer_partials"], R, 1)
    assert np.allclose(P, oracle.gemm(inp["x"], inp["w"]), rtol=0, atol=0)
    # X = 0: out is the sum of the peers (in ascending order)
    z = np.zeros_like(inp["x"])
    _, out0 = oracle.gemm_rs(z, inp["w"], inp["peer_partials"], R, 1)
    pp = inp["peer_partials"].astype(np.float64)
    assert np.array_equal(out0, ((0.0 + pp[0]) + 0.0) + pp[1] + pp[2])
    # rank r's output uses P's row chunk r
    for rank in range(R):
        _, o = oracle.gemm_rs(inp["x"], inp["w"], np.zeros((R - 1, 8, 8), np.float32), R, rank)
        assert np.array_equal(o, P[rank * 8:(rank + 1) * 8])


# --------------------------------------------------------------------------
def test_mlp2_identity_reduces_to_activation():
    rng = np.random.default_rng(11)
    x = _bits(rng.standard_normal((9, 32)))
    eye = _bits(np.eye(32))
    z, h, y = oracle.mlp2(x, eye, eye)
    xv = bf16_to_f64(x)
    assert np.array_equal(z, xv)
    # H is GELU(x) rounded once to bf16; with W2 = I, Y = H exactly
    for v, hb in zip(xv.ravel(), h.ravel()):
        g = 0.5 * v * (1 + math.erf(v / math.sqrt(2)))
        # half a bf16 quantum at g: 2^(floor(log2|g|) - 8)
        half_q = 2.0 ** (math.floor(math.log2(abs(g))) - 8) if g != 0 else 0.0
        assert abs(bf16_to_f64(np.array([hb]))[0] - g) <= half_q
    assert np.array_equal(y, bf16_to_f64(h))


def test_mlp2_brute_force_tiny():
    inp = mlp2_inputs(M=3, K1=16, N1=8, N2=5, seed=12)
    z, h, y = oracle.mlp2(inp["x"], inp["w1"], inp["w2"])
    xv, w1, w2 = bf16_to_f64(inp["x"]), bf16_to_f64(inp["w1"]), bf16_to_f64(inp["w2"])
    for i in range(3):
        hrow = []
        for j in range(8):
            zz = _fsum_dot(xv[i], w1[:, j])
            assert abs(z[i, j] - zz) < 1e-13
            hrow.append(bf16_to_f64(h[i:i + 1, j])[0])
            assert abs(hrow[-1] - 0.5 * zz * (1 + math.erf(zz / math.sqrt(2)))) <= 2 ** -8 * abs(hrow[-1]) + 1e-30
        for j in range(5):
            assert abs(y[i, j] - _fsum_dot(hrow, w2[:, j])) < 1e-13


# --------------------------------------------------------------------------
def _route_brute(ids, E):
    T, k = ids.shape
    counts = [0] * E
    order = []
    for e in range(E):
        for t in range(T):
            for s in range(k):
                if ids[t, s] == e:
                    counts[e] += 1
                    order.append(t * k + s)
    return counts, order


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (37, 8, 2), (200, 8, 2), (64, 3, 1), (50, 32, 5)])
def test_moe_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 31 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_ids = oracle.moe_route(ids, E)
    bc, bo = _route_brute(ids, E)
    assert list(counts) == bc and list(sorted_ids) == bo
    assert offsets[0] == 0 and offsets[-1] == T * k and sum(counts) == T * k
    assert sorted(sorted_ids) == list(range(T * k))


def test_moe_route_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.moe_route(np.array([[0, 8]]), 8)
    with pytest.raises(ValueError):
        oracle.moe_route(np.array([[-1, 2]]), 8)


def test_moe_tile_table_brute_force():
    counts = [0, 1, 128, 129, 300]
    poff, tiles = oracle.moe_tile_table(counts, 128)
    assert list(poff) == [0, 0, 128, 256, 512, 896]
    want = [(1, 0, 1), (2, 128, 128), (3, 256, 128), (3, 384, 1), (4, 512, 128), (4, 640, 128), (4, 768, 44)]
    assert tiles == want


def test_moe_combine_brute_force_tiny():
    inp = moe_inputs(T=5, H=8, I=16, E=3, k=2, seed=21)
    res = oracle.moe_expert_combine(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_up"], inp["w_down"])
    x = bf16_to_f64(inp["x"])
    for t in range(5):
        acc = [0.0] * 8
        for s in range(2):
            e = int(inp["topk_ids"][t, s])
            wu, wd = bf16_to_f64(inp["w_up"][e]), bf16_to_f64(inp["w_down"][e])
            h = []
            for j in range(16):
                u = _fsum_dot(x[t], wu[:, j])
                hv = u / (1 + math.exp(-u))
                hb = bf16_to_f64(res["h"][t * 2 + s:t * 2 + s + 1, j])[0]
                assert abs(hb - hv) <= 2 ** -8 * abs(hb) + 1e-30
                h.append(hb)
            for j in range(8):
                yv = _fsum_dot(h, wd[:, j])
                assert abs(res["y"][t * 2 + s, j] - yv) < 1e-13
                acc[j] += float(inp["topk_w"][t, s]) * yv
        assert np.allclose(res["out"][t], acc, rtol=1e-13, atol=1e-14)


def test_moe_combine_special_cases():
    T, H, I, E = 16, 32, 24, 4
    inp = moe_inputs(T=T, H=H, I=I, E=E, k=2, seed=22)
    # gates (1, 0): out is the first slot's expert output exactly
    g = np.zeros_like(inp["topk_w"])
    g[:, 0] = 1.0
    res = oracle.moe_expert_combine(inp["x"], inp["topk_ids"], g, inp["w_up"], inp["w_down"])
    assert np.array_equal(res["out"], res["y"][0::2])
    # identical experts, gates summing to one: out equals either slot's output
    wu = np.repeat(inp["w_up"][:1], E, axis=0)
    wd = np.repeat(inp["w_down"][:1], E, axis=0)
    res2 = oracle.moe_expert_combine(inp["x"], inp["topk_ids"], inp["topk_w"], wu, wd)
    assert np.allclose(res2["out"], res2["y"][0::2], rtol=1e-6, atol=1e-9)
    assert np.array_equal(res2["y"][0::2], res2["y"][1::2])
    # E = 1, k = 1: the dense up / SiLU / down MLP
    ids1 = np.zeros((T, 1), np.int32)
    g1 = np.ones((T, 1), np.float32)
    res3 = oracle.moe_expert_combine(inp["x"], ids1, g1, inp["w_up"][:1], inp["w_down"][:1])
    u = bf16_to_f64(inp["x"]) @ bf16_to_f64(inp["w_up"][0])
    h = oracle.f64_to_bf16_bits(u / (1 + np.exp(-u)))
    assert np.allclose(res3["out"], bf16_to_f64(h) @ bf16_to_f64(inp["w_down"][0]), rtol=1e-13, atol=1e-13)


def test_overlap_ratio_closed_form():
    assert oracle.overlap_ratio(10.0, 4.0, 12.0) == 0.5
    assert oracle.overlap_ratio(10.0, 4.0, 14.0) == 0.0
    assert oracle.overlap_ratio(10.0, 4.0, 10.0) == 1.0


def test_moe_ag_up_brute_force_tiny():
    # the gather side written out with Python loops: the gathered token rows
    # are the ranks' chunks in rank order, and each pair's h is the rounded
    # SiLU of its token row times its expert's up projection (math.exp)
    R, rank = 3, 1
    T, H, I, E, k = 6, 8, 5, 3, 2
    inp = moe_inputs(T=T, H=H, I=I, E=E, k=k, seed=61)
    loc, peers = split_chunks(inp["x"], R, rank)
    res = oracle.moe_ag_up(loc, peers, R, rank, inp["topk_ids"], inp["w_up"])
    assert np.array_equal(res["x_full"], inp["x"])
    x = bf16_to_f64(inp["x"])
    w = bf16_to_f64(inp["w_up"])
    for t in range(T):
        for s in range(k):
            e = int(inp["topk_ids"][t, s])
            for j in range(I):
                u = 0.0
                a = 0.0
                for kk in range(H):
                    u += x[t, kk] * w[e, kk, j]
                    a += abs(x[t, kk] * w[e, kk, j])
                want = _bits([u / (1.0 + math.exp(-u))])[0] if abs(u) < 80 else None
                got = int(res["h"][t * k + s, j])
                if want is not None:
                    # one rounding of the float64 value: equal unless the two
                    # sums straddle a bf16 rounding boundary
                    assert abs(bf16_to_f64(np.uint16(got)) - bf16_to_f64(np.uint16(want))) <= \
                        2.0 ** (math.frexp(abs(u / (1.0 + math.exp(-u))) or 1.0)[1] - 8), (t, s, j)
                assert math.isclose(res["scale"][t * k + s, j], a, rel_tol=1e-12, abs_tol=1e-300)


def test_moe_ag_up_matches_expert_path_and_rank_invariance():
    # the same h as the expert-compute path's for the gathered tokens, and
    # the same result whatever rank gathers
    R = 4
    inp = moe_inputs(T=32, H=16, I=24, E=5, k=2, seed=62)
    ref = oracle.moe_expert_combine(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_up"], inp["w_down"])
    for rank in range(R):
        loc, peers = split_chunks(inp["x"], R, rank)
        res = oracle.moe_ag_up(loc, peers, R, rank, inp["topk_ids"], inp["w_up"])
        assert np.array_equal(res["h"], ref["h"])
        assert np.array_equal(res["counts"], ref["counts"]) and np.array_equal(res["sorted_ids"], ref["sorted_ids"])


def test_attention_brute_force_tiny():
    # softmax attention written out with Python loops and math.exp
    rng = np.random.default_rng(63)
    Sq, S, H, D = 3, 5, 2, 4
    q = _bits(rng.standard_normal((Sq, H, D)))
    k = _bits(rng.standard_normal((S, H, D)))
    v = _bits(rng.standard_normal((S, H, D)))
    res = oracle.attention(q, k, v)
    qf, kf, vf = bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v)
    for i in range(Sq):
        for h in range(H):
            s = [sum(qf[i, h, d] * kf[j, h, d] for d in range(D)) / math.sqrt(D) for j in range(S)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for d in range(D):
                want = sum(w[j] / tot * vf[j, h, d] for j in range(S))
                assert math.isclose(res["out"][i, h, d], want, rel_tol=1e-12, abs_tol=1e-14)
                pv = sum(w[j] / tot * abs(vf[j, h, d]) for j in range(S))
                assert math.isclose(res["pv_abs"][i, h, d], pv, rel_tol=1e-12, abs_tol=1e-14)


def test_attention_special_cases_and_gather():
    rng = np.random.default_rng(64)
    S, H, D, R = 8, 2, 4, 4
    q = _bits(rng.standard_normal((2, H, D)))
    k = _bits(rng.standard_normal((S, H, D)))
    v = _bits(rng.standard_normal((S, H, D)))
    # one key: the output is its value row
    one = oracle.attention(q, k[:1], v[:1])
    assert np.allclose(one["out"], np.broadcast_to(bf16_to_f64(v[:1]), one["out"].shape), rtol=0, atol=0)
    # zero queries: uniform weights, the mean of the value rows
    z = oracle.attention(np.zeros_like(q), k, v)
    assert np.allclose(z["out"], bf16_to_f64(v).mean(axis=0)[None], rtol=1e-14, atol=1e-15)
    # the gathered context does not depend on the rank that gathers it
    base = oracle.attention(q, k, v)["out"]
    for rank in range(R):
        kl, kp = split_chunks(k, R, rank)
        vl, vp = split_chunks(v, R, rank)
        res = oracle.ag_kv_attention(q, kl, kp, vl, vp, R, rank)
        assert np.array_equal(res["k_full"], k) and np.array_equal(res["v_full"], v)
        assert np.array_equal(res["out"], base)
