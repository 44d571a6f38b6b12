"""MoE expert compute + overlapped gate-weighted combine on the GPU against
the oracle.

Before every call out is filled with NaN, and the whole workspace (routing
tables, h, y staging) with 0xFF bytes (NaN in bf16 and fp32, -1 in int32): a
down tile that read h before its row block's signal, or a combine that read y
before its tile's ready signal, yields a non-finite element.

Checked after each call:
  * expert_counts and sorted_ids bit for bit;
  * the device's lookup tables, read through tsg_moe_workspace_layout, bit
    for bit: the expert of each row block against oracle.moe_tile_table, the
    expert offsets, and the row of each pair and the pair of each row
    implied by the oracle's stable routing order and padded offsets;
  * the device's h (per pair, through the pair -> row table) against the
    oracle's h: u differs by at most the GEMM bound 1e-3 * sum_k |x w_up| +
    1e-5, SiLU changes that by at most |SiLU'| <= 1.1 times, and the two
    roundings to bf16 add at most one bf16 quantum;
  * out against the oracle's out under the GEMM bound of the down projection,
    1e-3 * sum_s g_s sum_k |h_sk w_down_kj| + 1e-5, plus the device's actual
    h difference carried through |w_down| and the gates,
    sum_s g_s sum_k |h_gpu - h_ref|_sk |w_down_kj| (with bf16 y staging, also
    the gate times one bf16 quantum of y per slot).
The ratio under the plain per-element GEMM bound (no h term) is printed too."""
import numpy as np
import pytest

import oracle
from _helpers import bf16_half_quantum, to_dev
from synth import CONFIGS, f32_to_bf16_bits, moe_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    ctx.close()


class MoeCase:
    def __init__(self, env, inp):
        torch, tsg, ctx = env
        self.env = env
        self.inp = inp
        T, H = inp["x"].shape
        E, _, I = inp["w_up"].shape
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, inp["topk_ids"].shape[1]
        self.x = to_dev(inp["x"], torch)
        self.ids = to_dev(inp["topk_ids"], torch)
        self.g = to_dev(inp["topk_w"], torch)
        self.wu = to_dev(inp["w_up"], torch)
        self.wd = to_dev(inp["w_down"], torch)
        self.out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        self.counts = torch.empty((E,), dtype=torch.int32, device="cuda")
        self.sorted = torch.empty((T * self.k,), dtype=torch.int32, device="cuda")
        dims = [T, H, I, E, self.k]
        self.wsb = tsg.workspace_bytes(tsg.OP_MOE, dims)
        assert self.wsb > 0
        self.lay = tsg.moe_workspace_layout(dims)
        assert self.lay["total"] == self.wsb
        self.ws = torch.empty((self.wsb,), dtype=torch.uint8, device="cuda")

    def run(self, mode=None, opts=None, expect=0, poison=True):
        """One call; outputs poisoned first, and the workspace too except in
        COMM_ONLY mode, whose combine reads the staging a previous call left."""
        torch, tsg, ctx = self.env
        mode = tsg.OVERLAP if mode is None else mode
        if poison:
            self.out.fill_(float("nan"))
            self.counts.fill_(-7)
            self.sorted.fill_(-7)
            if mode != tsg.COMM_ONLY:
                self.ws.fill_(0xFF)
        tsg.moe_expert_combine(ctx, self.x, self.ids, self.g, self.wu, self.wd, self.out, self.counts,
                               self.sorted, self.ws, self.wsb, self.T, self.H, self.I, self.E, self.k,
                               opts=opts, mode=mode)
        st = ctx.check()
        assert st == expect, (st, ctx.last_error())
        return (self.out.cpu().numpy().astype(np.float64), self.counts.cpu().numpy(),
                self.sorted.cpu().numpy())

    def tables(self):
        """The device's routing tables and h from the workspace of the last call."""
        L, E, P = self.lay, self.E, self.T * self.k
        ws = self.ws.cpu().numpy()

        def i32(field, n):
            o = L[field]
            return ws[o:o + 4 * n].view(np.int32).copy()
        rows = L["rows_max"]
        h = ws[L["h"]:L["h"] + rows * self.I * 2].view(np.uint16).reshape(rows, self.I)
        return dict(meta=i32("meta", 2), offs=i32("offs", E + 1), poffs=i32("poffs", E + 1),
                    rb_expert=i32("rb_expert", L["rb_max"]), row_pair=i32("row_pair", rows),
                    row_token=i32("row_token", rows), pair_row=i32("pair_row", P), h=h)


def _check_tables(case, res):
    """Bit-exact lookup tables: the oracle's tile table and the row <-> pair
    maps its stable order implies."""
    tb = case.tables()
    L, k, P = case.lay, case.k, case.T * case.k
    counts, offsets, sorted_ids = oracle.moe_route(case.inp["topk_ids"], case.E)
    poff, tiles = oracle.moe_tile_table(counts, L["bm"])
    n_rb = len(tiles)
    assert tb["meta"][0] == n_rb and tb["meta"][1] == P, tb["meta"]
    assert np.array_equal(tb["offs"], offsets)
    assert np.array_equal(tb["poffs"], poff)
    assert np.array_equal(tb["rb_expert"][:n_rb], np.array([t[0] for t in tiles], dtype=np.int32))
    assert np.all(tb["rb_expert"][n_rb:] == -1)
    pair_row = np.empty(P, dtype=np.int64)
    for e in range(case.E):
        pairs = sorted_ids[offsets[e]:offsets[e + 1]]
        pair_row[pairs] = poff[e] + np.arange(pairs.size)
    assert np.array_equal(tb["pair_row"], pair_row)
    row_pair = np.full(L["rows_max"], -1, dtype=np.int64)
    row_pair[pair_row] = np.arange(P)
    assert np.array_equal(tb["row_pair"], row_pair)
    assert np.array_equal(tb["row_token"], np.where(row_pair >= 0, row_pair // k, -1))
    return tb["h"][pair_row]


def _check(case, out, counts, sorted_ids, y_bf16=False, label=""):
    """Full check of one call; returns (max err/tol of out, of h, of out under
    the plain GEMM bound)."""
    inp = case.inp
    res = oracle.moe_expert_combine(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_up"], inp["w_down"])
    assert np.array_equal(counts, res["counts"])
    assert np.array_equal(sorted_ids, res["sorted_ids"])
    h_dev = _check_tables(case, res)
    x = oracle.bf16_to_f64(inp["x"])
    ids, g = inp["topk_ids"], inp["topk_w"].astype(np.float64)
    T, k = ids.shape
    H = case.H
    hg, hr = oracle.bf16_to_f64(h_dev), oracle.bf16_to_f64(res["h"])
    assert np.all(np.isfinite(hg))
    flat = ids.reshape(-1)
    rh, prop = 0.0, np.zeros((T * k, H))
    for e in range(case.E):
        pairs = np.nonzero(flat == e)[0]
        if pairs.size == 0:
            continue
        s_up = np.abs(x[pairs // k]) @ np.abs(oracle.bf16_to_f64(inp["w_up"][e]))
        tol_h = 1.1 * (1e-3 * s_up + 1e-5) + 2 * bf16_half_quantum(hr[pairs]) + 1e-7
        rh = max(rh, float(np.max(np.abs(hg[pairs] - hr[pairs]) / tol_h)))
        prop[pairs] = np.abs(hg[pairs] - hr[pairs]) @ np.abs(oracle.bf16_to_f64(inp["w_down"][e]))
    if y_bf16:
        prop = prop + 2 * bf16_half_quantum(res["y"])
    extra = (g.reshape(-1)[:, None] * prop).reshape(T, k, H).sum(axis=1)
    plain = 1e-3 * res["scale"] + 1e-5
    assert np.all(np.isfinite(out))
    err = np.abs(out - res["out"])
    r = float(np.max(err / (plain + extra)))
    r_plain = float(np.max(err / plain))
    if label:
        print(f"moe {label}: max err/tol {r:.4f} (h {rh:.4f}; plain GEMM bound {r_plain:.4f}), "
              f"expert counts {counts.tolist()}")
    assert rh <= 1.0, rh
    return r, rh, r_plain


# (9000, ...) and (32767, ...): routed pair blocks of 128 and 256 pairs, the
# second at the largest T * k the routing takes (65534 pairs); 16 to 40
# experts: more groups of pairs per wave in the counting and placement.
@pytest.mark.parametrize("T,H,I,E", [(100, 256, 128, 4), (37, 136, 200, 3), (1, 64, 64, 2), (300, 512, 256, 8),
                                     (9000, 64, 72, 5), (32767, 64, 64, 8), (300, 256, 128, 24),
                                     (2000, 64, 64, 40), (700, 64, 64, 16)])
def test_moe_small(env, T, H, I, E):
    inp = moe_inputs(T, H, I, E, k=2, seed=T + E)
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    r, _, _ = _check(case, out, counts, sorted_ids)
    assert r <= 1.0, r


def test_moe_back_to_back_calls_alternating_routings(env):
    # Calls back to back without a synchronisation, alternating two routings
    # (the larger with 256 blocks of pairs) on one context: each must leave
    # its own tables, h and out, whatever the previous call left in the
    # context's signals and queue.
    torch, tsg, ctx = env
    cases = [MoeCase(env, moe_inputs(T, 64, 64, E, k=2, seed=50 + T)) for T, E in ((32767, 8), (700, 16))]
    for c in cases:
        c.out.fill_(float("nan"))
        c.ws.fill_(0xFF)
    for i in range(8):
        c = cases[i % 2]
        tsg.moe_expert_combine(ctx, c.x, c.ids, c.g, c.wu, c.wd, c.out, c.counts, c.sorted, c.ws, c.wsb,
                               c.T, c.H, c.I, c.E, c.k, mode=tsg.OVERLAP)
    assert ctx.check() == tsg.OK, ctx.last_error()
    for c in cases:
        out = c.out.cpu().numpy().astype(np.float64)
        r, _, _ = _check(c, out, c.counts.cpu().numpy(), c.sorted.cpu().numpy())
        assert r <= 1.0, r


def test_moe_skewed_routing_single_expert_heavy(env):
    T, H, I, E = 512, 256, 128, 8
    inp = moe_inputs(T, H, I, E, k=2, seed=31)
    ids = inp["topk_ids"].copy()
    ids[:, 0] = 0                          # every token's first choice is expert 0
    ids[:, 1] = np.where(ids[:, 1] == 0, 1, ids[:, 1])
    inp["topk_ids"] = ids
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    r, _, _ = _check(case, out, counts, sorted_ids)
    assert r <= 1.0
    assert counts[0] == T


def test_moe_zero_gate_slot_is_ignored_bit_exactly(env):
    T, H, I, E = 200, 256, 128, 6
    inp = moe_inputs(T, H, I, E, k=2, seed=32)
    g = np.zeros_like(inp["topk_w"])
    g[:, 0] = 1.0
    inp["topk_w"] = g
    case1 = MoeCase(env, inp)
    out1, c1, s1 = case1.run()
    r, _, _ = _check(case1, out1, c1, s1)
    assert r <= 1.0
    # move every second slot to another expert: with gate 0 the output cannot change
    ids = inp["topk_ids"].copy()
    ids[:, 1] = (ids[:, 0] + 1 + (ids[:, 1] + 1) % (E - 1)) % E
    assert np.all(ids[:, 1] != ids[:, 0])
    inp2 = dict(inp, topk_ids=ids)
    out2, _, _ = MoeCase(env, inp2).run()
    assert np.array_equal(out1, out2)


def test_moe_identical_experts(env):
    T, H, I, E = 128, 256, 128, 4
    inp = moe_inputs(T, H, I, E, k=2, seed=33)
    inp["w_up"] = np.repeat(inp["w_up"][:1], E, axis=0)
    inp["w_down"] = np.repeat(inp["w_down"][:1], E, axis=0)
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    r, _, _ = _check(case, out, counts, sorted_ids)
    assert r <= 1.0


def test_moe_bad_expert_id_reported(env):
    torch, tsg, ctx = env
    inp = moe_inputs(64, 128, 64, 4, k=2, seed=34)
    ids = inp["topk_ids"].copy()
    ids[5, 1] = 9
    inp["topk_ids"] = ids
    MoeCase(env, inp).run(expect=tsg.E_INVALID)


def test_moe_rejects_small_workspace_and_k(env):
    torch, tsg, ctx = env
    inp = moe_inputs(64, 128, 64, 4, k=2, seed=35)
    c = MoeCase(env, inp)
    args = (ctx, c.x, c.ids, c.g, c.wu, c.wd, c.out, c.counts, c.sorted, c.ws)
    assert tsg.moe_expert_combine(*args, c.wsb - 1, 64, 128, 64, 4, 2, raise_on_error=False) == tsg.E_WORKSPACE
    assert tsg.moe_expert_combine(*args, c.wsb, 64, 128, 64, 4, 3, raise_on_error=False) == tsg.E_UNSUPPORTED
    # more routed pairs than the routing's 16-bit counts hold: rejected on the host, before any device work
    assert tsg.moe_expert_combine(*args, c.wsb, 32768, 128, 64, 4, 2, raise_on_error=False) == tsg.E_UNSUPPORTED
    # expert ids must be 16-byte aligned (read as vectors)
    ids_off = c.ids.view(-1)[1:]
    args_off = (ctx, c.x, ids_off, c.g, c.wu, c.wd, c.out, c.counts, c.sorted, c.ws)
    assert tsg.moe_expert_combine(*args_off, c.wsb, 31, 128, 64, 4, 2, raise_on_error=False) == tsg.E_ALIGN


def test_moe_missing_row_block_times_out_then_recovers(env):
    torch, tsg, ctx = env
    inp = moe_inputs(256, 256, 128, 4, k=2, seed=36)
    case = MoeCase(env, inp)
    case.run(opts={"debug_skip_mask": 1 << 1, "timeout_ms": 20}, expect=tsg.E_TIMEOUT)
    out, counts, sorted_ids = case.run()
    r, _, _ = _check(case, out, counts, sorted_ids)
    assert r <= 1.0


@pytest.mark.parametrize("T,H,I,E", [(300, 512, 256, 8), (37, 136, 200, 3)])
def test_moe_bf16_staging(env, T, H, I, E):
    # y staged in bf16: within the bound widened by one rounding of y per
    # slot; identical across modes and CU splits; a bad stage type is refused
    torch, tsg, ctx = env
    inp = moe_inputs(T, H, I, E, k=2, seed=40 + T)
    case = MoeCase(env, inp)
    opt = {"stage_dtype": tsg.BF16}
    out, counts, sorted_ids = case.run(opts=opt)
    r, _, _ = _check(case, out, counts, sorted_ids, y_bf16=True)
    assert r <= 1.0
    for mode in (tsg.SERIAL, tsg.COMPUTE_ONLY):
        case.run(mode=mode, opts=opt)
    out2, _, _ = case.run(mode=tsg.COMM_ONLY, opts=opt)
    assert np.array_equal(out2, out)
    out3, _, _ = case.run(opts=dict(opt, aux_cus=16))
    assert np.array_equal(out3, out)
    with pytest.raises(tsg.TsgError):
        case.run(opts={"stage_dtype": 2})


def test_moe_full_size_parity_modes_splits(env):
    # the Zipf-routed workload at full size: the shared-CU default and the
    # 16-CU combine consumer each checked in full against the oracle
    torch, tsg, ctx = env
    cfg = CONFIGS["moe"]
    inp = moe_inputs(cfg["T"], cfg["H"], cfg["I"], cfg["E"], k=cfg["k"], seed=cfg["seed"], zipf=cfg["zipf"])
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    r, _, r_plain = _check(case, out, counts, sorted_ids, label="overlap, shared CUs")
    # with fp32 staging the output also meets the plain per-element GEMM
    # bound of the down projection, with no allowance for h differences
    assert r <= 1.0 and r_plain <= 1.0
    out16, c16, s16 = case.run(opts={"aux_cus": 16})
    r16, _, r16_plain = _check(case, out16, c16, s16, label="overlap, 16-CU combine consumer")
    assert r16 <= 1.0 and r16_plain <= 1.0
    assert np.array_equal(out16, out)
    out2, c2, s2 = case.run(mode=tsg.SERIAL)
    assert np.array_equal(out2, out) and np.array_equal(c2, counts) and np.array_equal(s2, sorted_ids)
    # the combine alone, over the staging the serial call left
    out3, _, _ = case.run(mode=tsg.COMM_ONLY)
    assert np.array_equal(out3, out)
    for opts in ({"aux_cus": 32}, {"aux_cus": -1}):
        out4, _, _ = case.run(opts=opts)
        assert np.array_equal(out4, out), opts
    out5, c5, s5 = case.run(opts={"stage_dtype": tsg.BF16})
    r5, _, _ = _check(case, out5, c5, s5, y_bf16=True, label="bf16 y staging")
    assert r5 <= 1.0


def _remote_first_order(inp, E, bm, ep_ranks, ep_rank):
    """Row blocks in remote-critical order, from the oracle's routing: the
    blocks holding a pair of a token from another source rank (tokens of rank
    c are [c T / ep_ranks, (c + 1) T / ep_ranks)), then the others, each group
    by block index."""
    ids = inp["topk_ids"]
    T, k = ids.shape
    counts, offsets, sorted_ids = oracle.moe_route(ids, E)
    poff, tiles = oracle.moe_tile_table(counts, bm)
    remote = []
    for e, lo, n in tiles:
        pairs = sorted_ids[offsets[e] + (lo - poff[e]):offsets[e] + (lo - poff[e]) + n]
        remote.append(bool(np.any((pairs // k) // (T // ep_ranks) != ep_rank)))
    first = [rb for rb, r in enumerate(remote) if r]
    return np.array(first + [rb for rb, r in enumerate(remote) if not r], dtype=np.int32), remote


def test_moe_remote_critical_order(env):
    # opts.ep_ranks / ep_rank: the producer takes the row blocks holding a
    # token of another rank first.  The tokens of rank 1 go to experts 0 and 1
    # only and the others' to experts 2 and 3, so both kinds of block exist.
    # The device's order table is the oracle's, and every output is
    # bit-identical to the plain order's, in every mode and CU split.
    torch, tsg, ctx = env
    T, H, I, E, R, rank = 1024, 256, 128, 4, 4, 1
    inp = moe_inputs(T, H, I, E, k=2, seed=37)
    tpr = T // R
    rng = np.random.default_rng(38)
    ids = np.empty((T, 2), dtype=np.int32)
    for t in range(T):
        pool = [0, 1] if t // tpr == rank else [2, 3]
        ids[t] = rng.permutation(pool)
    inp["topk_ids"] = ids
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    _check(case, out, counts, sorted_ids)
    want, remote = _remote_first_order(inp, E, case.lay["bm"], R, rank)
    assert any(remote) and not all(remote)
    prio = {"ep_ranks": R, "ep_rank": rank}
    for mode, opts in ((tsg.OVERLAP, prio), (tsg.OVERLAP, dict(prio, aux_cus=16)), (tsg.SERIAL, prio),
                       (tsg.COMPUTE_ONLY, prio)):
        o2, c2, s2 = case.run(mode=mode, opts=opts)
        assert np.array_equal(c2, counts) and np.array_equal(s2, sorted_ids)
        n_rb = int(case.tables()["meta"][0])
        L = case.lay
        got = case.ws.cpu().numpy()[L["rb_order"]:L["rb_order"] + 4 * n_rb].view(np.int32)
        assert np.array_equal(got, want), (mode, opts)
        if mode != tsg.COMPUTE_ONLY:
            assert np.array_equal(o2, out), (mode, opts)
    # the combine alone over the staging of the last call: plain order
    o3, _, _ = case.run(mode=tsg.COMM_ONLY, opts=prio)
    assert np.array_equal(o3, out)
    for bad in ({"ep_ranks": 3, "ep_rank": 0}, {"ep_ranks": 4, "ep_rank": 4}, {"ep_ranks": 33, "ep_rank": 0},
                {"ep_ranks": -1, "ep_rank": 0}):
        with pytest.raises(tsg.TsgError):
            case.run(opts=bad)


def test_moe_remote_critical_order_full_size(env):
    # the Zipf-routed workload with 8 source ranks: each expert's rows are in
    # token order, so a row block spans few source ranks and some hold only
    # this rank's tokens; the order table matches the oracle's and out is
    # bit-identical to the plain order's
    torch, tsg, ctx = env
    cfg = CONFIGS["moe"]
    inp = moe_inputs(cfg["T"], cfg["H"], cfg["I"], cfg["E"], k=cfg["k"], seed=cfg["seed"], zipf=cfg["zipf"])
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    for rank in (0, 7):
        want, remote = _remote_first_order(inp, cfg["E"], case.lay["bm"], 8, rank)
        o2, _, _ = case.run(opts={"ep_ranks": 8, "ep_rank": rank})
        assert np.array_equal(o2, out)
        n_rb = len(want)
        L = case.lay
        got = case.ws.cpu().numpy()[L["rb_order"]:L["rb_order"] + 4 * n_rb].view(np.int32)
        assert np.array_equal(got, want), rank
        print(f"rank {rank}: {sum(remote)} of {n_rb} row blocks remote-critical")
