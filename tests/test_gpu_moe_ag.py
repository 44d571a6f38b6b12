"""AllGather + gather + grouped GEMM (the gather side of a tensor-parallel
MoE layer) on the GPU against the oracle.

Before every call x_full is filled with bf16 NaN and h with 0xFFFF (NaN), so a
tile that read gathered tokens before their chunk's signal, or a pair whose
row was never stored, shows up as a non-finite element.  x_full must equal the
gathered tokens bit for bit, expert_counts and sorted_ids the oracle's; h is
bf16(SiLU(u)) with u within the GEMM bound 1e-3 * sum_k |x w_up| + 1e-5 of the
oracle's, which |SiLU'| <= 1.1 carries into h, plus one bf16 quantum for the
two roundings.  Every rank and several arrival orders give bit-identical h."""
import numpy as np
import pytest

import oracle
from _helpers import bf16_from_dev, bf16_half_quantum, to_dev
from synth import CONFIGS, moe_inputs
from synth.gen import split_chunks

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    ctx.close()


class Case:
    def __init__(self, env, inp, R, rank):
        torch, tsg, ctx = env
        self.env, self.inp, self.R, self.rank = env, inp, R, rank
        T, H = inp["x"].shape
        E, _, I = inp["w_up"].shape
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, inp["topk_ids"].shape[1]
        loc, peers = split_chunks(inp["x"], R, rank)
        self.loc = to_dev(loc, torch)
        self.peers = to_dev(peers if R > 1 else np.zeros((1, 8), np.uint16), torch)
        self.ids = to_dev(inp["topk_ids"], torch)
        self.wu = to_dev(inp["w_up"], torch)
        self.full = torch.empty((T, H), dtype=torch.int16, device="cuda")
        self.h = torch.empty((T * self.k, I), dtype=torch.int16, device="cuda")
        self.counts = torch.empty((E,), dtype=torch.int32, device="cuda")
        self.sorted = torch.empty((T * self.k,), dtype=torch.int32, device="cuda")
        self.wsb = tsg.workspace_bytes(tsg.OP_MOE_AG, [T, H, I, E, self.k])
        assert self.wsb > 0
        self.ws = torch.empty((self.wsb,), dtype=torch.uint8, device="cuda")

    def run(self, mode=None, order=None, opts=None, expect=0, poison=True):
        torch, tsg, ctx = self.env
        mode = tsg.OVERLAP if mode is None else mode
        if poison:
            if mode != tsg.COMPUTE_ONLY:
                self.full.fill_(NAN_BF16)
            self.h.fill_(-1)
            self.counts.fill_(-7)
            self.sorted.fill_(-7)
            self.ws.fill_(0xFF)
        tsg.moe_ag_group_gemm(ctx, self.loc, self.peers, self.full, self.ids, self.wu, self.h, self.counts,
                              self.sorted, self.ws, self.wsb, self.T, self.H, self.I, self.E, self.k, self.R,
                              self.rank, arrival_order=order, opts=opts, mode=mode)
        st = ctx.check()
        assert st == expect, (st, ctx.last_error())
        return (bf16_from_dev(self.full), bf16_from_dev(self.h), self.counts.cpu().numpy(),
                self.sorted.cpu().numpy())


def _check(case, full, h, counts, sorted_ids, label=""):
    inp = case.inp
    loc, peers = split_chunks(inp["x"], case.R, case.rank)
    res = oracle.moe_ag_up(loc, peers, case.R, case.rank, inp["topk_ids"], inp["w_up"])
    assert np.array_equal(full, res["x_full"])
    assert np.array_equal(counts, res["counts"]) and np.array_equal(sorted_ids, res["sorted_ids"])
    hg, hr = oracle.bf16_to_f64(h), oracle.bf16_to_f64(res["h"])
    assert np.all(np.isfinite(hg))
    tol = 1.1 * (1e-3 * res["scale"] + 1e-5) + 2 * bf16_half_quantum(hr) + 1e-7
    r = float(np.max(np.abs(hg - hr) / tol))
    if label:
        print(f"moe_ag {label}: max err/tol {r:.4f}, expert counts {counts.tolist()}")
    assert r <= 1.0, r
    return r


@pytest.mark.parametrize("T,H,I,E,R", [(64, 256, 128, 4, 4), (60, 200, 72, 3, 3), (8, 64, 16, 2, 1),
                                       (512, 512, 448, 8, 8)])
def test_moe_ag_small_all_ranks(env, T, H, I, E, R):
    torch, tsg, ctx = env
    inp = moe_inputs(T, H, I, E, k=2, seed=T + H + R)
    first = None
    for rank in range(R):
        case = Case(env, inp, R, rank)
        full, h, counts, sorted_ids = case.run()
        _check(case, full, h, counts, sorted_ids)
        first = h if first is None else first
        assert np.array_equal(h, first), rank


def test_moe_ag_modes_orders_and_slabs(env):
    # serial, compute-only (over the gathered tokens of the previous call),
    # comm-only, other arrival orders and slab widths: the same bits
    torch, tsg, ctx = env
    T, H, I, E, R, rank = 96, 384, 224, 5, 4, 2
    inp = moe_inputs(T, H, I, E, k=2, seed=71)
    case = Case(env, inp, R, rank)
    full, h, counts, sorted_ids = case.run()
    _check(case, full, h, counts, sorted_ids)
    for mode in (tsg.SERIAL, tsg.COMPUTE_ONLY):
        _, h2, _, _ = case.run(mode=mode)
        assert np.array_equal(h2, h), mode
    full3, _, _, _ = case.run(mode=tsg.COMM_ONLY)
    assert np.array_equal(full3, inp["x"])
    for order in ([0, 1, 3], [3, 1, 0]):
        for ct in (0, 128, 64):
            _, h4, _, _ = case.run(order=order, opts={"comm_tile": ct})
            assert np.array_equal(h4, h), (order, ct)
    for bad in ({"aux_cus": 16}, {"comm_tile": 48}):
        st = tsg.moe_ag_group_gemm(ctx, case.loc, case.peers, case.full, case.ids, case.wu, case.h, case.counts,
                                   case.sorted, case.ws, case.wsb, T, H, I, E, 2, R, rank, opts=bad,
                                   raise_on_error=False)
        assert st in (tsg.E_UNSUPPORTED, tsg.E_INVALID), bad


def test_moe_ag_rank_mapping_waits_for_exactly_its_chunks(env):
    # dynamic rank mapping: with chunk c's signals withheld (20 ms bound),
    # the tiles that wait out the bound are exactly those of the row blocks
    # that gather a token of chunk c (computed here from the oracle's routing
    # and tile table).  Tokens of one chunk routed to one expert make the
    # blocks' rank sets differ.
    torch, tsg, ctx = env
    T, H, I, E, R, rank = 1024, 128, 224, 4, 4, 0
    inp = moe_inputs(T, H, I, E, k=2, seed=72)
    ids = np.zeros((T, 2), dtype=np.int32)
    tpr = T // R
    for t in range(T):
        ids[t] = (t // tpr, (t // tpr + 1) % E)   # chunk c -> experts c and c+1
    inp["topk_ids"] = ids
    case = Case(env, inp, R, rank)
    counts, offsets, sorted_ids = oracle.moe_route(ids, E)
    poff, tiles = oracle.moe_tile_table(counts, 256)
    masks = []
    for e, lo, n in tiles:
        pairs = sorted_ids[offsets[e] + (lo - poff[e]):offsets[e] + (lo - poff[e]) + n]
        masks.append({int(p // 2 // tpr) for p in pairs})
    case.run(opts={"tile": 0})  # one plain call first
    for c in range(R):
        want = {rb for rb, m in enumerate(masks) if c in m}
        case.run(opts={"debug_skip_mask": 1 << c, "timeout_ms": 20, "timeline": 1}, expect=tsg.E_TIMEOUT)
        recs = [r for r in ctx.timeline() if (r[0] >> 56) == 10]
        waited = {(r[0] & 0xFFFFFFFF) >> 16 for r in recs if r[2] - r[1] > 1_000_000}
        assert waited == want, (c, waited, want)
    full, h, counts_d, sorted_d = case.run()
    _check(case, full, h, counts_d, sorted_d)


def test_moe_ag_full_size(env):
    # the MoE workload's tokens and expert sizes, gathered from 8 ranks
    torch, tsg, ctx = env
    cfg = CONFIGS["moe"]
    inp = moe_inputs(cfg["T"], cfg["H"], cfg["I"], cfg["E"], k=cfg["k"], seed=cfg["seed"], zipf=cfg["zipf"])
    case = Case(env, inp, 8, 0)
    full, h, counts, sorted_ids = case.run()
    _check(case, full, h, counts, sorted_ids, label="overlap, 8 ranks")
    _, h2, _, _ = case.run(mode=tsg.SERIAL)
    assert np.array_equal(h2, h)
