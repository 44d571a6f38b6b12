"""MoE expert compute + overlapped gate-weighted combine on the GPU against
the oracle.

Routing bookkeeping (expert_counts, sorted_ids) must match bit for bit.  out is
pre-filled with NaN, so a token never combined, or combined from a tile read
before its ready signal, shows up as a non-finite element.

Bound on out: the GEMM bound on the down projection with the oracle's h,
1e-3 * sum_s g_s sum_k |h_sk w_down_kj| + 1e-5, plus the effect of the largest
difference the device's h may have from the oracle's: per element of h,
1.1 * (1e-3 * sum |x w_up| + 1e-5) (|SiLU'| <= 1.1) plus one bf16 quantum,
carried through |w_down| and the gates."""
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
        self.wsb = tsg.workspace_bytes(tsg.OP_MOE, [T, H, I, E, self.k])
        assert self.wsb > 0
        self.ws = torch.empty((self.wsb,), dtype=torch.uint8, device="cuda")

    def run(self, mode=None, opts=None, expect=0, poison=True):
        torch, tsg, ctx = self.env
        mode = tsg.OVERLAP if mode is None else mode
        if poison:
            self.out.fill_(float("nan"))
            self.counts.fill_(-7)
            self.sorted.fill_(-7)
        tsg.moe_expert_combine(ctx, self.x, self.ids, self.g, self.wu, self.wd, self.out, self.counts,
                               self.sorted, self.ws, self.wsb, self.T, self.H, self.I, self.E, self.k,
                               opts=opts, mode=mode)
        st = ctx.check()
        assert st == expect, (st, ctx.last_error())
        return (self.out.cpu().numpy().astype(np.float64), self.counts.cpu().numpy(),
                self.sorted.cpu().numpy())


def _bound(inp, res, y_bf16=False):
    """Per-element tolerance of out (see module docstring).  With the y
    staging in bf16, each slot's y is rounded once more before the combine:
    its gate times one bf16 quantum of y (twice the half quantum, as the
    device's y may lie across a power of two from the oracle's) is added."""
    x = oracle.bf16_to_f64(inp["x"])
    ids, g = inp["topk_ids"], inp["topk_w"].astype(np.float64)
    T, k = ids.shape
    H = inp["w_down"].shape[2]
    extra = np.zeros((T * k, H))
    for e in range(inp["w_up"].shape[0]):
        pairs = np.nonzero(ids.reshape(-1) == e)[0]
        if pairs.size == 0:
            continue
        s_up = np.abs(x[pairs // k]) @ np.abs(oracle.bf16_to_f64(inp["w_up"][e]))
        h = oracle.bf16_to_f64(res["h"][pairs])
        dh = 1.1 * (1e-3 * s_up + 1e-5) + 2 * bf16_half_quantum(h)
        extra[pairs] = dh @ np.abs(oracle.bf16_to_f64(inp["w_down"][e]))
    if y_bf16:
        extra = extra + 2 * bf16_half_quantum(res["y"])
    extra = (g.reshape(-1)[:, None] * extra).reshape(T, k, H).sum(axis=1)
    return 1e-3 * res["scale"] + 1e-5 + extra


def _check(inp, out, counts, sorted_ids, y_bf16=False):
    res = oracle.moe_expert_combine(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_up"], inp["w_down"])
    assert np.array_equal(counts, res["counts"])
    assert np.array_equal(sorted_ids, res["sorted_ids"])
    assert np.all(np.isfinite(out))
    r = float(np.max(np.abs(out - res["out"]) / _bound(inp, res, y_bf16)))
    return r, res


# (9000, ...) and (32767, ...): routed pair blocks of 128 and 256 pairs, the
# second at the largest T * k the routing takes (65534 pairs)
@pytest.mark.parametrize("T,H,I,E", [(100, 256, 128, 4), (37, 136, 200, 3), (1, 64, 64, 2), (300, 512, 256, 8),
                                     (9000, 64, 72, 5), (32767, 64, 64, 8)])
def test_moe_small(env, T, H, I, E):
    inp = moe_inputs(T, H, I, E, k=2, seed=T + E)
    out, counts, sorted_ids = MoeCase(env, inp).run()
    r, _ = _check(inp, out, counts, sorted_ids)
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
    r, _ = _check(inp, out, counts, sorted_ids)
    assert r <= 1.0
    assert counts[0] == T


def test_moe_zero_gate_slot_is_ignored_bit_exactly(env):
    T, H, I, E = 200, 256, 128, 6
    inp = moe_inputs(T, H, I, E, k=2, seed=32)
    g = np.zeros_like(inp["topk_w"])
    g[:, 0] = 1.0
    inp["topk_w"] = g
    out1, c1, s1 = MoeCase(env, inp).run()
    r, _ = _check(inp, out1, c1, s1)
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
    out, counts, sorted_ids = MoeCase(env, inp).run()
    r, res = _check(inp, out, counts, sorted_ids)
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
    r, _ = _check(inp, out, counts, sorted_ids)
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
    r, _ = _check(inp, out, counts, sorted_ids, y_bf16=True)
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
    torch, tsg, ctx = env
    cfg = CONFIGS["moe"]
    inp = moe_inputs(cfg["T"], cfg["H"], cfg["I"], cfg["E"], k=cfg["k"], seed=cfg["seed"], zipf=cfg["zipf"])
    case = MoeCase(env, inp)
    out, counts, sorted_ids = case.run()
    r, _ = _check(inp, out, counts, sorted_ids)
    print(f"moe max err/tol {r:.3f}, expert counts {counts.tolist()}")
    assert r <= 1.0
    out2, c2, s2 = case.run(mode=tsg.SERIAL)
    assert np.array_equal(out2, out) and np.array_equal(c2, counts) and np.array_equal(s2, sorted_ids)
    out3, _, _ = case.run(mode=tsg.COMM_ONLY)
    assert np.array_equal(out3, out)
    for opts in ({"aux_cus": 16}, {"aux_cus": 32}, {"aux_cus": -1}):
        out4, _, _ = case.run(opts=opts)
        assert np.array_equal(out4, out), opts
    out5, c5, s5 = case.run(opts={"stage_dtype": tsg.BF16})
    r5, _ = _check(inp, out5, c5, s5, y_bf16=True)
    print(f"moe bf16 staging max err/tol {r5:.3f}")
    assert r5 <= 1.0
