"""AllGather KV + self-attention (sequence parallel) on the GPU against the
oracle.

Before every call k_full / v_full are filled with bf16 NaN and out with
0xFFFF, so a tile that read a peer's keys or values before their signals, or
an output never written, shows up as a non-finite element.  k_full and
v_full must equal the gathered context bit for bit.  out is compared per
element with the oracle's float64 attention under the bound

    |gpu - ref| <= (1e-3 + 2^-8 + 2 ds) sum_j P_j |V_jd| + half a bf16 quantum of ref + 1e-5,

where 1e-3 sum_j P_j |V_jd| is the GEMM bound of the P V product, 2^-8
covers the device's rounding of P to bf16 (2^-9 relative per probability),
ds = D * 2^-24 * max_j sum_d |q_d K_jd| / sqrt(D) bounds the fp32 rounding of
a score (which moves each probability by at most a factor e^(2 ds)), and
the last terms cover the bf16 output.  For one arrival order, results are
bit-identical across modes and slab widths (a tile accumulates its own chunk
first, then the others in arrival order, so another order sums in another
order and is checked against the bound)."""
import numpy as np
import pytest

import oracle
from _helpers import bf16_from_dev, bf16_half_quantum, to_dev
from synth import f32_to_bf16_bits
from synth.gen import split_chunks

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0
D = 128


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    # a dedicated stream, as the benchmark uses (the null stream, on which
    # every call joins, is covered by its own test)
    torch.cuda.set_stream(torch.cuda.Stream())
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.default_stream())
    ctx.close()


def _inputs(S, heads, seed):
    rng = np.random.default_rng(seed)
    mk = lambda shape: f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    return dict(q_all=mk((S, heads, D)), k=mk((S, heads, D)), v=mk((S, heads, D)))


class Case:
    def __init__(self, env, inp, S, heads, R, rank):
        torch, tsg, ctx = env
        self.env, self.inp, self.S, self.heads, self.R, self.rank = env, inp, S, heads, R, rank
        sl = S // R
        self.q_np = inp["q_all"][rank * sl:(rank + 1) * sl]
        kl, kp = split_chunks(inp["k"], R, rank)
        vl, vp = split_chunks(inp["v"], R, rank)
        dummy = np.zeros((1, 8), np.uint16)
        self.q = to_dev(self.q_np, torch)
        self.kl, self.vl = to_dev(kl, torch), to_dev(vl, torch)
        self.kp = to_dev(kp if R > 1 else dummy, torch)
        self.vp = to_dev(vp if R > 1 else dummy, torch)
        self.kf = torch.empty((S, heads, D), dtype=torch.int16, device="cuda")
        self.vf = torch.empty((S, heads, D), dtype=torch.int16, device="cuda")
        self.out = torch.empty((sl, heads, D), dtype=torch.int16, device="cuda")

    def run(self, mode=None, order=None, opts=None, expect=0, poison=True):
        torch, tsg, ctx = self.env
        mode = tsg.OVERLAP if mode is None else mode
        if poison:
            if mode != tsg.COMPUTE_ONLY:
                self.kf.fill_(NAN_BF16)
                self.vf.fill_(NAN_BF16)
            self.out.fill_(-1)
        tsg.ag_kv_attention(ctx, self.q, self.kl, self.kp, self.vl, self.vp, self.kf, self.vf, self.out, self.S,
                            self.heads, D, self.R, self.rank, arrival_order=order, opts=opts, mode=mode)
        st = ctx.check()
        assert st == expect, (st, ctx.last_error())
        return bf16_from_dev(self.kf), bf16_from_dev(self.vf), bf16_from_dev(self.out)


def _check(case, kf, vf, out, rows=None, label=""):
    inp = case.inp
    assert np.array_equal(kf, inp["k"]) and np.array_equal(vf, inp["v"])
    q = case.q_np if rows is None else case.q_np[rows]
    ref = oracle.attention(q, inp["k"], inp["v"])
    got = oracle.bf16_to_f64(out if rows is None else out[rows])
    assert np.all(np.isfinite(got))
    ds = D * 2.0 ** -24 * ref["qk_abs_max"] / np.sqrt(D)
    tol = (1e-3 + 2.0 ** -8 + 2 * ds[:, :, None]) * ref["pv_abs"] + bf16_half_quantum(ref["out"]) + 1e-5
    r = float(np.max(np.abs(got - ref["out"]) / tol))
    if label:
        print(f"attention {label}: max err/tol {r:.4f}")
    assert r <= 1.0, r
    return r


@pytest.mark.parametrize("S,heads,R", [(256, 2, 4), (512, 3, 2), (128, 1, 1), (1536, 2, 8)])
def test_attention_small_all_ranks(env, S, heads, R):
    torch, tsg, ctx = env
    inp = _inputs(S, heads, seed=S + heads + R)
    for rank in range(R):
        case = Case(env, inp, S, heads, R, rank)
        kf, vf, out = case.run()
        _check(case, kf, vf, out)


def test_attention_modes_orders_slabs(env):
    torch, tsg, ctx = env
    S, heads, R, rank = 1024, 4, 4, 1
    inp = _inputs(S, heads, seed=81)
    case = Case(env, inp, S, heads, R, rank)
    kf, vf, out = case.run()
    _check(case, kf, vf, out)
    for mode in (tsg.SERIAL, tsg.COMPUTE_ONLY):
        _, _, o2 = case.run(mode=mode)
        assert np.array_equal(o2, out), mode
    # overlapped with the copy units in the attention kernel's own queue
    # instead of a copy kernel beside it: the same bits
    kf2, vf2, o2 = case.run(opts={"pull_units": 1})
    assert np.array_equal(o2, out)
    assert np.array_equal(kf2, inp["k"]) and np.array_equal(vf2, inp["v"])
    kf3, vf3, _ = case.run(mode=tsg.COMM_ONLY)
    assert np.array_equal(kf3, inp["k"]) and np.array_equal(vf3, inp["v"])
    # another arrival order changes the order in which a tile accumulates
    # the chunks (its own first, then as they arrive): within the bound;
    # for one order, every slab width gives the same bits
    for order in ([0, 2, 3], [3, 0, 2]):
        kf4, vf4, o_ord = case.run(order=order)
        _check(case, kf4, vf4, o_ord)
        for ct in (64, 256, 2048):
            _, _, o4 = case.run(order=order, opts={"comm_tile": ct})
            assert np.array_equal(o4, o_ord), (order, ct)
    for bad, want in (({"aux_cus": 16}, tsg.E_UNSUPPORTED), ({"comm_tile": 32}, tsg.E_INVALID)):
        st = tsg.ag_kv_attention(ctx, case.q, case.kl, case.kp, case.vl, case.vp, case.kf, case.vf, case.out, S,
                                 heads, D, R, rank, opts=bad, raise_on_error=False)
        assert st == want, bad
    st = tsg.ag_kv_attention(ctx, case.q, case.kl, case.kp, case.vl, case.vp, case.kf, case.vf, case.out, S,
                             heads, 64, R, rank, raise_on_error=False)
    assert st == tsg.E_UNSUPPORTED
    st = tsg.ag_kv_attention(ctx, case.q, case.kl, case.kp, case.vl, case.vp, case.kf, case.vf, case.out, 1000,
                             heads, D, R, rank, raise_on_error=False)
    assert st == tsg.E_SHAPE


def test_attention_joined_through_the_attention_kernel(env):
    # Overlapped with a copy kernel beside it, the caller's stream waits for
    # the attention kernel only; its tiles wait for their head's own-chunk
    # slabs after their stores.  Calls back to back with no synchronisation,
    # alternating two cases, then the other launch forms, must leave every
    # output whole when the stream alone is synchronised.
    torch, tsg, ctx = env
    S, heads, R = 1024, 4, 4
    inps = [_inputs(S, heads, seed=90 + i) for i in range(4)]
    cases = [Case(env, x, S, heads, R, i % R) for i, x in enumerate(inps)]

    def launch(c, mode=None, opts=None):
        c.kf.fill_(NAN_BF16)
        c.vf.fill_(NAN_BF16)
        c.out.fill_(-1)
        tsg.ag_kv_attention(ctx, c.q, c.kl, c.kp, c.vl, c.vp, c.kf, c.vf, c.out, S, heads, D, R, c.rank,
                            opts=opts, mode=tsg.OVERLAP if mode is None else mode)
    for i in range(8):
        launch(cases[i % 2])
    torch.cuda.current_stream().synchronize()
    for c in cases[:2]:
        _check(c, bf16_from_dev(c.kf), bf16_from_dev(c.vf), bf16_from_dev(c.out))
    launch(cases[0])                           # detached
    launch(cases[1], mode=tsg.SERIAL)          # copy units, then tiles, one kernel
    launch(cases[2], opts={"pull_units": 1})   # copy units in the attention kernel's own queue
    launch(cases[3])                           # detached
    torch.cuda.current_stream().synchronize()
    for c in cases:
        _check(c, bf16_from_dev(c.kf), bf16_from_dev(c.vf), bf16_from_dev(c.out))
    assert ctx.check() == tsg.OK, ctx.last_error()


def test_attention_on_the_null_stream(env):
    torch, tsg, ctx = env
    S, heads, R = 512, 2, 4
    inp = _inputs(S, heads, seed=95)
    with torch.cuda.stream(torch.cuda.default_stream()):
        case = Case(env, inp, S, heads, R, 2)
        kf, vf, out = case.run()
    _check(case, kf, vf, out)


def test_attention_special_cases(env):
    # constant V rows: every output equals that row; zero queries: the
    # output is the mean of the V rows
    torch, tsg, ctx = env
    S, heads, R, rank = 512, 2, 4, 2
    inp = _inputs(S, heads, seed=82)
    row = inp["v"][:1]
    inp_c = dict(inp, v=np.repeat(row, S, axis=0))
    case = Case(env, inp_c, S, heads, R, rank)
    kf, vf, out = case.run()
    assert np.array_equal(out, np.broadcast_to(row, out.shape))
    inp_z = dict(inp, q_all=np.zeros_like(inp["q_all"]))
    case = Case(env, inp_z, S, heads, R, rank)
    kf, vf, out = case.run()
    _check(case, kf, vf, out)
    mean = oracle.bf16_to_f64(inp["v"]).mean(axis=0)
    got = oracle.bf16_to_f64(out)
    assert np.max(np.abs(got - mean[None]) / (2.0 ** -7 * np.abs(mean[None]) + 2.0 ** -7)) <= 1.0


def test_attention_waits_for_its_chunks(env):
    # with chunk c's signals withheld (20 ms bound), every tile waits out the
    # bound unless c is this rank's own chunk, which tiles read in place
    torch, tsg, ctx = env
    S, heads, R, rank = 512, 2, 4, 1
    inp = _inputs(S, heads, seed=83)
    case = Case(env, inp, S, heads, R, rank)
    case.run()
    # both overlapped forms: copy kernel beside the tiles, copy units in
    # the attention kernel's queue
    for pull in (0, 1):
        for c in range(R):
            expect = tsg.OK if c == rank else tsg.E_TIMEOUT
            case.run(opts={"debug_skip_mask": 1 << c, "timeout_ms": 20, "timeline": 1, "pull_units": pull},
                     expect=expect)
            recs = [r for r in ctx.timeline() if (r[0] >> 56) == 11]
            assert len(recs) == heads * ((S // R + 127) // 128)
            long = sum(1 for r in recs if r[2] - r[1] > 1_000_000)
            assert long == (0 if c == rank else len(recs)), (pull, c, long)
    kf, vf, out = case.run()
    _check(case, kf, vf, out)


def test_attention_16k_sampled(env):
    # the 16k-token context of 32 heads at one rank's share of 8: 2048
    # queries; the oracle checks a sample of query rows in full
    torch, tsg, ctx = env
    S, heads, R, rank = 16384, 32, 8, 3
    inp = _inputs(S, heads, seed=84)
    case = Case(env, inp, S, heads, R, rank)
    kf, vf, out = case.run()
    rows = np.random.default_rng(5).choice(S // R, size=48, replace=False)
    _check(case, kf, vf, out, rows=rows, label="16k context, 32 heads, 48 sampled queries")
    _, _, o2 = case.run(mode=tsg.SERIAL)
    assert np.array_equal(o2, out)
