"""GEMM + ReduceScatter on the GPU against the oracle.

The partial buffer and the output are pre-filled with NaN, so an output tile
that added its local partial before the producer's done signal, or a tile that
was never written, shows up as a non-finite element."""
import numpy as np
import pytest

import oracle
from _helpers import err_ratio, to_dev
from synth import CONFIGS, rs_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    # a dedicated stream, as the benchmark uses (the null stream is covered
    # by its own test)
    torch.cuda.set_stream(torch.cuda.Stream())
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.default_stream())
    ctx.close()


class RsCase:
    def __init__(self, env, inp, M, N, K, R, rank):
        torch, tsg, ctx = env
        self.env, self.M, self.N, self.K, self.R, self.rank = env, M, N, K, R, rank
        self.x = to_dev(inp["x"], torch)
        self.w = to_dev(inp["w"], torch)
        self.peers = to_dev(inp["peer_partials"] if R > 1 else np.zeros((1, 4), np.float32), torch)
        self.partial = torch.empty((M, N), dtype=torch.float32, device="cuda")
        self.out = torch.empty((M // R, N), dtype=torch.float32, device="cuda")

    def run(self, mode=None, opts=None, poison=True, expect=0):
        torch, tsg, ctx = self.env
        mode = tsg.OVERLAP if mode is None else mode
        if poison:
            self.out.fill_(float("nan"))
            if mode != tsg.COMM_ONLY:
                self.partial.fill_(float("nan"))
        tsg.gemm_rs_overlap(ctx, self.x, self.w, self.partial, self.peers, self.out, self.M, self.N, self.K,
                            self.R, self.rank, opts=opts, mode=mode)
        st = ctx.check()
        assert st == expect, (st, ctx.last_error())
        return self.partial.cpu().numpy().astype(np.float64), self.out.cpu().numpy().astype(np.float64)


def _ref(inp, R, rank):
    P, out = oracle.gemm_rs(inp["x"], inp["w"], inp["peer_partials"], R, rank)
    sP = oracle.gemm_abs(inp["x"], inp["w"])
    mr = P.shape[0] // R
    s_out = sP[rank * mr:(rank + 1) * mr] + np.abs(inp["peer_partials"].astype(np.float64)).sum(axis=0)
    return P, out, sP, s_out


@pytest.mark.parametrize("tile", [3, 1, 4, 6])
def test_rs_small_all_ranks(env, tile):
    M, N, K, R = 512, 256, 128, 4
    inp = rs_inputs(M, K, N, R, seed=3)
    outs = []
    for rank in range(R):
        inp_r = rs_inputs(M, K, N, R, rank=rank, seed=3)
        P, out, sP, s_out = _ref(inp_r, R, rank)
        case = RsCase(env, inp_r, M, N, K, R, rank)
        gP, gout = case.run(opts={"tile": tile})
        assert err_ratio(gP, P, sP) <= 1.0
        assert err_ratio(gout, out, s_out) <= 1.0
        outs.append(gP)
    assert all(np.array_equal(o, outs[0]) for o in outs)


@pytest.mark.parametrize("tile", [3, 1])
def test_rs_ragged(env, tile):
    M, N, K, R = 600, 200, 136, 3      # 200-row chunks straddle 128-row signal tiles
    for rank in range(R):
        inp = rs_inputs(M, K, N, R, rank=rank, seed=4)
        P, out, sP, s_out = _ref(inp, R, rank)
        case = RsCase(env, inp, M, N, K, R, rank)
        gP, gout = case.run(opts={"tile": tile})
        assert err_ratio(gP, P, sP) <= 1.0 and err_ratio(gout, out, s_out) <= 1.0


def test_rs_zero_peers_gives_local_partial_exactly(env):
    M, N, K, R = 512, 384, 256, 4
    inp = rs_inputs(M, K, N, R, rank=2, seed=5)
    inp["peer_partials"] = np.zeros_like(inp["peer_partials"])
    case = RsCase(env, inp, M, N, K, R, 2)
    gP, gout = case.run()
    assert np.array_equal(gout, gP[256:384])


def test_rs_single_rank(env):
    M, N, K, R = 256, 128, 64, 1
    inp = rs_inputs(M, K, N, R, seed=6)
    P, out, sP, s_out = _ref(inp, R, 0)
    case = RsCase(env, inp, M, N, K, R, 0)
    gP, gout = case.run()
    assert np.array_equal(gout, gP) and err_ratio(gP, P, sP) <= 1.0


def test_rs_missing_tile_times_out_then_recovers(env):
    torch, tsg, ctx = env
    M, N, K, R = 512, 256, 128, 4
    inp = rs_inputs(M, K, N, R, rank=1, seed=7)
    P, out, sP, s_out = _ref(inp, R, 1)
    case = RsCase(env, inp, M, N, K, R, 1)
    case.run(opts={"debug_skip_mask": 1 << 1, "timeout_ms": 20}, expect=tsg.E_TIMEOUT)
    gP, gout = case.run()
    assert err_ratio(gout, out, s_out) <= 1.0


def test_rs_full_size_parity_and_modes(env):
    torch, tsg, ctx = env
    cfg = CONFIGS["gemm_rs"]
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    inp = rs_inputs(M, K, N, R, rank=0, seed=cfg["seed"])
    P, out, sP, s_out = _ref(inp, R, 0)
    case = RsCase(env, inp, M, N, K, R, 0)
    gP, gout = case.run()
    rP, rout = err_ratio(gP, P, sP), err_ratio(gout, out, s_out)
    print(f"gemm_rs max err/tol partial {rP:.3f} out {rout:.3f}")
    assert rP <= 1.0 and rout <= 1.0
    for mode in (tsg.SERIAL,):
        gP2, gout2 = case.run(mode=mode)
        assert np.array_equal(gP2, gP) and np.array_equal(gout2, gout)
    _, gout3 = case.run(mode=tsg.COMM_ONLY, poison=True)
    assert np.array_equal(gout3, gout)
    for aux in (16, 32):
        gP4, gout4 = case.run(opts={"aux_cus": aux})
        assert np.array_equal(gP4, gP) and np.array_equal(gout4, gout)
    gP5, gout5 = case.run(opts={"order": 1})
    assert np.array_equal(gP5, gP) and np.array_equal(gout5, gout)
    # the eight-wave 16x16x32 tile: another accumulation order, checked
    # against the oracle; overlap and serial give the same bits
    gP6, gout6 = case.run(opts={"tile": 6})
    assert err_ratio(gP6, P, sP) <= 1.0 and err_ratio(gout6, out, s_out) <= 1.0
    gP7, gout7 = case.run(mode=tsg.SERIAL, opts={"tile": 6})
    assert np.array_equal(gP7, gP6) and np.array_equal(gout7, gout6)


def _launch(case, mode=None, opts=None):
    """Poison the outputs and enqueue one call, with no synchronisation."""
    torch, tsg, ctx = case.env
    mode = tsg.OVERLAP if mode is None else mode
    case.out.fill_(float("nan"))
    if mode != tsg.COMM_ONLY:
        case.partial.fill_(float("nan"))
    tsg.gemm_rs_overlap(ctx, case.x, case.w, case.partial, case.peers, case.out, case.M, case.N, case.K,
                        case.R, case.rank, opts=opts, mode=mode)


def test_rs_overlap_joined_through_the_gemm(env):
    # Overlap on shared CUs: the caller's stream waits for the GEMM only,
    # whose last workgroup waits for the reduce's end signal; the reduce
    # stores its final out coherently.  Calls of every launch form follow
    # with no synchronisation in between, and a stream synchronisation alone
    # must show every output whole.
    torch, tsg, ctx = env
    M, N, K, R = 2048, 1024, 512, 8
    inps = [rs_inputs(M, K, N, R, rank=r, seed=60 + r) for r in range(6)]
    refs = [_ref(x, R, r) for r, x in enumerate(inps)]
    cases = [RsCase(env, x, M, N, K, R, r) for r, x in enumerate(inps)]

    def check(j):
        P, out, sP, s_out = refs[j]
        gP = cases[j].partial.cpu().numpy().astype(np.float64)
        gout = cases[j].out.cpu().numpy().astype(np.float64)
        assert err_ratio(gP, P, sP) <= 1.0 and err_ratio(gout, out, s_out) <= 1.0, j
    for i in range(12):                      # back to back on two buffer sets
        _launch(cases[i % 2])
    torch.cuda.current_stream().synchronize()
    check(0)
    check(1)
    _launch(cases[0])                                    # detached
    _launch(cases[1], mode=tsg.SERIAL)                   # GEMM, then the reduce
    _launch(cases[2])                                    # detached
    _launch(cases[3], opts={"aux_cus": 16})              # CU split, joined
    _launch(cases[4], opts={"tile": 6})                  # back to back (no room beside tile 6)
    _launch(cases[5])                                    # detached
    torch.cuda.current_stream().synchronize()
    for j in range(6):
        check(j)
    assert ctx.check() == tsg.OK, ctx.last_error()


def test_rs_overlap_on_the_null_stream(env):
    torch, tsg, ctx = env
    M, N, K, R = 1024, 512, 256, 4
    inp = rs_inputs(M, K, N, R, rank=1, seed=66)
    P, out, sP, s_out = _ref(inp, R, 1)
    with torch.cuda.stream(torch.cuda.default_stream()):
        case = RsCase(env, inp, M, N, K, R, 1)
        gP, gout = case.run()
    assert err_ratio(gP, P, sP) <= 1.0 and err_ratio(gout, out, s_out) <= 1.0


def test_rs_tile6_needs_k_multiple_of_128(env):
    torch, tsg, ctx = env
    M, N, K, R = 512, 256, 192, 4
    inp = rs_inputs(M, K, N, R, rank=0, seed=9)
    case = RsCase(env, inp, M, N, K, R, 0)
    st = tsg.gemm_rs_overlap(ctx, case.x, case.w, case.partial, case.peers, case.out, M, N, K, R, 0, opts={"tile": 6},
                             raise_on_error=False)
    assert st == tsg.E_UNSUPPORTED
