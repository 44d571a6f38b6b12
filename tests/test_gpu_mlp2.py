"""CTA-pipelined two-GEMM MLP on the GPU against the oracle.

H and Y are pre-filled with NaN, so a GEMM2 tile that read its H rows before
the row block's signal completed shows up as a non-finite element.

Bounds: H is bf16(GELU(z)); |GELU'| <= 1.13, so the device's H may differ from
the oracle's by 1.13 * (1e-3 * S1 + 1e-5) before rounding, plus one bf16
quantum from the two roundings (S1 = sum_k |x_ik w1_kj|).  Y is compared with
the GEMM bound on S2 = sum_k |H_ik w2_kj| plus the propagated effect of the
actual H difference, sum_k |H_gpu - H_ref|_ik |w2_kj|."""
import numpy as np
import pytest

import oracle
from _helpers import bf16_from_dev, bf16_half_quantum, to_dev
from synth import CONFIGS, f32_to_bf16_bits, mlp2_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    ctx.close()


def _run(env, inp, M, K1, N1, N2, mode=None, opts=None, expect=0):
    torch, tsg, ctx = env
    mode = tsg.OVERLAP if mode is None else mode
    x, w1, w2 = to_dev(inp["x"], torch), to_dev(inp["w1"], torch), to_dev(inp["w2"], torch)
    h = torch.full((M, N1), 0x7FC0, dtype=torch.int16, device="cuda")
    y = torch.full((M, N2), float("nan"), dtype=torch.float32, device="cuda")
    tsg.mlp2_pipelined(ctx, x, w1, h, w2, y, M, K1, N1, N2, opts=opts, mode=mode)
    st = ctx.check()
    assert st == expect, (st, ctx.last_error())
    return bf16_from_dev(h), y.cpu().numpy().astype(np.float64)


def _ref(inp):
    z, h_ref, y_ref = oracle.mlp2(inp["x"], inp["w1"], inp["w2"])
    return h_ref, y_ref, oracle.gemm_abs(inp["x"], inp["w1"])


def _check(inp, h_gpu, y_gpu, ref=None):
    h_ref, y_ref, s1 = ref if ref is not None else _ref(inp)
    hg, hr = oracle.bf16_to_f64(h_gpu), oracle.bf16_to_f64(h_ref)
    tol_h = 1.13 * (1e-3 * s1 + 1e-5) + 2 * bf16_half_quantum(hr) + 1e-7
    assert np.all(np.isfinite(hg))
    rh = float(np.max(np.abs(hg - hr) / tol_h))
    w2 = np.abs(oracle.bf16_to_f64(inp["w2"]))
    s2 = np.abs(hr) @ w2
    prop = np.abs(hg - hr) @ w2
    ry = float(np.max(np.abs(y_gpu - y_ref) / (1e-3 * s2 + 1e-5 + prop)))
    assert np.all(np.isfinite(y_gpu))
    return rh, ry


@pytest.mark.parametrize("tile", [3, 5, 1, 6, 7])
def test_mlp2_small_ragged(env, tile):
    M, K1, N1, N2 = 300, 256, 384, 200
    inp = mlp2_inputs(M, K1, N1, N2, seed=11)
    h, y = _run(env, inp, M, K1, N1, N2, opts={"tile": tile})
    rh, ry = _check(inp, h, y)
    assert rh <= 1.0 and ry <= 1.0, (rh, ry)


def test_mlp2_k_not_multiple_of_128(env):
    M, K1, N1, N2 = 256, 200, 136, 264
    inp = mlp2_inputs(M, K1, N1, N2, seed=12)
    h, y = _run(env, inp, M, K1, N1, N2)
    rh, ry = _check(inp, h, y)
    assert rh <= 1.0 and ry <= 1.0, (rh, ry)


def test_mlp2_eight_wave_tiles_need_k_multiple_of_128(env):
    torch, tsg, ctx = env
    M, K1, N1, N2 = 256, 200, 256, 256
    inp = mlp2_inputs(M, K1, N1, N2, seed=16)
    x, w1, w2 = to_dev(inp["x"], torch), to_dev(inp["w1"], torch), to_dev(inp["w2"], torch)
    h = torch.empty((M, N1), dtype=torch.int16, device="cuda")
    y = torch.empty((M, N2), dtype=torch.float32, device="cuda")
    for tile in (6, 7):
        st = tsg.mlp2_pipelined(ctx, x, w1, h, w2, y, M, K1, N1, N2, opts={"tile": tile}, raise_on_error=False)
        assert st == tsg.E_UNSUPPORTED


def test_mlp2_large_k_not_multiple_of_128_default(env):
    # at this size the default takes the 32x32x16 tiles, because K1 % 128 != 0
    M, K1, N1, N2 = 1024, 1000, 1024, 1024
    inp = mlp2_inputs(M, K1, N1, N2, seed=17)
    h, y = _run(env, inp, M, K1, N1, N2)
    rh, ry = _check(inp, h, y)
    assert rh <= 1.0 and ry <= 1.0, (rh, ry)


def test_mlp2_identity_w1_is_elementwise_gelu(env):
    M, K = 256, 256
    inp = mlp2_inputs(M, K, K, 128, seed=13)
    inp["w1"] = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    h, y = _run(env, inp, M, K, K, 128)
    g = oracle.gelu_erf(oracle.bf16_to_f64(inp["x"]))
    hg = oracle.bf16_to_f64(h)
    # fp32 erf vs exact: the bf16 results agree within one quantum
    assert np.all(np.abs(hg - g) <= 2 * bf16_half_quantum(g) + 1e-30)


def test_mlp2_missing_row_block_times_out_then_recovers(env):
    torch, tsg, ctx = env
    M, K1, N1, N2 = 512, 128, 256, 256
    inp = mlp2_inputs(M, K1, N1, N2, seed=14)
    _run(env, inp, M, K1, N1, N2, opts={"debug_skip_mask": 1 << 2, "timeout_ms": 20}, expect=tsg.E_TIMEOUT)
    h, y = _run(env, inp, M, K1, N1, N2)
    rh, ry = _check(inp, h, y)
    assert rh <= 1.0 and ry <= 1.0


def test_mlp2_comm_only_unsupported(env):
    torch, tsg, ctx = env
    inp = mlp2_inputs(128, 64, 64, 64, seed=15)
    x = to_dev(inp["x"], torch)
    assert tsg.mlp2_pipelined(ctx, x, x, x, x, x, 128, 64, 64, 64, mode=tsg.COMM_ONLY,
                              raise_on_error=False) == tsg.E_UNSUPPORTED


def test_mlp2_full_size_parity_modes_splits(env):
    torch, tsg, ctx = env
    cfg = CONFIGS["mlp2"]
    M, K1, N1, N2 = cfg["M"], cfg["K1"], cfg["N1"], cfg["N2"]
    inp = mlp2_inputs(M, K1, N1, N2, seed=cfg["seed"])
    ref = _ref(inp)
    h, y = _run(env, inp, M, K1, N1, N2)
    rh, ry = _check(inp, h, y, ref)
    print(f"mlp2 max err/tol H {rh:.3f} Y {ry:.3f}")
    assert rh <= 1.0 and ry <= 1.0
    # the 32x32x16 pair (another accumulation order) against the oracle too
    h5, y5 = _run(env, inp, M, K1, N1, N2, opts={"tile": 5})
    rh5, ry5 = _check(inp, h5, y5, ref)
    assert rh5 <= 1.0 and ry5 <= 1.0, (rh5, ry5)
    for mode in (tsg.SERIAL, tsg.COMPUTE_ONLY):
        h2, y2 = _run(env, inp, M, K1, N1, N2, mode=mode)
        assert np.array_equal(h2, h) and np.array_equal(y2, y)
    for opts in ({"aux_cus": 64, "main_cus": 192}, {"aux_cus": 128}, {"aux_cus": -1}):
        h3, y3 = _run(env, inp, M, K1, N1, N2, opts=opts)
        assert np.array_equal(h3, h) and np.array_equal(y3, y), opts
