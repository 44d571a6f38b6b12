"""moe_expert_combine_noalloc: the MoE path with its workspace in the
library's static per-GPU buffer instead of a caller-allocated one.  Its
results must equal those of moe_expert_combine on the same inputs bit for bit
(same kernels, same order), on two calls in a row, the second with a smaller
input, in overlap, serial and combine-only mode; dims beyond the buffer and
options that would need a stream or a memset are refused before anything is
queued.  Placed last in collection order: a failure here hides no other test."""
import numpy as np
import pytest

from _helpers import to_dev
from synth import moe_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    ctx.close()


def _dev(torch, inp):
    T, H = inp["x"].shape
    E = inp["w_up"].shape[0]
    k = inp["topk_ids"].shape[1]
    d = {n: to_dev(inp[n], torch) for n in ("x", "topk_ids", "topk_w", "w_up", "w_down")}
    d["out"] = torch.empty((T, H), dtype=torch.float32, device="cuda")
    d["counts"] = torch.empty((E,), dtype=torch.int32, device="cuda")
    d["sorted"] = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    return d


def _poison(d):
    d["out"].fill_(float("nan"))
    d["counts"].fill_(-7)
    d["sorted"].fill_(-7)


def _with_workspace(env, d, dims, mode, opts=None):
    torch, tsg, ctx = env
    T, H, I, E, k = dims
    wsb = tsg.workspace_bytes(tsg.OP_MOE, list(dims))
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda")
    _poison(d)
    tsg.moe_expert_combine(ctx, d["x"], d["topk_ids"], d["topk_w"], d["w_up"], d["w_down"], d["out"], d["counts"],
                           d["sorted"], ws, wsb, T, H, I, E, k, opts=opts, mode=mode)
    assert ctx.check() == tsg.OK, ctx.last_error()
    return d["out"].cpu().numpy(), d["counts"].cpu().numpy(), d["sorted"].cpu().numpy()


def _noalloc(env, d, dims, mode, opts=None, poison=True):
    torch, tsg, ctx = env
    T, H, I, E, k = dims
    if poison:
        _poison(d)
    tsg.moe_expert_combine_noalloc(ctx, d["x"], d["topk_ids"], d["topk_w"], d["w_up"], d["w_down"], d["out"],
                                   d["counts"], d["sorted"], T, H, I, E, k, opts=opts, mode=mode)
    assert ctx.check() == tsg.OK, ctx.last_error()
    return d["out"].cpu().numpy(), d["counts"].cpu().numpy(), d["sorted"].cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls(env):
    torch, tsg, ctx = env
    # first call: the full hidden and expert sizes at 512 tokens (about 60 MB
    # of workspace, near the 64 MiB buffer); second: a smaller, ragged input
    cases = [((512, 4096, 1408, 8, 2), dict(seed=51, zipf=1.2)), ((300, 1024, 520, 5, 2), dict(seed=52))]
    for dims, kw in cases:
        T, H, I, E, k = dims
        assert tsg.workspace_bytes(tsg.OP_MOE, list(dims)) <= tsg.MOE_NOALLOC_BYTES
        inp = moe_inputs(T, H, I, E, k=k, **kw)
        d = _dev(torch, inp)
        for mode, opts in ((tsg.OVERLAP, None), (tsg.SERIAL, None), (tsg.OVERLAP, {"stage_dtype": tsg.BF16})):
            ref = _with_workspace(env, d, dims, mode, opts)
            got = _noalloc(env, d, dims, mode, opts)
            assert np.all(np.isfinite(got[0])), (dims, mode)
            for a, b in zip(got, ref):
                assert np.array_equal(a, b), (dims, mode, opts)
        # the combine alone over the staging the last no-alloc call left
        d["out"].fill_(float("nan"))
        _noalloc(env, d, dims, tsg.SERIAL, poison=False)
        full = d["out"].cpu().numpy()
        d["out"].fill_(float("nan"))
        got = _noalloc(env, d, dims, tsg.COMM_ONLY, poison=False)
        assert np.array_equal(got[0], full), dims


def test_noalloc_refusals(env):
    torch, tsg, ctx = env
    inp = moe_inputs(64, 256, 128, 4, k=2, seed=53)
    d = _dev(torch, inp)
    args = (ctx, d["x"], d["topk_ids"], d["topk_w"], d["w_up"], d["w_down"], d["out"], d["counts"], d["sorted"])
    # the full 4096-token workload needs about 200 MB: beyond the buffer
    assert tsg.workspace_bytes(tsg.OP_MOE, [4096, 4096, 1408, 8, 2]) > tsg.MOE_NOALLOC_BYTES
    assert tsg.moe_expert_combine_noalloc(*args, 4096, 4096, 1408, 8, 2, raise_on_error=False) == tsg.E_WORKSPACE
    assert "static buffer" in ctx.last_error()
    for opts in ({"aux_cus": 16}, {"timeline": 1}):
        assert tsg.moe_expert_combine_noalloc(*args, 64, 256, 128, 4, 2, opts=opts,
                                              raise_on_error=False) == tsg.E_UNSUPPORTED, opts
    assert tsg.moe_expert_combine_noalloc(*args, 64, 256, 128, 4, 3, raise_on_error=False) == tsg.E_UNSUPPORTED
    # the context is still usable
    out = _noalloc(env, d, (64, 256, 128, 4, 2), tsg.OVERLAP)
    assert np.all(np.isfinite(out[0]))
