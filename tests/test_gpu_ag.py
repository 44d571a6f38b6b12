"""AllGather + GEMM on the GPU against the oracle.

Every call runs with the gathered buffer and the output pre-filled with NaN
patterns, so a tile that read its rows before acquiring their chunk signal, or
a tile that was never written, shows up as a non-finite element."""
import numpy as np
import pytest

import oracle
from _helpers import bf16_from_dev, err_ratio, to_dev
from synth import CONFIGS, ag_inputs
from synth.gen import split_chunks

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def env():
    import torch
    import tile_level_communication_signaled_amd as tsg
    ctx = tsg.Context(0)
    # a dedicated stream, as the benchmark uses: on the null stream the GEMM
    # runs on a side stream too and every call joins
    torch.cuda.set_stream(torch.cuda.Stream())
    yield torch, tsg, ctx
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.default_stream())
    ctx.close()


class AgCase:
    def __init__(self, env, inp, M, N, K, R, rank, out_bf16):
        torch, tsg, ctx = env
        self.env, self.M, self.N, self.K, self.R, self.rank, self.out_bf16 = env, M, N, K, R, rank, out_bf16
        loc, peers = split_chunks(inp["a"], R, rank)
        self.loc = to_dev(loc, torch)
        self.peers = to_dev(peers if R > 1 else np.zeros((1, 8), np.uint16), torch)
        self.b = to_dev(inp["b"], torch)
        self.full = torch.empty((M, K), dtype=torch.int16, device="cuda")
        self.c = torch.empty((M, N), dtype=torch.int16 if out_bf16 else torch.float32, device="cuda")

    def run(self, mode=None, order=None, opts=None, poison=True, expect=0):
        torch, tsg, ctx = self.env
        mode = tsg.OVERLAP if mode is None else mode
        if poison:
            self.full.fill_(NAN_BF16)
            self.c.fill_(NAN_BF16 if self.out_bf16 else float("nan"))
        tsg.gemm_ag_overlap(ctx, self.loc, self.peers, self.full, self.b, self.c,
                            tsg.BF16 if self.out_bf16 else tsg.F32, self.M, self.N, self.K, self.R,
                            self.rank, arrival_order=order, opts=opts, mode=mode)
        st = ctx.check()
        assert st == expect, (st, ctx.last_error())
        full = bf16_from_dev(self.full)
        if self.out_bf16:
            c = oracle.bf16_to_f64(bf16_from_dev(self.c))
        else:
            c = self.c.cpu().numpy().astype(np.float64)
        return full, c


def _ref(inp):
    return oracle.gemm(inp["a"], inp["b"]), oracle.gemm_abs(inp["a"], inp["b"])


def test_tiny_ag_all_ranks_tiles_orders(env):
    cfg = CONFIGS["tiny_ag"]
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    inp = ag_inputs(M, K, N, R, seed=cfg["seed"], dist="uniform")
    ref, scale = _ref(inp)
    first = None
    for rank in range(R):
        case = AgCase(env, inp, M, N, K, R, rank, out_bf16=False)
        peers = [r for r in range(R) if r != rank]
        for tile in (6, 7, 3, 1):              # 64x64, 128x64 (spans two chunks), 128x128, 256x256
            for order in (None, peers[::-1]):
                full, c = case.run(order=order, opts={"tile": tile, "aux_cus": 8})
                assert np.array_equal(full, inp["a"])
                assert err_ratio(c, ref, scale) <= 1.0
                if first is None:
                    first = c
                assert np.array_equal(c, first), (rank, tile, order)


def test_tiny_ag_integer_inputs_exact(env):
    M, N, K, R = 256, 128, 256, 4
    rng = np.random.default_rng(5)
    from synth import f32_to_bf16_bits
    inp = {"a": f32_to_bf16_bits(rng.integers(-2, 3, (M, K)).astype(np.float32)),
           "b": f32_to_bf16_bits(rng.integers(-2, 3, (K, N)).astype(np.float32))}
    case = AgCase(env, inp, M, N, K, R, 1, out_bf16=False)
    _, c = case.run(opts={"aux_cus": 8})
    assert np.array_equal(c, oracle.gemm(inp["a"], inp["b"]))


@pytest.mark.parametrize("tile", [6, 3, 1, 2])
def test_ag_ragged_shapes(env, tile):
    # 3 ranks of 200 rows: tiles straddle chunks; N and K are not multiples of
    # the tile; K is not a multiple of 64 (communication slabs of 64 columns:
    # 64, 64 and a last slab of 8)
    M, N, K, R = 600, 200, 136, 3
    inp = ag_inputs(M, K, N, R, seed=7)
    ref, scale = _ref(inp)
    for rank in range(R):
        for out_bf16 in (False, True):
            case = AgCase(env, inp, M, N, K, R, rank, out_bf16)
            for ct in (0, 64):
                full, c = case.run(opts={"tile": tile, "aux_cus": 16, "comm_tile": ct})
                assert np.array_equal(full, inp["a"])
                assert err_ratio(c, ref, scale, bf16_out=out_bf16) <= 1.0


@pytest.mark.parametrize("tile", [8, 2, 1, 9])
def test_ag_direct_path_ragged(env, tile):
    # K a multiple of 128 (operands go straight to LDS); M and N ragged against
    # the 256-row tiles and 224- or 256-column tiles; 3 ranks of 200 rows, so
    # tiles straddle chunks; shared CUs (the GEMM pulls copy units) and a CU
    # split; slabs of 128 columns
    M, N, K, R = 600, 232, 384, 3
    inp = ag_inputs(M, K, N, R, seed=8)
    ref, scale = _ref(inp)
    for rank in range(R):
        for out_bf16 in (True, False):
            case = AgCase(env, inp, M, N, K, R, rank, out_bf16)
            for aux in (-1, 16):
                full, c = case.run(opts={"tile": tile, "aux_cus": aux, "comm_tile": 128})
                assert np.array_equal(full, inp["a"])
                assert err_ratio(c, ref, scale, bf16_out=out_bf16) <= 1.0


def test_ag_tile9_needs_k_multiple_of_128(env):
    # 16x16x32-fragment tiles load operands straight to LDS only
    torch, tsg, ctx = env
    M, N, K, R = 512, 224, 392, 2
    inp = ag_inputs(M, K, N, R, seed=10)
    case = AgCase(env, inp, M, N, K, R, 0, True)
    st = tsg.gemm_ag_overlap(ctx, case.loc, case.peers, case.full, case.b, case.c, tsg.BF16, M, N, K, R, 0,
                             opts={"tile": 9}, raise_on_error=False)
    assert st == tsg.E_UNSUPPORTED
    full, c = case.run(opts={"tile": 8})
    ref, scale = _ref(inp)
    assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale, bf16_out=True) <= 1.0


def test_ag_copy_engine(env):
    # the gathered data moved by the DMA copy engines, one stream per chunk,
    # each channel followed by an 8-byte copy of its signal: bit-identical
    # results in overlap (shared CUs and a CU split), serial and comm-only
    # mode, for one and two channels per rank, every rank
    torch, tsg, ctx = env
    M, N, K, R = 600, 232, 384, 3
    inp = ag_inputs(M, K, N, R, seed=11)
    ref, scale = _ref(inp)
    first = None
    for rank in range(R):
        case = AgCase(env, inp, M, N, K, R, rank, True)
        for mode, aux in ((tsg.OVERLAP, -1), (tsg.OVERLAP, 16), (tsg.SERIAL, -1), (tsg.COMM_ONLY, -1)):
            for ch in (1, 2):
                full, c = case.run(mode=mode, opts={"copy_engine": 1, "aux_cus": aux, "channels": ch})
                assert np.array_equal(full, inp["a"]), (rank, mode, aux, ch)
                if mode != tsg.COMM_ONLY:
                    assert err_ratio(c, ref, scale, bf16_out=True) <= 1.0, (rank, mode, aux, ch)
                    first = c if first is None else first
                    assert np.array_equal(c, first), (rank, mode, aux, ch)
    for bad, want in (({"copy_engine": 1, "arrival_gbps": 2}, tsg.E_INVALID), ({"copy_engine": 2}, tsg.E_INVALID)):
        st = tsg.gemm_ag_overlap(ctx, case.loc, case.peers, case.full, case.b, case.c, tsg.BF16, M, N, K, R, 0,
                                 opts=bad, raise_on_error=False)
        assert st == want, bad


@pytest.mark.parametrize("tile", [3, 1, 6])
def test_ag_channels_bit_exact(env, tile):
    # C channels per rank ([TL] section 4.1): 200-row chunks cut into 2, 4
    # and 8 channels (100, 50, 25 rows), so 128- and 256-row tiles span
    # several channels whose edges fall inside tiles; every rank, overlap and
    # serial, CU copy and copy engines: the same bits as one channel
    torch, tsg, ctx = env
    M, N, K, R = 600, 256, 256, 3
    inp = ag_inputs(M, K, N, R, seed=21)
    ref, scale = _ref(inp)
    for rank in range(R):
        case = AgCase(env, inp, M, N, K, R, rank, False)
        _, base = case.run(opts={"tile": tile})
        assert err_ratio(base, ref, scale) <= 1.0
        for C in (2, 4, 8):
            for mode in (tsg.OVERLAP, tsg.SERIAL):
                for ce in (0, 1):
                    opts = {"tile": tile, "channels": C, "copy_engine": ce, "comm_tile": 0 if ce else 64}
                    full, c = case.run(mode=mode, opts=opts)
                    assert np.array_equal(full, inp["a"]), (rank, C, mode, ce)
                    assert np.array_equal(c, base), (rank, C, mode, ce)


def test_ag_channels_rejected(env):
    torch, tsg, ctx = env
    M, N, K, R = 600, 64, 128, 3
    case = AgCase(env, ag_inputs(M, K, N, R, seed=22), M, N, K, R, 0, False)
    for C, want in ((3, tsg.E_INVALID), (65, tsg.E_INVALID), (-1, tsg.E_INVALID), (40, tsg.E_SHAPE)):
        st = tsg.gemm_ag_overlap(ctx, case.loc, case.peers, case.full, case.b, case.c, tsg.F32, M, N, K, R, 0,
                                 opts={"channels": C}, raise_on_error=False)
        assert st == want, C


@pytest.mark.parametrize("copy_engine", [0, 1])
def test_ag_channel_mapping_matches_static_map(env, copy_engine):
    # The signals a GEMM tile waits for are those of the channels its rows
    # belong to under TileLink's static mapping (oracle.static_map_ag, pinned
    # by tests/golden/static_mapping.txt).  For each global channel g the
    # signal of g alone is withheld (20 ms bound); the device timeline then
    # shows which tiles waited out the bound: exactly the non-local tiles
    # whose rows map to channel g.  M 384, R 4, C 2: 48-row channels, 64-row
    # tiles that straddle channel and chunk edges.
    torch, tsg, ctx = env
    M, N, K, R, C, rank = 384, 64, 128, 4, 2, 1
    inp = ag_inputs(M, K, N, R, seed=23)
    case = AgCase(env, inp, M, N, K, R, rank, False)
    BM = 64
    n_mt = M // BM
    spans = []
    for mt in range(n_mt):
        rows = range(mt * BM, (mt + 1) * BM)
        maps = [oracle.static_map_ag(r, 1, M, R, C) for r in rows]
        local = all(m[2] == rank for m in maps)
        spans.append(set() if local else {m[3] for m in maps})
    # one plain call first: the first copy-engine call after the set of copy
    # streams has grown can take milliseconds longer (runtime engine set-up)
    case.run(opts={"channels": C, "tile": 6, "copy_engine": copy_engine})
    for g in range(R * C):
        want = {mt for mt in range(n_mt) if g in spans[mt]}
        opts = {"channels": C, "tile": 6, "copy_engine": copy_engine, "debug_skip_mask": 1 << g,
                "timeout_ms": 20, "timeline": 1, "comm_tile": 0 if copy_engine else 128}
        case.run(opts=opts, expect=tsg.E_TIMEOUT if want else tsg.OK)
        recs = [r for r in ctx.timeline() if (r[0] >> 56) == 2]
        assert len(recs) == n_mt
        waited = {(r[0] & 0xFFFFFFFF) >> 16 for r in recs if r[2] - r[1] > 1_000_000}   # > 10 ms at 100 MHz
        assert waited == want, (g, waited, want)
    full, c = case.run(opts={"channels": C, "tile": 6, "copy_engine": copy_engine})
    ref, scale = _ref(inp)
    assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0


def test_ag_paced_arrival(env):
    # arrival paced at 2 GB/s: the same results, and a call takes at least
    # the gathered bytes over the rate (in every mode that copies)
    import time
    torch, tsg, ctx = env
    M, N, K, R = 600, 232, 384, 3
    inp = ag_inputs(M, K, N, R, seed=9)
    ref, scale = _ref(inp)
    case = AgCase(env, inp, M, N, K, R, 1, True)
    gbps = 2
    floor_s = M * K * 2 / (gbps * 1e9)
    for mode in (tsg.OVERLAP, tsg.SERIAL, tsg.COMM_ONLY):
        for aux in (-1, 16):
            opts = {"arrival_gbps": gbps, "aux_cus": aux, "comm_tile": 128}
            case.run(mode=mode, opts=opts)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            full, c = case.run(mode=mode, opts=opts)
            elapsed = time.perf_counter() - t0
            assert np.array_equal(full, inp["a"])
            if mode != tsg.COMM_ONLY:
                assert err_ratio(c, ref, scale, bf16_out=True) <= 1.0
            assert elapsed >= 0.9 * floor_s, (mode, aux, elapsed, floor_s)
    st = tsg.gemm_ag_overlap(ctx, case.loc, case.peers, case.full, case.b, case.c, tsg.BF16, M, N, K, R, 1,
                             opts={"arrival_gbps": -1}, raise_on_error=False)
    assert st == tsg.E_INVALID


@pytest.mark.parametrize("K", [512, 320])
def test_ag_comm_tile_slabs(env, K):
    # Chunks move as column slabs; tiles wait slab by slab inside the K loop.
    # K = 512 runs the direct-to-LDS main loop, K = 320 the register path with
    # a partial last slab (128, 128, 64).  Few copy workgroups so that tiles
    # really do wait on later slabs.  Every combination gives the same bits.
    M, N, R = 512, 256, 4
    inp = ag_inputs(M, K, N, R, seed=11)
    ref, scale = _ref(inp)
    first = None
    for rank in (0, 3):
        case = AgCase(env, inp, M, N, K, R, rank, out_bf16=False)
        for tile in (6, 3, 1):                 # 256-row tiles span two 128-row chunks
            for ct in (64, 128, 1024):
                for wgs in (3, 64):
                    full, c = case.run(opts={"tile": tile, "aux_cus": -1, "comm_tile": ct, "aux_wgs": wgs})
                    assert np.array_equal(full, inp["a"]), (rank, tile, ct, wgs)
                    assert err_ratio(c, ref, scale) <= 1.0
                    if first is None:
                        first = c
                    assert np.array_equal(c, first), (rank, tile, ct, wgs)


def test_ag_comm_tile_ragged_rows_and_unaligned_buffer(env):
    # 3 chunks of 200 rows, K a multiple of 64: the last 128-row tile has rows
    # beyond M (read as a stand-in row of the tile); then the same with the
    # gathered buffer 16 bytes off a 128-byte boundary, where slabs share
    # cache lines and the waits take the general acquire.
    torch, tsg, ctx = env
    M, N, K, R = 600, 192, 512, 3
    inp = ag_inputs(M, K, N, R, seed=13)
    ref, scale = _ref(inp)
    case = AgCase(env, inp, M, N, K, R, 2, out_bf16=False)
    for tile in (3, 6):
        full, c = case.run(opts={"tile": tile, "comm_tile": 64, "aux_wgs": 4})
        assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0
    store = torch.empty((M * K + 64,), dtype=torch.int16, device="cuda")
    case.full = store[8:8 + M * K].view(M, K)
    assert case.full.data_ptr() % 128 == 16
    for tile in (3, 6):
        full, c = case.run(opts={"tile": tile, "comm_tile": 64, "aux_wgs": 4})
        assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0


def test_ag_pull_units_variants(env):
    # The GEMM's first workgroups may pull any number of the copy's units from
    # the shared work queue (none, the default, a few, more than there are):
    # every variant gathers the same buffer and computes the same bits, and
    # calls alternating between variants keep the queue's reset consistent.
    M, N, K, R = 1024, 512, 512, 4
    inp = ag_inputs(M, K, N, R, seed=21)
    ref, scale = _ref(inp)
    first = None
    for rank, tile in ((1, 3), (2, 1)):
        case = AgCase(env, inp, M, N, K, R, rank, out_bf16=False)
        for pull in (-1, 0, 1, 5, 100000):
            for ct, wgs in ((64, 4), (256, 0)):
                full, c = case.run(opts={"tile": tile, "aux_cus": -1, "pull_units": pull, "comm_tile": ct,
                                         "aux_wgs": wgs})
                assert np.array_equal(full, inp["a"]), (rank, tile, pull, ct)
                assert err_ratio(c, ref, scale) <= 1.0
                if first is None:
                    first = c
                assert np.array_equal(c, first), (rank, tile, pull, ct)


def test_ag_comm_only_and_serial_fill_gathered_buffer(env):
    torch, tsg, ctx = env
    M, N, K, R = 512, 128, 256, 8
    inp = ag_inputs(M, K, N, R, seed=12)
    ref, scale = _ref(inp)
    case = AgCase(env, inp, M, N, K, R, 6, out_bf16=False)
    full, _ = case.run(mode=tsg.COMM_ONLY, opts={"comm_tile": 64})
    assert np.array_equal(full, inp["a"])
    full, c = case.run(mode=tsg.SERIAL, opts={"comm_tile": 64, "aux_wgs": 5})
    assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0


def _launch(case, mode=None, opts=None):
    """Poison the outputs and enqueue one call, with no synchronisation."""
    torch, tsg, ctx = case.env
    case.full.fill_(NAN_BF16)
    case.c.fill_(NAN_BF16 if case.out_bf16 else float("nan"))
    tsg.gemm_ag_overlap(ctx, case.loc, case.peers, case.full, case.b, case.c,
                        tsg.BF16 if case.out_bf16 else tsg.F32, case.M, case.N, case.K, case.R, case.rank,
                        opts=opts, mode=tsg.OVERLAP if mode is None else mode)


def _result(case):
    full = bf16_from_dev(case.full)
    c = oracle.bf16_to_f64(bf16_from_dev(case.c)) if case.out_bf16 else case.c.cpu().numpy().astype(np.float64)
    return full, c


def test_ag_overlap_joined_through_the_gemm(env):
    # Overlap on shared CUs: the caller's stream waits for the GEMM only, and
    # the copy kernel's workgroups may still be leaving their work queue when
    # the next call starts.  Calls of every other launch form follow with no
    # synchronisation in between; each must find its queue words at zero and
    # leave every output whole, and a stream synchronisation alone must show
    # the whole gathered buffer (the local chunk included).
    torch, tsg, ctx = env
    M, N, K, R = 2048, 448, 1024, 8          # a 4 MiB copy: a copy kernel runs beside the GEMM
    inps = [ag_inputs(M, K, N, R, seed=40 + i) for i in range(6)]
    refs = [_ref(x) for x in inps]
    cases = [AgCase(env, x, M, N, K, R, 0, out_bf16=True) for x in inps]
    tcfg = CONFIGS["tiny_ag"]
    tinp = ag_inputs(tcfg["M"], tcfg["K"], tcfg["N"], tcfg["R"], seed=46, dist="uniform")
    tiny = AgCase(env, tinp, tcfg["M"], tcfg["N"], tcfg["K"], tcfg["R"], 0, out_bf16=False)
    for i in range(12):                      # back to back on two buffer sets
        _launch(cases[i % 2])
    torch.cuda.current_stream().synchronize()
    for j in range(2):
        full, c = _result(cases[j])
        assert np.array_equal(full, inps[j]["a"]) and err_ratio(c, *refs[j]) <= 1.0, j
    _launch(cases[0])                                     # detached
    _launch(cases[1], mode=tsg.COMM_ONLY)                 # copy on the caller's stream
    _launch(cases[2])                                     # detached
    _launch(cases[3], mode=tsg.SERIAL)                    # copy, then GEMM
    _launch(cases[4], opts={"aux_cus": 16})               # CU split, joined
    _launch(tiny)                                         # the GEMM moves the whole copy
    _launch(cases[5])                                     # detached
    torch.cuda.current_stream().synchronize()
    for j in (0, 1, 2, 3, 4, 5):
        full, c = _result(cases[j])
        assert np.array_equal(full, inps[j]["a"]), j
        if j != 1:
            assert err_ratio(c, *refs[j]) <= 1.0, j
    full, c = _result(tiny)
    assert np.array_equal(full, tinp["a"]) and err_ratio(c, *_ref(tinp)) <= 1.0
    assert ctx.check() == tsg.OK, ctx.last_error()
    # the same after the copy queue has been used by all of them
    full, c = cases[0].run()
    assert np.array_equal(full, inps[0]["a"]) and err_ratio(c, *refs[0]) <= 1.0


def test_ag_overlap_on_the_null_stream(env):
    # from the null stream the GEMM runs on a side stream too, and the call
    # joins both back
    torch, tsg, ctx = env
    M, N, K, R = 2048, 448, 1024, 8
    inp = ag_inputs(M, K, N, R, seed=47)
    with torch.cuda.stream(torch.cuda.default_stream()):
        case = AgCase(env, inp, M, N, K, R, 3, out_bf16=False)
        full, c = case.run()
    assert np.array_equal(full, inp["a"]) and err_ratio(c, *_ref(inp)) <= 1.0


def test_ag_rejects_bad_comm_tile(env):
    torch, tsg, ctx = env
    inp = ag_inputs(64, 64, 64, 4, seed=9)
    case = AgCase(env, inp, 64, 64, 64, 4, 0, out_bf16=False)
    for ct in (32, 96, -64):
        st = tsg.gemm_ag_overlap(ctx, case.loc, case.peers, case.full, case.b, case.c, tsg.F32, 64, 64, 64, 4, 0,
                                 opts={"comm_tile": ct}, raise_on_error=False)
        assert st == tsg.E_INVALID, ct


def test_ag_degenerate_single_rank_and_small(env):
    torch, tsg, ctx = env
    M, N, K, R = 8, 8, 8, 1
    inp = ag_inputs(M, K, N, R, seed=8)
    ref, scale = _ref(inp)
    case = AgCase(env, inp, M, N, K, R, 0, out_bf16=False)
    for mode in (tsg.OVERLAP, tsg.SERIAL):
        full, c = case.run(mode=mode, opts={"aux_cus": 8})
        assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0


def test_ag_rejects_bad_arguments(env):
    torch, tsg, ctx = env
    inp = ag_inputs(64, 64, 64, 4, seed=9)
    case = AgCase(env, inp, 64, 64, 64, 4, 0, out_bf16=False)
    args = (ctx, case.loc, case.peers, case.full, case.b, case.c, tsg.F32)
    assert tsg.gemm_ag_overlap(*args, 64, 64, 60, 4, 0, raise_on_error=False) == tsg.E_SHAPE
    assert tsg.gemm_ag_overlap(*args, 66, 64, 64, 4, 0, raise_on_error=False) == tsg.E_SHAPE
    assert tsg.gemm_ag_overlap(*args, 64, 64, 64, 4, 4, raise_on_error=False) == tsg.E_SHAPE
    assert tsg.gemm_ag_overlap(*args, 64, 64, 64, 4, 0, arrival_order=[1, 1, 2],
                               raise_on_error=False) == tsg.E_INVALID
    assert tsg.gemm_ag_overlap(ctx, case.loc.data_ptr() + 2, case.peers, case.full, case.b, case.c, tsg.F32,
                               64, 64, 64, 4, 0, raise_on_error=False) == tsg.E_ALIGN


def test_ag_missing_chunk_times_out_then_recovers(env):
    torch, tsg, ctx = env
    M, N, K, R = 512, 256, 128, 4
    inp = ag_inputs(M, K, N, R, seed=10)
    ref, scale = _ref(inp)
    case = AgCase(env, inp, M, N, K, R, 0, out_bf16=False)
    case.run(opts={"aux_cus": 8, "debug_skip_mask": 1 << 2, "timeout_ms": 20}, expect=tsg.E_TIMEOUT)
    full, c = case.run(opts={"aux_cus": 8})
    assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0
    # the same with two slabs per chunk: the waits inside the K loop time out too
    case.run(opts={"aux_cus": 8, "debug_skip_mask": 1 << 1, "timeout_ms": 20, "comm_tile": 64},
             expect=tsg.E_TIMEOUT)
    full, c = case.run(opts={"aux_cus": 8, "comm_tile": 64})
    assert np.array_equal(full, inp["a"]) and err_ratio(c, ref, scale) <= 1.0


def test_ag_llama_shape_full_parity(env):
    torch, tsg, ctx = env
    cfg = CONFIGS["llama_ag"]
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    inp = ag_inputs(M, K, N, R, seed=cfg["seed"])
    ref, scale = _ref(inp)
    case = AgCase(env, inp, M, N, K, R, 0, out_bf16=True)
    full, c = case.run()
    assert np.array_equal(full, inp["a"])
    r = err_ratio(c, ref, scale, bf16_out=True)
    print(f"llama_ag max err/tol = {r:.3f}")
    assert r <= 1.0
    _, c_serial = case.run(mode=tsg.SERIAL)
    assert np.array_equal(c_serial, c)
    _, c_comp = case.run(mode=tsg.COMPUTE_ONLY, poison=False)
    assert np.array_equal(c_comp, c)
    # another rank, another arrival order: same product, bit for bit
    inp5 = dict(inp)
    case5 = AgCase(env, inp5, M, N, K, R, 5, out_bf16=True)
    full5, c5 = case5.run(order=[2, 7, 0, 4, 1, 6, 3])
    assert np.array_equal(full5, inp["a"]) and np.array_equal(c5, c)


@pytest.mark.parametrize("aux", [16, 32, 64, -1])
def test_ag_llama_shape_cu_splits(env, aux):
    torch, tsg, ctx = env
    cfg = CONFIGS["llama_ag"]
    M, N, K, R = cfg["M"], cfg["N"], cfg["K"], cfg["R"]
    inp = ag_inputs(M, K, N, R, seed=cfg["seed"])
    case = AgCase(env, inp, M, N, K, R, 3, out_bf16=True)
    full, c = case.run(opts={"aux_cus": aux})
    _, c_serial = case.run(mode=tsg.SERIAL)
    assert np.array_equal(full, inp["a"]) and np.array_equal(c, c_serial)
