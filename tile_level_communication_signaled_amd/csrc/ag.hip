// AllGather + GEMM at one rank's share.
//
// Producer: a copy kernel standing in for the peers' arrival.  It moves the
// peers' shards into the gathered buffer in arrival order, then the local
// shard (GEMM tiles inside the local chunk read it in place and never wait),
// and signals what it has moved ("Triton-distributed: Programming
// Overlapping Kernels on Distributed AI Systems with the Triton Compiler",
// section 3.2, Algorithm 2, pull mode: local copy and signal, then one copy
// and one signal per peer).  The unit of communication is not the whole chunk
// but a column slab of it: chunk c, K columns [s * W, (s + 1) * W).  The
// communication tile is sized independently of the compute tile ("TileLink:
// Generating Efficient Compute-Communication Overlapping Kernels using
// Tile-Centric Primitives", section 3.1, decoupled tile sizes; section 4.1,
// the static mapping from a compute tile to the communication tiles it
// needs).  Slabs are moved slab-major: slab 0 of every chunk in arrival
// order, then slab 1, and so on, each slab in pieces of rows; the last piece
// of a slab to finish publishes its signal (counted arrivals).
//
// Consumer: the MFMA GEMM.  Workgroup w takes the w-th tile of a swizzled
// order that starts at the local chunk and follows the arrival order (the
// Triton-distributed page, section 3.7: the compute tile order follows the
// arrival order of the communication tiles).  It waits (acquire) for slab 0
// of every chunk its rows span, and then, just before it issues the loads of
// the first K step of slab s, for slab s.  The signal of slab s + 1 is read
// as soon as slab s has been passed, so when the copy runs ahead the wait
// costs no round trip.  The signal a row belongs to is the static mapping of
// the TileLink page, section 4.1: each rank's chunk is cut into C channels of
// M / (R C) rows, and row r belongs to channel floor(r / M_per_channel) of
// rank floor(r / M_per_rank).  Each (channel, slab) has its own signal.  The
// copy moves, for each slab, channel 0 of every chunk in arrival order, then
// channel 1, and so on: sub-chunks arrive from all peers at each step (the
// Triton-distributed page, section 3.7, the full-mesh swizzle of Figure 8).
//
// Copy-engine arrival (opts.copy_engine): the signals are set by the DMA
// engines instead of a kernel (the Triton-distributed page, section 3.6: AMD
// intra-node AllGather with copy engines on several streams at once, the
// signal sent as a separate data transfer).  One stream per chunk copies the
// chunk channel by channel, each channel followed by a copy that sets the
// channel's signal: 64 KB, because the runtime runs smaller device copies as
// kernels on the CUs, ending with the call's signal value.
#include "tsg_copy.hpp"
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"

using namespace tsg;

namespace {
constexpr int kMaxMTiles = 1024;
constexpr size_t kSigBase = size_t(1) << 18;  // AG slab signals in the context's pool
constexpr size_t kSigCap = size_t(1) << 18;   // slots up to the next op's region
constexpr int kQueueSlot = 40;                // copy work queue in the context's ticket words: a
                                              // copy the caller's stream does not wait for (on the
                                              // side stream only) uses words 40-41, every other 42-43
constexpr size_t kPaceSlot = 8;               // arrival-pacing start time in the context's pool
constexpr int kMaxChannels = 64;               // channels per rank
constexpr int64_t kPullAllBytes = 1 << 20;     // overlap: copies up to this size run inside the GEMM

// Copy kernel: takes units from the queue in order (slab-major) until none
// is left.  It never waits, so it always drains the queue.
//
// Capped at 32 registers (the attribute counts half the unified register
// file): beside two waves of a 512-thread GEMM tile of up to 240 registers
// each, a copy wave still fits on every SIMD.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(16))) ag_copy_kernel(const CopyArgs a) {
  __shared__ int slot;
  for (int u = claim_unit(a, &slot); u < a.n_units; u = claim_unit(a, &slot)) copy_unit<256>(a, u);
  if (threadIdx.x == 0) leave_queue(a);
}

// Copy-engine arrival: entry i of the signal-value ring holds {base + i | 1},
// the value a channel signal takes in the call whose epoch is base + i.  The
// DMA engines copy the 64 KB window of the ring that ends with the call's
// entry into each channel's signal block, whose last word is its signal.
__global__ void ag_dma_ring_kernel(uint64_t* ring, int n, uint32_t base) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    ring[i] = sig_target(base + (uint32_t)i, 1u);
}

// ---------------------------------------------------------------- GEMM
struct AgGemmArgs {
  const uint16_t* a_full;
  const uint16_t* a_local;  // the local chunk, read in place by tiles inside it
  const uint16_t* b;
  void* c;
  uint64_t* sig;          // slab signals: channel g, slab s at g * sig_stride + s
  int sig_stride;         // words between consecutive channels' signals (n_slab, or a signal block)
  SyncArgs sa;
  Timeline tl;
  int M, N, K;
  int chunk_rows;
  int ch_rows;            // rows per channel: row r waits on channel r / ch_rows
  int rank;
  int n_tiles_n;
  int wait;               // 0: no waits (compute-only)
  uint32_t arrivals;      // arrivals that complete one slab signal
  int n_slab;
  int slab_log2;          // log2 of the slab width in K columns
  int l1_only;            // slabs never share a 128-byte line
  int per_xcd;            // resident tiles per XCD (0 = no XCD remap)
  int pull_wgs;           // workgroups 0 .. pull_wgs - 1 first move one copy unit each
  int pull_all;           // ... or every unit left in the queue (the whole copy; no copy kernel)
  int wait_local_end;     // tiles inside the local chunk wait for its arrival after their stores
  CopyArgs copy;
  uint16_t mt_order[kMaxMTiles];
};

// Slab waits inside the K loop, per wave.  Slabs below `ready_until` are
// known complete and already acquired.  Reaching slab s >= ready_until, the
// wave polls a window of signals in one load: lane l reads channel
// c_lo + l mod n_span at slab s + l / n_span.  The window's complete prefix
// becomes ready; if slab s itself is incomplete the wave polls it until it
// is.  One acquire then covers every slab of the prefix.  As the copy runs
// ahead of the GEMM, a tile polls a few times instead of once per slab.
//
// The general acquire invalidates the wave's L1 and its XCD's L2, which also
// drops the L2's copy of the B panel that all tiles of the XCD share.  When
// no 128-byte line of the gathered buffer holds bytes of two slabs (a
// 128-byte aligned buffer, rows of a multiple of 128 bytes, slabs of at least
// 64 columns) nothing on this XCD can have read a line of slab s before slab
// s was complete: tiles load a slab only after its wait, rows outside the
// operand are read as its last row, and the L2 was invalidated when the tile
// started.  Then invalidating L1 alone is enough.  The flag loads have
// returned before the invalidate (their values decided the branch), so loads
// issued after it see the producer's released data.
struct SlabWait {
  const uint64_t* sig;
  SyncArgs sa;
  uint64_t target;
  uint64_t waited;  // ticks spent polling inside the K loop (timeline only)
  int n_slab, slab_log2, c_lo, n_span;
  int sig_stride;   // words between consecutive channels' signals
  int ready_until;
  bool active;
  bool l1_only;     // slabs are line-aligned: the acquire only invalidates L1

  __device__ __forceinline__ void before_a(int k0) {
    if (!active || (k0 & ((1 << slab_log2) - 1))) return;
    const int s = k0 >> slab_log2;
    if (s < ready_until) return;
    const int lane = __lane_id();
    const int win = 64 / n_span;                 // slabs per window
    const int ls = s + lane / n_span;            // this lane's slab
    const bool valid = lane < win * n_span && ls < n_slab;
    uint64_t v = ~0ull;
    if (valid)
      v = __hip_atomic_load(sig + (size_t)(c_lo + lane % n_span) * sig_stride + ls, __ATOMIC_RELAXED,
                            TSG_SIG_SCOPE);
    const uint64_t bad = __builtin_amdgcn_ballot_w64(v < target);
    if (bad == 0) {
      ready_until = min(s + win, n_slab);
    } else {
      const int f = (int)__builtin_ctzll(bad);   // first incomplete lane, slab-major
      if (f >= n_span) {
        ready_until = s + f / n_span;
      } else {
        const uint64_t t = wall_clock64();
        for (int i = 0; i < n_span; ++i) wave_poll_ge(sig + (size_t)(c_lo + i) * sig_stride + s, target, sa);
        waited += wall_clock64() - t;
        ready_until = s + 1;
      }
    }
    acquire_lines(l1_only);
  }
};

template <class Cfg, bool OUT_BF16, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) ag_gemm_kernel(const AgGemmArgs args) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  const int w = xcd_remap(blockIdx.x, gridDim.x, args.per_xcd);
  const int mt = args.mt_order[w / args.n_tiles_n];
  const int nt = w % args.n_tiles_n;
  const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
  const uint64_t t0 = args.tl.buf ? wall_clock64() : 0;
  if ((int)blockIdx.x < args.pull_wgs) {
    // tile_pull_data: move copy units before any wait.  Workgroup b moves
    // unit b (the first slab's pieces, taken without a ticket: the copy
    // kernel's queue starts after them), or with pull_all every unit left in
    // the queue (the LDS is not in use yet, so its first word carries the
    // ticket).
    if (args.pull_all) {
      for (int u = claim_unit(args.copy, (volatile int*)lds); u < args.copy.n_units;
           u = claim_unit(args.copy, (volatile int*)lds))
        copy_unit<Cfg::NT>(args.copy, u);
      if (threadIdx.x == 0) leave_queue(args.copy);
    } else if ((int)blockIdx.x < args.copy.n_units) {
      if (blockIdx.x == 0 && threadIdx.x == 0) pace_start(args.copy);
      copy_unit<Cfg::NT>(args.copy, (int)blockIdx.x);
    }
  }
  SlabWait hook;
  hook.active = false;
  hook.waited = 0;
  const int last = min(row0 + Cfg::BM, args.M) - 1;
  const int c_lo = row0 / args.chunk_rows, c_hi = last / args.chunk_rows;
  // A tile inside the local chunk reads it where it already is and waits for
  // nothing; every other tile reads the gathered buffer behind the signals
  // of the channels its rows span.
  const bool local = c_lo == args.rank && c_hi == args.rank;
  if (args.wait && !local) {
    const int g_lo = row0 / args.ch_rows, g_hi = last / args.ch_rows;
    hook.sig = args.sig;
    hook.sa = args.sa;
    hook.target = sig_target(args.sa.epoch, args.arrivals);
    hook.n_slab = args.n_slab;
    hook.sig_stride = args.sig_stride;
    hook.slab_log2 = args.slab_log2;
    hook.c_lo = g_lo;
    hook.n_span = g_hi - g_lo + 1;
    hook.active = args.n_slab > 1;
    hook.l1_only = args.l1_only != 0;
    hook.ready_until = 1;
    for (int g = g_lo; g <= g_hi; ++g) block_poll_ge(args.sig + (size_t)g * args.sig_stride, hook.target, args.sa);
    acquire_lines(hook.l1_only);
  }
  const uint64_t t1 = args.tl.buf ? wall_clock64() : 0;
  typename GemmTile<Cfg>::Acc acc;
  const ARowsLinear ar = local ? ARowsLinear{args.a_local, args.K, row0 - args.rank * args.chunk_rows,
                                             args.chunk_rows}
                               : ARowsLinear{args.a_full, args.K, row0, args.M};
  if (DIRECT)
    GemmTile<Cfg>::run_direct(ar, args.b, args.N, col0, args.N, args.K, lds, acc, hook);
  else
    GemmTile<Cfg>::run_regs(ar, args.b, args.N, col0, args.N, args.K, lds, acc, hook);
  const int M = args.M, N = args.N;
  if (OUT_BF16) {
    uint16_t* C = (uint16_t*)args.c;
    GemmTile<Cfg>::template store_bf16_staged<sizeof(lds), false>(
        acc, lds, C + (int64_t)row0 * N + col0, N, M - row0, N - col0, [](float v) { return v; });
  } else {
    float* C = (float*)args.c;
    GemmTile<Cfg>::for_each(acc, [&](int r, int c, float v) {
      const int gr = row0 + r, gc = col0 + c;
      if (gr < M && gc < N) C[(int64_t)gr * N + gc] = v;
    });
  }
  // When the caller's stream does not wait for the copy kernel, the GEMM's
  // end must imply that every chunk has arrived.  The tiles that read a
  // remote channel waited for it; the local chunk, moved last and read in
  // place, is waited for here by the tiles inside it (one load per lane,
  // long complete in practice), so the gathered buffer is whole when the
  // GEMM is.
  if (args.wait_local_end && local && threadIdx.x < 64) {
    const int g_lo = row0 / args.ch_rows;
    const int n = (last / args.ch_rows - g_lo + 1) * args.n_slab;
    const uint64_t target = sig_target(args.sa.epoch, args.arrivals);
    auto at = [&](int i) { return args.sig + (size_t)(g_lo + i / args.n_slab) * args.sig_stride + i % args.n_slab; };
    for (int base = 0; base < n; base += 64) {
      const int i = base + (int)__lane_id();
      const uint64_t v = i < n ? __hip_atomic_load(at(i), __ATOMIC_RELAXED, TSG_SIG_SCOPE) : ~0ull;
      for (uint64_t bad = __builtin_amdgcn_ballot_w64(v < target); bad; bad &= bad - 1)
        wave_poll_ge(at(base + (int)__builtin_ctzll(bad)), target, args.sa);
    }
  }
  if (args.tl.buf && threadIdx.x == 0)
    timeline_put(args.tl, 2, (uint32_t)(mt << 16 | nt), t0, t1 + hook.waited, wall_clock64());
}

// Tile configurations (id -> BM x BN, waves).
using Cfg1 = TileCfg<256, 256, 2, 2>;
using Cfg2 = TileCfg<256, 224, 4, 1>;
using Cfg3 = TileCfg<128, 128, 2, 2>;
using Cfg4 = TileCfg<256, 128, 2, 2>;
using Cfg5 = TileCfg<128, 256, 2, 2>;
using Cfg6 = TileCfg<64, 64, 1, 1>;
using Cfg7 = TileCfg<128, 64, 2, 1>;
using Cfg8 = TileCfg<256, 224, 8, 1>;
using Cfg9 = TileCfg<256, 224, 4, 2, 16>;  // 16x16x32 fragments, waves of 64 x 112

struct TileShape {
  int bm, bn;
};

TileShape shape_of(int id) {
  switch (id) {
    case 1: return {256, 256};
    case 2: return {256, 224};
    case 3: return {128, 128};
    case 4: return {256, 128};
    case 5: return {128, 256};
    case 6: return {64, 64};
    case 7: return {128, 64};
    case 8: return {256, 224};
    case 9: return {256, 224};
    default: return {0, 0};
  }
}

template <class Cfg>
hipError_t launch_gemm_cfg(const AgGemmArgs& a, bool bf16, int grid, hipStream_t s) {
  const bool direct = a.K % (2 * Cfg::BK) == 0;
  if (bf16 && direct)
    hipLaunchKernelGGL((ag_gemm_kernel<Cfg, true, true>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else if (bf16)
    hipLaunchKernelGGL((ag_gemm_kernel<Cfg, true, false>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else if (direct)
    hipLaunchKernelGGL((ag_gemm_kernel<Cfg, false, true>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else
    hipLaunchKernelGGL((ag_gemm_kernel<Cfg, false, false>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  return hipGetLastError();
}

template <class Cfg>
const void* gemm_fn_cfg(bool bf16, bool direct) {
  if (bf16 && direct) return (const void*)&ag_gemm_kernel<Cfg, true, true>;
  if (bf16) return (const void*)&ag_gemm_kernel<Cfg, true, false>;
  if (direct) return (const void*)&ag_gemm_kernel<Cfg, false, true>;
  return (const void*)&ag_gemm_kernel<Cfg, false, false>;
}

// The GEMM kernel a launch uses, and its workgroup size.
const void* gemm_fn(int id, bool bf16, int K, int* nt) {
  switch (id) {
#define TSG_AG_CFG(i, C)                                     \
  case i:                                                    \
    *nt = C::NT;                                             \
    return gemm_fn_cfg<C>(bf16, K % (2 * C::BK) == 0);
    TSG_AG_CFG(1, Cfg1)
    TSG_AG_CFG(2, Cfg2)
    TSG_AG_CFG(3, Cfg3)
    TSG_AG_CFG(4, Cfg4)
    TSG_AG_CFG(5, Cfg5)
    TSG_AG_CFG(6, Cfg6)
    TSG_AG_CFG(7, Cfg7)
    TSG_AG_CFG(8, Cfg8)
    TSG_AG_CFG(9, Cfg9)
#undef TSG_AG_CFG
    default: *nt = 0; return nullptr;
  }
}

hipError_t launch_gemm(int id, const AgGemmArgs& a, bool bf16, int grid, hipStream_t s) {
  switch (id) {
    case 1: return launch_gemm_cfg<Cfg1>(a, bf16, grid, s);
    case 2: return launch_gemm_cfg<Cfg2>(a, bf16, grid, s);
    case 3: return launch_gemm_cfg<Cfg3>(a, bf16, grid, s);
    case 4: return launch_gemm_cfg<Cfg4>(a, bf16, grid, s);
    case 5: return launch_gemm_cfg<Cfg5>(a, bf16, grid, s);
    case 6: return launch_gemm_cfg<Cfg6>(a, bf16, grid, s);
    case 7: return launch_gemm_cfg<Cfg7>(a, bf16, grid, s);
    case 8: return launch_gemm_cfg<Cfg8>(a, bf16, grid, s);
    case 9: return launch_gemm_cfg<Cfg9>(a, bf16, grid, s);
    default: return hipErrorInvalidValue;
  }
}

int default_tile(int M, int N, int K) {
  // 256 x 224 when it gives whole waves of 256 tiles (e.g. 8192 x 1792):
  // eight waves of 64 x 112 on 16x16x32 fragments where K allows, which read
  // 31% fewer LDS bytes per MFMA than waves of 32 x 224 on 32x32x16 ones
  if (N % 224 == 0 && M % 256 == 0 && ((M / 256) * (N / 224)) % 256 == 0) return K % 128 ? 8 : 9;
  if (M >= 2048 && N >= 1024) return 1;
  if (M >= 512 && N >= 256) return 3;
  return 6;
}

}  // namespace

// Piece plan of the copy (see CopyArgs): every piece ends with the
// workgroup draining its stores to the coherence point before it arrives,
// which idles it for a memory round trip, so body pieces are as large as the
// workgroup count allows (about the copy volume over the workgroups, between
// 32 KB and 128 KB).  Slab 0, which every tile waits for first, is cut so
// that all workgroups share it; each following head slab gets half as many
// pieces, down to the body size.  Pieces never straddle channels: np counts
// pieces per channel.  Returns false when the copy's 32-bit offsets or the
// unit count would overflow.
bool copy_plan(int R, int C, int chunk_rows, int K, int n_slab, int vpr_log2, int nwg, int* np, int* ustart,
               int64_t* n_units_out) {
  using tsg::kHead;
  const int ch_rows = chunk_rows / C;
  const int64_t total_vec = (int64_t)R * chunk_rows * (K / 8);
  int64_t unit_vec = 2048;
  while (unit_vec < 8192 && unit_vec * 2 * nwg <= total_vec) unit_vec *= 2;
  const int rows_q = 256 >> vpr_log2;  // rows one pass of the workgroup moves
  auto pieces_for_rows = [&](int64_t rows) {
    rows = std::max<int64_t>(1, std::max<int64_t>(rows, std::min(rows_q, ch_rows)));
    return (int)std::max<int64_t>(1, (ch_rows + rows - 1) / rows);
  };
  const int np_body = pieces_for_rows(unit_vec >> vpr_log2);
  int np_head = std::max(np_body, pieces_for_rows(std::max<int64_t>(1, (int64_t)chunk_rows * R / nwg)));
  for (int h = 0; h < kHead; ++h) {
    np[h] = std::max(np_body, np_head);
    np_head /= 2;
  }
  np[kHead] = np_body;
  for (int h = 0; h <= kHead; ++h) {  // no empty piece: every piece arrives once
    const int rp = (ch_rows + np[h] - 1) / np[h];
    np[h] = (ch_rows + rp - 1) / rp;
  }
  int64_t rows_max = 0;
  for (int h = 0; h <= kHead; ++h) rows_max = std::max<int64_t>(rows_max, (ch_rows + np[h] - 1) / np[h]);
  if (rows_max * K * 2 >= (int64_t)1 << 31) return false;
  int64_t n_units = 0;
  for (int h = 0; h < kHead; ++h) {
    ustart[h] = (int)n_units;
    if (h < n_slab) n_units += (int64_t)R * C * np[h];
  }
  ustart[kHead] = (int)n_units;
  n_units += (int64_t)std::max(0, n_slab - kHead) * R * C * np[kHead];
  if (n_units >= ((int64_t)1 << 30)) return false;
  *n_units_out = n_units;
  return true;
}

tsg_status tsg_op_ag(tsg_ctx* ctx, const void* a_local, const void* a_peers, void* a_full,
                     const void* b, void* c, int c_dtype, int M, int N, int K, int R, int rank,
                     const int* arrival_order, const tsg_opts* opts, int mode, void* stream) {
  using namespace tsgh;
  if (!a_local || !a_full || !b || !c || (R > 1 && !a_peers))
    return fail(ctx, TSG_E_INVALID, "gemm_ag_overlap: null pointer");
  if (c_dtype != TSG_F32 && c_dtype != TSG_BF16) return fail(ctx, TSG_E_INVALID, "bad c_dtype");
  if (mode < TSG_MODE_OVERLAP || mode > TSG_MODE_COMM_ONLY) return fail(ctx, TSG_E_INVALID, "bad mode");
  if (R < 1 || R > kMaxRanks || rank < 0 || rank >= R)
    return fail(ctx, TSG_E_SHAPE, "need 1 <= R <= %d and 0 <= rank < R", kMaxRanks);
  if (M < R || M % R || N < 8 || K < 8 || N % 8 || K % 8)
    return fail(ctx, TSG_E_SHAPE, "gemm_ag_overlap: bad shape M=%d N=%d K=%d R=%d", M, N, K, R);
  if (!aligned16(a_local) || (a_peers && !aligned16(a_peers)) || !aligned16(a_full) ||
      !aligned16(b) || !aligned16(c))
    return fail(ctx, TSG_E_ALIGN, "gemm_ag_overlap: pointers must be 16-byte aligned");

  // Arrival order of the chunks: local first, then the given peers (or the
  // ring rank+1, rank+2, ...).
  ChunkOrder ord;
  int pos_of[kMaxRanks];
  for (int i = 0; i < kMaxRanks; ++i) pos_of[i] = -1;
  ord.chunk[0] = (int8_t)rank;
  pos_of[rank] = 0;
  for (int p = 1; p < R; ++p) {
    const int cc = arrival_order ? arrival_order[p - 1] : (rank + p) % R;
    if (cc < 0 || cc >= R || pos_of[cc] >= 0)
      return fail(ctx, TSG_E_INVALID, "arrival_order must be a permutation of the peer ranks");
    ord.chunk[p] = (int8_t)cc;
    pos_of[cc] = p;
  }
  for (int p = R; p < kMaxRanks; ++p) ord.chunk[p] = 0;

  const Opts o = resolve(opts, -1);
  if (o.arrival_gbps < 0) return fail(ctx, TSG_E_INVALID, "arrival_gbps must be >= 0");
  if (o.copy_engine != 0 && o.copy_engine != 1) return fail(ctx, TSG_E_INVALID, "copy_engine must be 0 or 1");
  if (o.copy_engine && o.arrival_gbps)
    return fail(ctx, TSG_E_INVALID, "copy_engine and arrival_gbps cannot be combined");
  const int tile = o.tile ? o.tile : default_tile(M, N, K);
  const TileShape ts = shape_of(tile);
  if (!ts.bm) return fail(ctx, TSG_E_INVALID, "unknown tile id %d", tile);
  if (tile == 9 && K % 128)
    return fail(ctx, TSG_E_UNSUPPORTED, "tile 9 needs K a multiple of 128 (direct-to-LDS loads only)");
  const int chunk_rows = M / R;
  // Channels ([TL] section 4.1): C signals per rank, M / (R C) rows each.
  const int C = o.channels > 0 ? o.channels : 1;
  if (o.channels < 0 || C > kMaxChannels || chunk_rows % C)
    return fail(ctx, TSG_E_INVALID, "channels must be in [1, %d] and divide the %d rows per rank", kMaxChannels,
                chunk_rows);
  const int ch_rows = chunk_rows / C;
  if (C > 1 && ch_rows < 8)
    return fail(ctx, TSG_E_SHAPE, "channels of %d rows: at least 8 rows per channel are needed", ch_rows);
  const int n_mt = (M + ts.bm - 1) / ts.bm, n_nt = (N + ts.bn - 1) / ts.bn;
  if (n_mt > kMaxMTiles) return fail(ctx, TSG_E_UNSUPPORTED, "M / BM exceeds %d", kMaxMTiles);

  // Communication tile: slab width W (power of two, >= 64; capped at 2048
  // columns and at the first power of two >= K, which is one slab per chunk).
  // The copy engines move whole channels: one slab.
  int slab = o.comm_tile ? o.comm_tile : 512;
  if (slab < 64 || (slab & (slab - 1)))
    return fail(ctx, TSG_E_INVALID, "comm_tile must be a power of two >= 64 (got %d)", slab);
  int k_pow2 = 64;
  while (k_pow2 < K) k_pow2 *= 2;
  slab = o.copy_engine ? k_pow2 : std::min(std::min(slab, k_pow2), 2048);
  int slab_log2 = 0;
  while ((1 << slab_log2) < slab) ++slab_log2;
  const int n_slab = (K + slab - 1) / slab;
  if ((size_t)R * C * n_slab > kSigCap)
    return fail(ctx, TSG_E_UNSUPPORTED, "R * channels * ceil(K / comm_tile) exceeds %zu signals", kSigCap);
  const int vpr_log2 = std::min(slab_log2, 11) - 3;
  TSG_HIP(ctx, hipSetDevice(ctx->device));

  // Copy workgroups and streams.  Overlap: in shared mode one workgroup per
  // CU, resident beside the GEMM's workgroups (the copy needs few
  // registers and no LDS); in split mode four per copy CU.  Serial: two per
  // CU.
  // In shared mode the GEMM runs on the caller's stream and the copy on a
  // side stream; their workgroups must be able to share a CU, or a GEMM that
  // fills every CU first would leave the copy no room while it waits for the
  // copy.  Otherwise the two run back to back.  The copy engines need no CU.
  Pair pr{(hipStream_t)stream, (hipStream_t)stream, ctx->n_cus, 0};
  int nwg = o.aux_wgs > 0 ? o.aux_wgs : ctx->n_cus * 2;
  bool back_to_back = mode == TSG_MODE_SERIAL && !o.copy_engine;
  if (!o.copy_engine && (mode == TSG_MODE_OVERLAP || mode == TSG_MODE_COMM_ONLY)) {
    const tsg_status ss = streams(ctx, o, &pr, (hipStream_t)stream);
    if (ss != TSG_OK) return ss;
    if (o.aux_wgs <= 0) nwg = o.aux_cus < 0 ? ctx->n_cus : pr.aux_cus * 4;
    if (mode == TSG_MODE_OVERLAP && o.aux_cus < 0) {
      int nt = 0;
      const void* fn = gemm_fn(tile, c_dtype == TSG_BF16, K, &nt);
      back_to_back = !co_resident(ctx, fn, nt, (const void*)&ag_copy_kernel, 256);
    }
  }
  if (o.copy_engine && mode == TSG_MODE_OVERLAP && o.aux_cus >= 0) {
    // the GEMM on its CU share; the copies on the DMA streams
    const tsg_status ss = streams(ctx, o, &pr, (hipStream_t)stream);
    if (ss != TSG_OK) return ss;
  }
  // A copy of at most kPullAllBytes (every chunk together) is moved by the
  // GEMM's own workgroups, each taking units until none is left before its
  // first wait: one launch on the caller's stream, no copy kernel and no
  // second stream, whose fork and join would cost more than such a copy.
  // Every unit is then taken by a running workgroup before any waits, so the
  // queue drains whatever the grid.  The units are sized for the GEMM's grid.
  const bool pull_all = mode == TSG_MODE_OVERLAP && o.aux_cus < 0 && o.pull_units == 0 && !o.copy_engine &&
                        o.arrival_gbps == 0 && (int64_t)R * chunk_rows * K * 2 <= kPullAllBytes;
  if (pull_all) nwg = n_mt * n_nt;
  int np[kHead + 1], ustart[kHead + 1];
  int64_t n_units = 0;
  if (!copy_plan(R, C, chunk_rows, K, n_slab, vpr_log2, nwg, np, ustart, &n_units))
    return fail(ctx, TSG_E_UNSUPPORTED, "gemm_ag_overlap: K too large for the copy's 32-bit offsets, or too many "
                                        "copy units");
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);

  AgGemmArgs ga;
  ga.a_full = (const uint16_t*)a_full;
  ga.a_local = (const uint16_t*)a_local;
  ga.rank = rank;
  ga.b = (const uint16_t*)b;
  ga.c = c;
  ga.sig = ctx->d_sig + kSigBase;
  ga.sa = sync_args(ctx, o);
  ga.tl = timeline(ctx, o);
  ga.M = M;
  ga.N = N;
  ga.K = K;
  ga.chunk_rows = chunk_rows;
  ga.ch_rows = ch_rows;
  ga.n_tiles_n = n_nt;
  ga.arrivals = 1;  // any completed count: a signal is only published once complete
  ga.n_slab = n_slab;
  ga.sig_stride = n_slab;
  ga.slab_log2 = slab_log2;
  ga.l1_only = ((uintptr_t)a_full % 128 == 0 && K % 64 == 0) ? 1 : 0;

  // The copy moves the peers' chunks in arrival order and the local chunk
  // last: tiles inside the local chunk read it in place, so only the
  // gathered buffer's own content (and tiles straddling it) waits for it.
  ChunkOrder co;
  int copy_pos[kMaxRanks];
  for (int p = 0; p < kMaxRanks; ++p) co.chunk[p] = 0;
  for (int p = 1; p < R; ++p) co.chunk[p - 1] = ord.chunk[p];
  co.chunk[R - 1] = (int8_t)rank;
  for (int p = 0; p < R; ++p) copy_pos[co.chunk[p]] = p;
  // M-tile order: tiles inside the local chunk first, then by the copy step
  // (channel-major, then arrival position) of the last channel a tile spans,
  // ties by row (order knob 1 = plain row order).
  {
    std::vector<std::pair<int, int>> key(n_mt);
    for (int m = 0; m < n_mt; ++m) {
      const int lo = m * ts.bm, hi = std::min(M, lo + ts.bm) - 1;
      int ready = -1;
      if (!(lo / chunk_rows == rank && hi / chunk_rows == rank))
        for (int g = lo / ch_rows; g <= hi / ch_rows; ++g)
          ready = std::max(ready, (g % C) * R + copy_pos[g / C]);
      key[m] = {o.order == 1 ? 0 : ready, m};
    }
    std::sort(key.begin(), key.end());
    for (int m = 0; m < n_mt; ++m) ga.mt_order[m] = (uint16_t)key[m].second;
  }
  const int grid_gemm = n_mt * n_nt;
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  CopyArgs ca;
  ca.a_local = (const u32x4_t*)a_local;
  ca.a_peers = (const u32x4_t*)a_peers;
  ca.a_full = (u32x4_t*)a_full;
  ca.sig = ctx->d_sig + kSigBase;
  ca.cnt = ctx->d_cnt + kSigBase;
  ca.sa = ga.sa;
  ca.tl = ga.tl;
  ca.ord = co;
  ca.k8 = K / 8;
  ca.chunk_rows = chunk_rows;
  ca.R = R;
  ca.rank = rank;
  ca.C = C;
  ca.ch_rows = ch_rows;
  ca.n_slab = n_slab;
  ca.vpr_log2 = vpr_log2;
  for (int h = 0; h <= kHead; ++h) {
    ca.np[h] = np[h];
    ca.ustart[h] = ustart[h];
  }
  ca.n_units = (int)n_units;
  ca.skip_mask = o.skip_mask;
  // Overlap on shared CUs: the caller's stream waits for the GEMM alone (a
  // join would put a barrier packet between consecutive GEMMs on its queue,
  // about 4 us per call).  The GEMM observes every arrival, the local
  // chunk's at the end of the tiles inside it, so the gathered buffer and C
  // are whole when the stream passes the call; the copy kernel's workgroups
  // may then still be leaving their work queue, whose words no other launch
  // uses than later copies on the same side stream.  With a timeline the
  // copy's rows are written after its arrivals, so the call joins.
  const bool detached = mode == TSG_MODE_OVERLAP && o.aux_cus < 0 && pr.main == caller && !pull_all &&
                        !back_to_back && !o.copy_engine && !o.timeline && o.skip_mask == 0;
  ca.queue = ctx->d_queue + kQueueSlot + (detached ? 0 : 2);
  ca.pace_word = ctx->d_sig + kPaceSlot;
  // pacing: ticks (100 MHz wall clock) per unit at the requested rate
  ca.pace_ticks = o.arrival_gbps > 0
                      ? (float)((double)R * chunk_rows * K * 2 / (double)n_units / (double)o.arrival_gbps *
                                ((double)ctx->wall_khz / 1e6))
                      : 0.f;
  // Units the GEMM pulls itself (overlap on shared CUs, tiles of 256 or 512 threads,
  // whose workgroups move a unit the way the copy's do): by default one per
  // workgroup of the first wave of tiles, at most the first slab's units.
  const int copy_grid = (int)std::min<int64_t>(nwg, n_units);
  int pull = 0;
  int gemm_nt = 0;
  (void)gemm_fn(tile, c_dtype == TSG_BF16, K, &gemm_nt);
  if (pull_all) {
    pull = grid_gemm;
  } else if (mode == TSG_MODE_OVERLAP && !back_to_back && o.aux_cus < 0 && o.pull_units >= 0 && !o.copy_engine &&
             (gemm_nt == 256 || gemm_nt == 512)) {
    pull = o.pull_units > 0 ? o.pull_units : std::min(ctx->n_cus, ustart[1]);
    pull = (int)std::min<int64_t>(std::min(pull, grid_gemm), n_units);
  }
  // Units 0 .. pull - 1 are moved by GEMM workgroups 0 .. pull - 1 directly
  // (no ticket: at the start every workgroup of the GPU would claim from the
  // one counter at once); the copy kernel's queue hands out the rest.
  ca.unit_base = (!pull_all && pull > 0) ? pull : 0;
  ca.n_workers = (uint32_t)(pull_all ? pull : copy_grid);
  ga.pull_wgs = 0;
  ga.pull_all = pull_all ? 1 : 0;
  ga.wait_local_end = detached ? 1 : 0;
  ga.copy = ca;

  auto gemm = [&](hipStream_t s, int wait, int cus) -> tsg_status {
    ga.wait = wait;
    ga.pull_wgs = wait ? pull : 0;
    ga.per_xcd = cus / 8;
    time_begin(ctx, 0, s);
    hipError_t e = launch_gemm(tile, ga, c_dtype == TSG_BF16, grid_gemm, s);
    time_end(ctx, 0, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "ag_gemm_kernel");
    return TSG_OK;
  };

  if (o.copy_engine) {
    // ---- copy engines: one stream per chunk, fork from / join to `caller`
    if (mode == TSG_MODE_COMPUTE_ONLY) return gemm(caller, 0, ctx->n_cus);
    // The runtime runs device copies below 64 KB as blit kernels on the
    // CUs and larger ones on the DMA engines, so each signal is a 64 KB copy
    // too: the window of the ring of signal values that ends with this
    // call's entry, into the channel's signal block, whose last word is what
    // the GEMM polls (the window's other words land in the block's unread
    // part).  The ring is refilled (a short kernel ahead of the fork) once
    // the epochs it covers are used up.
    const uint32_t e = ga.sa.epoch;
    hipStream_t ds[kMaxRanks];
    for (int p = 0; p < R; ++p) {
      tsg_status st = dma_stream(ctx, p, &ds[p]);
      if (st != TSG_OK) return st;
    }
    hipStream_t join_s = nullptr;
    {
      tsg_status st = dma_stream(ctx, kMaxRanks, &join_s);
      if (st != TSG_OK) return st;
    }
    // A copy below 64 KB runs as a kernel on the CUs; beside a GEMM that
    // holds every CU it could not start while the tiles wait for it.
    if (mode == TSG_MODE_OVERLAP && o.aux_cus < 0 && grid_gemm >= ctx->n_cus &&
        (size_t)ch_rows * K * 2 < tsg_ctx::kDmaSigBytes)
      return fail(ctx, TSG_E_UNSUPPORTED,
                  "copy engines beside a GEMM on every CU need channel copies of at least 64 KB "
                  "(rows per channel x K x 2 bytes); use fewer channels or a CU split");
    {
      tsg_status st = dma_sig_blocks(ctx, R * C);
      if (st != TSG_OK) return st;
    }
    uint64_t* const ring = ctx->d_dma_ring + tsg_ctx::kDmaRingPad;
    if (!ctx->dma_ring_valid || e < ctx->dma_ring_base || e - ctx->dma_ring_base >= (uint32_t)tsg_ctx::kDmaRing) {
      hipLaunchKernelGGL(ag_dma_ring_kernel, dim3(64), dim3(256), 0, caller, ring, (int)tsg_ctx::kDmaRing, e);
      tsg_status st = check_launch(ctx, "ag_dma_ring_kernel");
      if (st != TSG_OK) return st;
      ctx->dma_ring_base = e;
      ctx->dma_ring_valid = true;
    }
    // the window of the ring that ends with this call's entry
    const char* win = (const char*)(ring + (e - ctx->dma_ring_base) + 1) - tsg_ctx::kDmaSigBytes;
    ga.sig = (uint64_t*)((char*)ctx->d_dma_sig + tsg_ctx::kDmaSigBytes) - 1;
    ga.sig_stride = (int)(tsg_ctx::kDmaSigBytes / sizeof(uint64_t));
    // Fork, then every copy, then the GEMM: the copies are all queued on
    // the engines' streams before the GEMM is queued, so that none of them
    // can be ordered behind the GEMM whose tiles wait for it.
    TSG_HIP(ctx, hipEventRecord(ctx->ev_fork, caller));
    hipStream_t gs = caller;
    if (mode == TSG_MODE_OVERLAP && pr.main != caller) {
      gs = pr.main;  // the GEMM on its CU share
      TSG_HIP(ctx, hipStreamWaitEvent(gs, ctx->ev_fork, 0));
    }
    TSG_HIP(ctx, hipStreamWaitEvent(join_s, ctx->ev_fork, 0));
    for (int p = 0; p < R; ++p) TSG_HIP(ctx, hipStreamWaitEvent(ds[p], ctx->ev_fork, 0));
    time_begin(ctx, 1, join_s);
    const size_t ch_bytes = (size_t)ch_rows * K * 2;
    const size_t chunk_bytes = (size_t)chunk_rows * K * 2;
    // Copy (arrival position p, channel ch) goes to stream (p C + ch) mod
    // R: with one channel, one stream per chunk; with C = R channels,
    // stream j takes channel j of every chunk in arrival order, so that a
    // whole chunk lands at each step, moved by every engine at once.
    for (int p = 0; p < R; ++p) {
      const int cc = co.chunk[p];
      const char* src = cc == rank ? (const char*)a_local
                                   : (const char*)a_peers + (size_t)(cc < rank ? cc : cc - 1) * chunk_bytes;
      char* dst = (char*)a_full + (size_t)cc * chunk_bytes;
      for (int ch = 0; ch < C; ++ch) {
        hipStream_t st = ds[(p * C + ch) % R];
        // copies on one stream complete in order: the signal lands after
        // the channel's data (both run on the engines: 64 KB and more)
        TSG_HIP(ctx, hipMemcpyAsync(dst + ch * ch_bytes, src + ch * ch_bytes, ch_bytes,
                                    hipMemcpyDeviceToDeviceNoCU, st));
        const int g = cc * C + ch;
        if (!(g < 32 && ((o.skip_mask >> g) & 1u)))
          TSG_HIP(ctx, hipMemcpyAsync((char*)ctx->d_dma_sig + (size_t)g * tsg_ctx::kDmaSigBytes, win,
                                      tsg_ctx::kDmaSigBytes, hipMemcpyDeviceToDeviceNoCU, st));
      }
    }
    for (int p = 0; p < R; ++p) {
      TSG_HIP(ctx, hipEventRecord(ctx->ev_dma[p], ds[p]));
      TSG_HIP(ctx, hipStreamWaitEvent(join_s, ctx->ev_dma[p], 0));
    }
    time_end(ctx, 1, join_s);
    TSG_HIP(ctx, hipEventRecord(ctx->ev_join[1], join_s));
    if (mode == TSG_MODE_OVERLAP) {
      // GEMM last: dispatched at once, its tiles wait for the channels the
      // engines deliver.
      tsg_status st = gemm(gs, 1, gs == caller ? ctx->n_cus : pr.main_cus);
      if (st != TSG_OK) return st;
    }
    if (mode == TSG_MODE_SERIAL) {
      // the whole gather first, then the GEMM (its waits already satisfied)
      TSG_HIP(ctx, hipStreamWaitEvent(caller, ctx->ev_join[1], 0));
      return gemm(caller, 1, ctx->n_cus);
    }
    if (gs != caller) {
      TSG_HIP(ctx, hipEventRecord(ctx->ev_join[0], gs));
      TSG_HIP(ctx, hipStreamWaitEvent(caller, ctx->ev_join[0], 0));
    }
    TSG_HIP(ctx, hipStreamWaitEvent(caller, ctx->ev_join[1], 0));
    return TSG_OK;
  }

  auto copy = [&](hipStream_t s) -> tsg_status {
    time_begin(ctx, 1, s);
    hipLaunchKernelGGL(ag_copy_kernel, dim3(copy_grid), dim3(256), 0, s, ca);
    time_end(ctx, 1, s);
    return check_launch(ctx, "ag_copy_kernel");
  };

  tsg_status st = TSG_OK;
  if (pull_all) return gemm(caller, 1, ctx->n_cus);
  if (back_to_back) {
    st = copy(caller);
    if (st == TSG_OK) st = gemm(caller, 1, ctx->n_cus);
    return st;
  }
  if (mode == TSG_MODE_COMPUTE_ONLY) return gemm(caller, 0, ctx->n_cus);
  // the copy alone on shared CUs has nothing to overlap with: no fork
  if (mode == TSG_MODE_COMM_ONLY && o.aux_cus < 0) return copy(caller);

  st = fork(ctx, caller, pr);
  if (st != TSG_OK) return st;
  // Producer (copy) first, consumer (GEMM) second.  The copy never waits and
  // can always find room (split CUs, or a CU shared with a GEMM workgroup);
  // the GEMM's waits are bounded, so a consumer dispatched ahead of a producer
  // that cannot run (as under a profiler that serialises kernels) ends in a
  // reported timeout rather than a hang.
  if (mode == TSG_MODE_OVERLAP && pr.main == caller) {
    // The GEMM needs no fork: launched first it is dispatched at once, and the
    // copy's workgroups join it on the same CUs.
    st = gemm(pr.main, 1, pr.main_cus);
    if (st == TSG_OK) st = copy(pr.aux);
    if (detached) return st;
  } else {
    st = copy(pr.aux);
    if (st == TSG_OK && mode == TSG_MODE_OVERLAP) st = gemm(pr.main, 1, pr.main_cus);
  }
  tsg_status sj = join(ctx, caller, pr);
  return st != TSG_OK ? st : sj;
}
