// GEMM + ReduceScatter at one rank's share.
//
// Producer: the MFMA GEMM computes the full fp32 partial P = X W.  Row chunk c
// of P (M/R rows) is the contribution destined for rank c.  As soon as a tile
// is stored, one lane releases the done signal of every 128 x 128 sub-tile it
// covers ("TileLink: Generating Efficient Compute-Communication Overlapping
// Kernels using Tile-Centric Primitives", Table 3: producer_tile_notify;
// section 5, Figure 4: the producer GEMM stores partial outputs and notifies
// its consumer per tile).  Tiles of the local chunk come first by default
// ("Triton-distributed: Programming Overlapping Kernels on Distributed AI
// Systems with the Triton Compiler", section 3.7: the producer's tile order
// follows the order its consumers need; the inter-node variant puts the local
// chunk last, which the order knob selects).
//
// Consumer: the reduction stream of that page's Algorithm 3 (section 3.3):
// for each 128 x 128 tile of the local chunk it sums the R-1 peers' partials
// (already resident, no wait), then acquires the tile's done signal
// (consumer_tile_wait) and adds the local partial.  Summation order: peers in
// ascending rank order, then the local partial.
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"

using namespace tsg;

namespace {

constexpr int kMaxRanks = 32;
constexpr int kMaxMTiles = 1024;
constexpr size_t kSigBase = 4096;      // RS signals start here in the context's pool
constexpr int kFlagTile = 128;         // signal granularity (rows and columns)
constexpr size_t kDoneSlot = 24;       // the reduce's completion signal in the context's pool

struct RsGemmArgs {
  const uint16_t* x;
  const uint16_t* w;
  float* partial;
  uint64_t* flags;
  SyncArgs sa;
  Timeline tl;
  int M, N, K;
  int n_tiles_n, n_tiles_m;
  int group;              // tile rows per group of the grouped order
  int n_ftn;             // 128-column signal tiles per row of signals
  int per_xcd;
  int chunk_rows;
  uint32_t skip_mask;    // chunks whose signals are not published (test hook)
  const uint64_t* reduce_done;  // non-null: the last workgroup waits for the reduce's end
  uint32_t reduce_n;            // ... signalled as {epoch | reduce_n}
  uint16_t mt_order[kMaxMTiles];
};

template <class Cfg, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) rs_gemm_kernel(const RsGemmArgs args) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  const int t = xcd_remap(blockIdx.x, gridDim.x, args.per_xcd);
  int ml, nt;
  grouped_tile(t, args.n_tiles_m, args.n_tiles_n, args.group, ml, nt);
  const int mt = args.mt_order[ml];
  const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
  const uint64_t t0 = args.tl.buf ? wall_clock64() : 0;
  typename GemmTile<Cfg>::Acc acc;
  const ARowsLinear ar{args.x, args.K, row0, args.M};
  if (DIRECT)
    GemmTile<Cfg>::run_direct(ar, args.w, args.N, col0, args.N, args.K, lds, acc);
  else
    GemmTile<Cfg>::run_regs(ar, args.w, args.N, col0, args.N, args.K, lds, acc);
  const int M = args.M, N = args.N;
  GemmTile<Cfg>::template store_f32<true>(acc, args.partial + (int64_t)row0 * N + col0, N, M - row0, N - col0);
  // producer_tile_notify: the tile's stores went through to the coherence
  // point; once every wave has them acknowledged, one store per covered
  // 128 x 128 signal publishes it (no L2 write-back).
  block_coherent_complete();
  if (threadIdx.x == 0) {
    const uint64_t v = sig_target(args.sa.epoch, 1);
    for (int i = 0; i < Cfg::BM / kFlagTile; ++i) {
      const int r = row0 + i * kFlagTile;
      if (r >= M || ((args.skip_mask >> (r / args.chunk_rows)) & 1u)) continue;
      for (int j = 0; j < Cfg::BN / kFlagTile; ++j) {
        const int c = col0 + j * kFlagTile;
        if (c >= N) continue;
        __hip_atomic_store(args.flags + (int64_t)(r / kFlagTile) * args.n_ftn + c / kFlagTile, v,
                           __ATOMIC_RELAXED, TSG_SIG_SCOPE);
      }
    }
    if (args.tl.buf) timeline_put(args.tl, 3, (uint32_t)(mt << 16 | nt), t0, t0, wall_clock64());
  }
  // When the caller's stream does not wait for the reduce kernel, the
  // GEMM's end must imply the reduce's: the workgroup dispatched last waits
  // for the reduce's completion signal.
  if (args.reduce_done && blockIdx.x == gridDim.x - 1 && threadIdx.x < 64)
    wave_poll_ge(args.reduce_done, sig_target(args.sa.epoch, args.reduce_n), args.sa);
}

struct RsReduceArgs {
  const float* partial;
  const float* peers;
  float* out;
  const uint64_t* flags;
  SyncArgs sa;
  Timeline tl;
  int M, N, R, rank;
  int chunk_rows;
  int n_ftn;
  int ftm0, n_ftm;       // signal rows covering the local chunk
  int wait;
  uint64_t* done_sig;    // DETACHED: every workgroup arrives here at its end
  uint32_t* done_cnt;
};

// Coherent store of one row segment of 128 floats held as a float4 per lane
// by each 32-lane half of the wave, in 8-byte stores laid out so that every
// store instruction writes whole 128-byte lines: store i of lane l (l within
// its half) writes floats 64 i + 2 l and 64 i + 2 l + 1, which lane
// 16 i + l / 2 of the half holds.  A lane writes only a valid lane's floats.
// Every lane of the wave executes it.
__device__ __forceinline__ void store_segment_coherent(float* seg, float4 v, bool ok) {
  const int lane = __lane_id(), l = lane & 31, half = lane & 32;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int src = half | (16 * i + (l >> 1));
    const float x = __shfl(v.x, src), y = __shfl(v.y, src), z = __shfl(v.z, src), w = __shfl(v.w, src);
    const int src_ok = __shfl((int)ok, src);
    const float lo = (l & 1) ? z : x, hi = (l & 1) ? w : y;
    if (src_ok)
      store_coherent((uint64_t*)(seg + 64 * i + 2 * l),
                     (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32));
  }
}

// Work unit: 16 rows x 128 columns of one 128 x 128 signal tile of the
// local chunk; thread (ry, cx) owns rows ry and ry + 8 at float4 column cx.
// Workgroup g owns units g, g + G, ... and runs two phases over them.
//   Phase 1 (no wait): out = sum of the R - 1 peers' partials, ascending
//   rank, four peers (eight 16-byte loads) in flight at a time.
//   Phase 2 (in unit order, which follows the producer's tile order):
//   acquire the tile's done signal, then out += the local partial.
// Phase 1 depends on nothing the GEMM computes, so it runs beside the
// GEMM's first tiles; only the last third of the traffic waits for them.
// When no GEMM runs beside the reduce (back to back, or the reduce alone),
// each unit is done in one pass instead: acquire its tile's signal (already
// complete), load the peers and the local partial together and store out
// once, which saves writing and re-reading out; the additions are the same.
// Every thread re-reads exactly the elements it stored, so the two phases
// need no synchronisation between threads.  Summation order per element:
// peers in ascending rank order, then the local partial.
// Streaming read of four floats that is not kept in the caches (the peers'
// partials are read once; the L2 keeps serving the GEMM beside the reduce).
__device__ __forceinline__ float4 nt_load4(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

// P_MAX peers per load batch (2 P_MAX 16-byte loads in flight per thread):
// 4 beside the GEMM (the registers a reduce wave has next to a GEMM wave), 8
// when the reduce runs on CUs of its own or after the GEMM (seven peers in
// one batch: one memory round trip per unit).  The summation order is the
// same for both.
// DETACHED (two phases): phase 2 stores out coherently, and every workgroup
// arrives on done_sig at its end, for a GEMM that waits for the reduce.
// Phase 2 then rewrites every line phase 1 left in this XCD's L2, so a later
// write-back of those lines carries the same values.
template <int P_MAX, bool ONE_PASS, bool DETACHED = false>
__global__ void __launch_bounds__(256) rs_reduce_kernel(const RsReduceArgs a) {
  static_assert(!DETACHED || !ONE_PASS, "a detached reduce runs in two phases");
  const int n_units = a.n_ftm * a.n_ftn * 8;
  const int c0 = a.rank * a.chunk_rows, c1 = c0 + a.chunk_rows;
  const int cx = threadIdx.x & 31;
  const int ry = threadIdx.x >> 5;
  auto where = [&](int u, int& ftm, int& ftn, int& r0, int& col) {
    const int tile = u >> 3, part = u & 7;
    ftm = a.ftm0 + tile / a.n_ftn;
    ftn = tile % a.n_ftn;
    col = ftn * kFlagTile + cx * 4;
    r0 = ftm * kFlagTile + part * 16 + ry;
  };
  if constexpr (ONE_PASS) {
    for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
      int ftm, ftn, r0, col;
      where(u, ftm, ftn, r0, col);
      const int r1 = r0 + 8;
      const bool ok0 = col < a.N && r0 >= c0 && r0 < c1;
      const bool ok1 = col < a.N && r1 >= c0 && r1 < c1;
      const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
      if (a.wait) block_poll_ge(a.flags + (int64_t)ftm * a.n_ftn + ftn, sig_target(a.sa.epoch, 1), a.sa);
      const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
      float4 q0, q1;
      if (ok0) q0 = load_coherent((const float4*)(a.partial + (int64_t)r0 * a.N + col));
      if (ok1) q1 = load_coherent((const float4*)(a.partial + (int64_t)r1 * a.N + col));
      float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
      const uint32_t o0 = (uint32_t)((r0 - c0) * a.N + col), o1 = o0 + 8u * (uint32_t)a.N;
      for (int p0 = 0; p0 < a.R - 1; p0 += P_MAX) {
        const int np = min(P_MAX, a.R - 1 - p0);
        float4 v0[P_MAX], v1[P_MAX];
#pragma unroll
        for (int p = 0; p < P_MAX; ++p) {
          if (p < np) {
            const float* pp = a.peers + (int64_t)(p0 + p) * a.chunk_rows * a.N;
            if (ok0) v0[p] = nt_load4(pp + o0);
            if (ok1) v1[p] = nt_load4(pp + o1);
          }
        }
#pragma unroll
        for (int p = 0; p < P_MAX; ++p) {
          if (p < np) {
            if (ok0) { s0.x += v0[p].x; s0.y += v0[p].y; s0.z += v0[p].z; s0.w += v0[p].w; }
            if (ok1) { s1.x += v1[p].x; s1.y += v1[p].y; s1.z += v1[p].z; s1.w += v1[p].w; }
          }
        }
      }
      if (ok0) *(float4*)(a.out + o0) = make_float4(s0.x + q0.x, s0.y + q0.y, s0.z + q0.z, s0.w + q0.w);
      if (ok1) *(float4*)(a.out + o1) = make_float4(s1.x + q1.x, s1.y + q1.y, s1.z + q1.z, s1.w + q1.w);
      if (a.tl.buf && threadIdx.x == 0 && (u & 7) == 0)
        timeline_put(a.tl, 4, (uint32_t)(ftm << 16 | ftn), t0, t1, wall_clock64());
    }
    return;
  }
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    int ftm, ftn, r0, col;
    where(u, ftm, ftn, r0, col);
    const int r1 = r0 + 8;
    const bool ok0 = col < a.N && r0 >= c0 && r0 < c1;
    const bool ok1 = col < a.N && r1 >= c0 && r1 < c1;
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
    for (int p0 = 0; p0 < a.R - 1; p0 += P_MAX) {
      const int np = min(P_MAX, a.R - 1 - p0);
      float4 v0[P_MAX], v1[P_MAX];
      // uniform peer base + 32-bit element offsets (a chunk is < 2^31 elements)
      const uint32_t o0 = (uint32_t)((r0 - c0) * a.N + col), o1 = o0 + 8u * (uint32_t)a.N;
#pragma unroll
      for (int p = 0; p < P_MAX; ++p) {
        if (p < np) {
          const float* pp = a.peers + (int64_t)(p0 + p) * a.chunk_rows * a.N;
          if (ok0) v0[p] = nt_load4(pp + o0);
          if (ok1) v1[p] = nt_load4(pp + o1);
        }
      }
#pragma unroll
      for (int p = 0; p < P_MAX; ++p) {
        if (p < np) {
          if (ok0) { s0.x += v0[p].x; s0.y += v0[p].y; s0.z += v0[p].z; s0.w += v0[p].w; }
          if (ok1) { s1.x += v1[p].x; s1.y += v1[p].y; s1.z += v1[p].z; s1.w += v1[p].w; }
        }
      }
    }
    if (ok0) *(float4*)(a.out + (int64_t)(r0 - c0) * a.N + col) = s0;
    if (ok1) *(float4*)(a.out + (int64_t)(r1 - c0) * a.N + col) = s1;
  }
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    int ftm, ftn, r0, col;
    where(u, ftm, ftn, r0, col);
    const int r1 = r0 + 8;
    const bool ok0 = col < a.N && r0 >= c0 && r0 < c1;
    const bool ok1 = col < a.N && r1 >= c0 && r1 < c1;
    const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
    // consumer_tile_wait; the partial is then read with coherent loads, so the
    // wait needs no cache invalidation (which would also drop the L2 data of
    // the GEMM running beside the reduce).
    if (a.wait) block_poll_ge(a.flags + (int64_t)ftm * a.n_ftn + ftn, sig_target(a.sa.epoch, 1), a.sa);
    const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
    float4 q0, q1, o0, o1;
    float* d0 = a.out + (int64_t)(r0 - c0) * a.N + col;
    float* d1 = a.out + (int64_t)(r1 - c0) * a.N + col;
    if (ok0) { q0 = load_coherent((const float4*)(a.partial + (int64_t)r0 * a.N + col)); o0 = *(const float4*)d0; }
    if (ok1) { q1 = load_coherent((const float4*)(a.partial + (int64_t)r1 * a.N + col)); o1 = *(const float4*)d1; }
    if constexpr (DETACHED) {
      const int seg = ftn * kFlagTile;  // first column of the half-wave's 128
      store_segment_coherent(a.out + (int64_t)(r0 - c0) * a.N + seg,
                             make_float4(o0.x + q0.x, o0.y + q0.y, o0.z + q0.z, o0.w + q0.w), ok0);
      store_segment_coherent(a.out + (int64_t)(r1 - c0) * a.N + seg,
                             make_float4(o1.x + q1.x, o1.y + q1.y, o1.z + q1.z, o1.w + q1.w), ok1);
    } else {
      if (ok0) *(float4*)d0 = make_float4(o0.x + q0.x, o0.y + q0.y, o0.z + q0.z, o0.w + q0.w);
      if (ok1) *(float4*)d1 = make_float4(o1.x + q1.x, o1.y + q1.y, o1.z + q1.z, o1.w + q1.w);
    }
    if (a.tl.buf && threadIdx.x == 0 && (u & 7) == 0)
      timeline_put(a.tl, 4, (uint32_t)(ftm << 16 | ftn), t0, t1, wall_clock64());
  }
  if constexpr (DETACHED) {
    block_coherent_complete();
    if (threadIdx.x == 0) sig_arrive_counted_coherent(a.done_cnt, a.done_sig, gridDim.x, a.sa.epoch);
  }
}

using Cfg1 = TileCfg<256, 256, 2, 2>;
using Cfg3 = TileCfg<128, 128, 2, 2>;
using Cfg4 = TileCfg<256, 128, 2, 2>;
using Cfg5 = TileCfg<128, 256, 2, 2>;
using Cfg6 = TileCfg<256, 256, 4, 2, 16>;  // 16x16x32 fragments, eight waves of 64 x 128

struct TileShape {
  int bm, bn;
};

TileShape shape_of(int id) {
  switch (id) {
    case 1: return {256, 256};
    case 3: return {128, 128};
    case 4: return {256, 128};
    case 5: return {128, 256};
    case 6: return {256, 256};
    default: return {0, 0};
  }
}

template <class Cfg>
hipError_t launch_cfg(const RsGemmArgs& a, int grid, hipStream_t s) {
  if (a.K % (2 * Cfg::BK) == 0)
    hipLaunchKernelGGL((rs_gemm_kernel<Cfg, true>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else
    hipLaunchKernelGGL((rs_gemm_kernel<Cfg, false>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  return hipGetLastError();
}

// The GEMM kernel of a tile id and its workgroup size (threads).
template <class Cfg>
const void* fn_cfg(bool direct, int* nt) {
  *nt = Cfg::NT;
  return direct ? (const void*)&rs_gemm_kernel<Cfg, true> : (const void*)&rs_gemm_kernel<Cfg, false>;
}

const void* gemm_fn(int id, bool direct, int* nt) {
  switch (id) {
    case 1: return fn_cfg<Cfg1>(direct, nt);
    case 3: return fn_cfg<Cfg3>(direct, nt);
    case 4: return fn_cfg<Cfg4>(direct, nt);
    case 5: return fn_cfg<Cfg5>(direct, nt);
    case 6: return fn_cfg<Cfg6>(direct, nt);
    default: return nullptr;
  }
}

hipError_t launch_gemm(int id, const RsGemmArgs& a, int grid, hipStream_t s) {
  switch (id) {
    case 1: return launch_cfg<Cfg1>(a, grid, s);
    case 3: return launch_cfg<Cfg3>(a, grid, s);
    case 4: return launch_cfg<Cfg4>(a, grid, s);
    case 5: return launch_cfg<Cfg5>(a, grid, s);
    case 6: return launch_cfg<Cfg6>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

tsg_status tsg_op_rs(tsg_ctx* ctx, const void* x, const void* w, float* partial,
                     const float* peer_partials, float* out, int M, int N, int K, int R, int rank,
                     const tsg_opts* opts, int mode, void* stream) {
  using namespace tsgh;
  if (!x || !w || !partial || !out || (R > 1 && !peer_partials))
    return fail(ctx, TSG_E_INVALID, "gemm_rs_overlap: null pointer");
  if (mode < TSG_MODE_OVERLAP || mode > TSG_MODE_COMM_ONLY) return fail(ctx, TSG_E_INVALID, "bad mode");
  if (R < 1 || R > kMaxRanks || rank < 0 || rank >= R)
    return fail(ctx, TSG_E_SHAPE, "need 1 <= R <= %d and 0 <= rank < R", kMaxRanks);
  if (M < R || M % R || N < 8 || K < 8 || N % 8 || K % 8)
    return fail(ctx, TSG_E_SHAPE, "gemm_rs_overlap: bad shape M=%d N=%d K=%d R=%d", M, N, K, R);
  if (!aligned16(x) || !aligned16(w) || !aligned16(partial) || !aligned16(out) ||
      (peer_partials && !aligned16(peer_partials)))
    return fail(ctx, TSG_E_ALIGN, "gemm_rs_overlap: pointers must be 16-byte aligned");
  if ((int64_t)(M / R) * N >= (int64_t(1) << 31))
    return fail(ctx, TSG_E_UNSUPPORTED, "gemm_rs_overlap: a chunk of 2^31 elements or more is not supported");
  if ((int64_t)M * K * 2 >= (int64_t(1) << 32) || (int64_t)K * N * 2 >= (int64_t(1) << 32))
    return fail(ctx, TSG_E_UNSUPPORTED, "operands of 4 GiB or more are not supported");

  const Opts o = resolve(opts, -1);
  const int tile = o.tile ? o.tile : ((M >= 2048 && N >= 1024) ? 1 : 3);
  const TileShape ts = shape_of(tile);
  if (!ts.bm) return fail(ctx, TSG_E_INVALID, "tile id %d is not available for gemm_rs_overlap", tile);
  if (tile == 6 && K % 128)
    return fail(ctx, TSG_E_UNSUPPORTED, "tile 6 needs K a multiple of 128 (direct-to-LDS loads only)");
  const int chunk_rows = M / R;
  const int n_mt = (M + ts.bm - 1) / ts.bm, n_nt = (N + ts.bn - 1) / ts.bn;
  if (n_mt > kMaxMTiles) return fail(ctx, TSG_E_UNSUPPORTED, "M / BM exceeds %d", kMaxMTiles);
  const int n_ftm = (M + kFlagTile - 1) / kFlagTile, n_ftn = (N + kFlagTile - 1) / kFlagTile;
  if (kSigBase + (size_t)n_ftm * n_ftn > ctx->n_sig)
    return fail(ctx, TSG_E_UNSUPPORTED, "too many 128x128 tiles for the signal pool");

  TSG_HIP(ctx, hipSetDevice(ctx->device));
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);

  RsGemmArgs ga;
  ga.x = (const uint16_t*)x;
  ga.w = (const uint16_t*)w;
  ga.partial = partial;
  ga.flags = ctx->d_sig + kSigBase;
  ga.sa = sync_args(ctx, o);
  ga.tl = timeline(ctx, o);
  ga.M = M;
  ga.N = N;
  ga.K = K;
  ga.n_tiles_n = n_nt;
  ga.n_tiles_m = n_mt;
  ga.group = 8;
  ga.n_ftn = n_ftn;
  ga.chunk_rows = chunk_rows;
  ga.skip_mask = o.skip_mask;
  ga.reduce_done = nullptr;
  ga.reduce_n = 0;
  // M-tile order: by the position of the tile's first chunk in the order
  // local, rank+1, rank+2, ... (order 0) or rank+1, ..., local last (order 1).
  {
    std::vector<std::pair<int, int>> key(n_mt);
    for (int m = 0; m < n_mt; ++m) {
      const int c = (m * ts.bm) / chunk_rows;
      int pos = (c - rank + R) % R;
      if (o.order == 1) pos = (pos + R - 1) % R;
      key[m] = {pos, m};
    }
    std::sort(key.begin(), key.end());
    for (int m = 0; m < n_mt; ++m) ga.mt_order[m] = (uint16_t)key[m].second;
  }

  RsReduceArgs ra;
  ra.partial = partial;
  ra.peers = peer_partials;
  ra.out = out;
  ra.flags = ga.flags;
  ra.sa = ga.sa;
  ra.tl = ga.tl;
  ra.M = M;
  ra.N = N;
  ra.R = R;
  ra.rank = rank;
  ra.chunk_rows = chunk_rows;
  ra.n_ftn = n_ftn;
  ra.ftm0 = (rank * chunk_rows) / kFlagTile;
  ra.n_ftm = ((rank + 1) * chunk_rows - 1) / kFlagTile - ra.ftm0 + 1;
  ra.done_sig = ctx->d_sig + kDoneSlot;
  ra.done_cnt = ctx->d_cnt + kDoneSlot;
  const int n_red_tiles = ra.n_ftm * n_ftn;
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  auto gemm = [&](hipStream_t s, int cus) -> tsg_status {
    ga.per_xcd = cus / 8;
    time_begin(ctx, 0, s);
    hipError_t e = launch_gemm(tile, ga, n_mt * n_nt, s);
    time_end(ctx, 0, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "rs_gemm_kernel");
    return TSG_OK;
  };
  // beside: the GEMM runs at the same time (on the same or other CUs)
  auto red_grid = [&](int nwg) { return std::max(1, std::min(nwg, 8 * n_red_tiles)); };
  auto reduce = [&](hipStream_t s, int nwg, int wait, bool beside, bool detached = false) -> tsg_status {
    ra.wait = wait;
    const dim3 grid(red_grid(nwg));
    time_begin(ctx, 1, s);
    if (detached)
      hipLaunchKernelGGL((rs_reduce_kernel<4, false, true>), grid, dim3(256), 0, s, ra);
    else if (beside && o.aux_cus < 0)  // sharing every CU with the GEMM: fewer registers
      hipLaunchKernelGGL((rs_reduce_kernel<4, false>), grid, dim3(256), 0, s, ra);
    else if (beside)
      hipLaunchKernelGGL((rs_reduce_kernel<8, false>), grid, dim3(256), 0, s, ra);
    else
      hipLaunchKernelGGL((rs_reduce_kernel<8, true>), grid, dim3(256), 0, s, ra);
    time_end(ctx, 1, s);
    return check_launch(ctx, "rs_reduce_kernel");
  };

  tsg_status st = TSG_OK;
  if (mode == TSG_MODE_COMPUTE_ONLY) return gemm(caller, ctx->n_cus);
  // In shared mode the GEMM runs on the caller's stream and the reduce on a
  // side stream, one workgroup per CU beside the GEMM's; when the two cannot
  // share a CU they run back to back instead.
  // Overlap on shared CUs from a stream of the caller's own: the caller's
  // stream waits for the GEMM alone (a join would put a barrier packet
  // between consecutive GEMMs on its queue).  The reduce stores its final
  // out coherently and signals its end, and the GEMM's last workgroup waits
  // for that signal, so out and the partial are whole when the stream passes
  // the call.  With a timeline (written after the reduce's stores) or a
  // debug skip mask the call joins.
  bool detached = mode == TSG_MODE_OVERLAP && o.aux_cus < 0 && caller != nullptr && !o.timeline &&
                  o.skip_mask == 0;
  bool back_to_back = mode == TSG_MODE_SERIAL;
  if (mode == TSG_MODE_OVERLAP && o.aux_cus < 0) {
    // (a reduce workgroup placed where the GEMM's next tile cannot then fit
    // would wait for that tile until its time-out)
    const bool direct = K % 128 == 0;
    int gemm_nt = 0;
    const void* fn = gemm_fn(tile, direct, &gemm_nt);
    const void* red = detached ? (const void*)&rs_reduce_kernel<4, false, true>
                               : (const void*)&rs_reduce_kernel<4, false>;
    back_to_back = !co_resident(ctx, fn, gemm_nt, red, 256);
    detached = detached && !back_to_back;
  }
  if (back_to_back) {
    st = gemm(caller, ctx->n_cus);
    if (st == TSG_OK) st = reduce(caller, o.aux_wgs > 0 ? o.aux_wgs : ctx->n_cus * 2, 1, false);
    return st;
  }

  // the reduce alone on shared CUs has nothing to overlap with: no fork
  if (mode == TSG_MODE_COMM_ONLY && o.aux_cus < 0)
    return reduce(caller, o.aux_wgs > 0 ? o.aux_wgs : 2 * ctx->n_cus, 0, false);
  Pair pr;
  st = streams(ctx, o, &pr, caller);
  if (st != TSG_OK) return st;
  const int nwg = o.aux_wgs > 0 ? o.aux_wgs : (o.aux_cus < 0 ? 2 * ctx->n_cus : pr.aux_cus * 2);
  st = fork(ctx, caller, pr);
  if (st != TSG_OK) return st;
  if (detached) {
    ga.reduce_done = ra.done_sig;
    ga.reduce_n = (uint32_t)red_grid(nwg);
  }
  // Producer (GEMM) first, consumer (reduce) second: the GEMM waits for the
  // reduce only in its last workgroup, at its end.
  if (mode == TSG_MODE_OVERLAP) st = gemm(pr.main, pr.main_cus);
  if (st == TSG_OK) st = reduce(pr.aux, nwg, mode == TSG_MODE_OVERLAP ? 1 : 0, mode == TSG_MODE_OVERLAP, detached);
  if (detached) return st;
  tsg_status sj = join(ctx, caller, pr);
  return st != TSG_OK ? st : sj;
}
