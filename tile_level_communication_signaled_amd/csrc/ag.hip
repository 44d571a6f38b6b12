// AllGather + GEMM at one rank's share.
//
// Producer: a copy kernel standing in for the peers' arrival.  It moves the
// shards chunk by chunk in arrival order (the local shard first) into the
// gathered buffer and releases each chunk's signal once every copy workgroup
// has finished its slice of that chunk ("Triton-distributed: Programming
// Overlapping Kernels on Distributed AI Systems with the Triton Compiler",
// section 3.2, Algorithm 2, pull mode: local copy and signal, then one copy
// and one signal per peer).
//
// Consumer: the MFMA GEMM.  Workgroup w takes the w-th tile of a swizzled
// order that starts at the local chunk and follows the arrival order (same
// page, section 3.7: the compute tile order is aligned with the arrival order
// of the communication tiles), waits (acquire) on the signals of every chunk
// its rows span, then runs its K loop.  The chunk a row belongs to is the
// static rank mapping of "TileLink: Generating Efficient Compute-
// Communication Overlapping Kernels using Tile-Centric Primitives", section
// 4.1 (rank = floor(row / M_per_rank)) with one channel per rank.
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"

using namespace tsg;

namespace {

constexpr int kMaxRanks = 32;
constexpr int kMaxMTiles = 1024;

struct ChunkOrder {
  int8_t chunk[kMaxRanks];  // chunk copied at arrival position p (p = 0: local)
};

// ---------------------------------------------------------------- copy
__global__ void __launch_bounds__(256) ag_copy_kernel(const uint16_t* __restrict__ a_local,
                                                      const uint16_t* __restrict__ a_peers,
                                                      uint16_t* __restrict__ a_full,
                                                      int64_t chunk_vec, int R, int rank,
                                                      ChunkOrder ord, uint64_t* sig, uint32_t* cnt,
                                                      SyncArgs sa, uint32_t skip_mask, Timeline tl) {
  constexpr int U = 8;  // 16-byte vectors in flight per thread
  const int64_t nwg = gridDim.x, w = blockIdx.x;
  const int64_t lo = chunk_vec * w / nwg, hi = chunk_vec * (w + 1) / nwg;
  for (int p = 0; p < R; ++p) {
    const int c = ord.chunk[p];
    const uint64_t t0 = tl.buf ? wall_clock64() : 0;
    const u32x4_t* __restrict__ src =
        (const u32x4_t*)(c == rank ? a_local : a_peers + (int64_t)(c < rank ? c : c - 1) * chunk_vec * 8);
    u32x4_t* __restrict__ dst = (u32x4_t*)a_full + (int64_t)c * chunk_vec;
    int64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * 256 < hi; i += U * 256) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
      for (int u = 0; u < U; ++u) dst[i + u * 256] = v[u];
    }
    for (; i < hi; i += 256) dst[i] = __builtin_nontemporal_load(src + i);
    block_release_fence();
    if (threadIdx.x == 0 && !((skip_mask >> c) & 1u))
      sig_arrive_counted_lane(cnt + c, sig + c, (uint32_t)nwg, sa.epoch);
    if (threadIdx.x == 0 && tl.buf) timeline_put(tl, 1, (uint32_t)(c << 16 | w), t0, t0, wall_clock64());
  }
}

// ---------------------------------------------------------------- GEMM
struct AgGemmArgs {
  const uint16_t* a_full;
  const uint16_t* b;
  void* c;
  uint64_t* sig;
  SyncArgs sa;
  Timeline tl;
  int M, N, K;
  int chunk_rows;
  int n_tiles_n;
  int wait;               // 0: no waits (compute-only)
  uint32_t arrivals;      // arrivals that complete one chunk signal
  int per_xcd;            // resident tiles per XCD (0 = no XCD remap)
  uint16_t mt_order[kMaxMTiles];
};

template <class Cfg, bool OUT_BF16, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) ag_gemm_kernel(const AgGemmArgs args) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  const int w = xcd_remap(blockIdx.x, gridDim.x, args.per_xcd);
  const int mt = args.mt_order[w / args.n_tiles_n];
  const int nt = w % args.n_tiles_n;
  const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
  const uint64_t t0 = args.tl.buf ? wall_clock64() : 0;
  if (args.wait) {
    const int last = min(row0 + Cfg::BM, args.M) - 1;
    const uint64_t target = sig_target(args.sa.epoch, args.arrivals);
    for (int c = row0 / args.chunk_rows; c <= last / args.chunk_rows; ++c)
      block_wait_ge(args.sig + c, target, args.sa);
  }
  const uint64_t t1 = args.tl.buf ? wall_clock64() : 0;
  typename GemmTile<Cfg>::Acc acc;
  const ARowsLinear ar{args.a_full, args.K, row0, args.M};
  if (DIRECT)
    GemmTile<Cfg>::run_direct(ar, args.b, args.N, col0, args.N, args.K, lds, acc);
  else
    GemmTile<Cfg>::run_regs(ar, args.b, args.N, col0, args.N, args.K, lds, acc);
  const int M = args.M, N = args.N;
  if (OUT_BF16) {
    uint16_t* C = (uint16_t*)args.c;
    GemmTile<Cfg>::for_each(acc, [&](int r, int c, float v) {
      const int gr = row0 + r, gc = col0 + c;
      if (gr < M && gc < N) C[(int64_t)gr * N + gc] = (uint16_t)f32_to_bf16(v);
    });
  } else {
    float* C = (float*)args.c;
    GemmTile<Cfg>::for_each(acc, [&](int r, int c, float v) {
      const int gr = row0 + r, gc = col0 + c;
      if (gr < M && gc < N) C[(int64_t)gr * N + gc] = v;
    });
  }
  if (args.tl.buf && threadIdx.x == 0)
    timeline_put(args.tl, 2, (uint32_t)(mt << 16 | nt), t0, t1, wall_clock64());
}

// Tile configurations (id -> BM x BN, waves).
using Cfg1 = TileCfg<256, 256, 2, 2>;
using Cfg2 = TileCfg<256, 224, 4, 1>;
using Cfg3 = TileCfg<128, 128, 2, 2>;
using Cfg4 = TileCfg<256, 128, 2, 2>;
using Cfg5 = TileCfg<128, 256, 2, 2>;
using Cfg6 = TileCfg<64, 64, 1, 1>;
using Cfg7 = TileCfg<128, 64, 2, 1>;

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

hipError_t launch_gemm(int id, const AgGemmArgs& a, bool bf16, int grid, hipStream_t s) {
  switch (id) {
    case 1: return launch_gemm_cfg<Cfg1>(a, bf16, grid, s);
    case 2: return launch_gemm_cfg<Cfg2>(a, bf16, grid, s);
    case 3: return launch_gemm_cfg<Cfg3>(a, bf16, grid, s);
    case 4: return launch_gemm_cfg<Cfg4>(a, bf16, grid, s);
    case 5: return launch_gemm_cfg<Cfg5>(a, bf16, grid, s);
    case 6: return launch_gemm_cfg<Cfg6>(a, bf16, grid, s);
    case 7: return launch_gemm_cfg<Cfg7>(a, bf16, grid, s);
    default: return hipErrorInvalidValue;
  }
}

int default_tile(int M, int N) {
  // 256 x 224 when it gives whole waves of 256 tiles (e.g. 8192 x 1792)
  if (N % 224 == 0 && M % 256 == 0 && ((M / 256) * (N / 224)) % 256 == 0) return 2;
  if (M >= 2048 && N >= 1024) return 1;
  if (M >= 512 && N >= 256) return 3;
  return 6;
}

}  // namespace

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
  const int tile = o.tile ? o.tile : default_tile(M, N);
  const TileShape ts = shape_of(tile);
  if (!ts.bm) return fail(ctx, TSG_E_INVALID, "unknown tile id %d", tile);
  const int chunk_rows = M / R;
  const int n_mt = (M + ts.bm - 1) / ts.bm, n_nt = (N + ts.bn - 1) / ts.bn;
  if (n_mt > kMaxMTiles) return fail(ctx, TSG_E_UNSUPPORTED, "M / BM exceeds %d", kMaxMTiles);

  TSG_HIP(ctx, hipSetDevice(ctx->device));
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);

  AgGemmArgs ga;
  ga.a_full = (const uint16_t*)a_full;
  ga.b = (const uint16_t*)b;
  ga.c = c;
  ga.sig = ctx->d_sig;  // chunk signals 0 .. R-1
  ga.sa = sync_args(ctx, o);
  ga.tl = timeline(ctx, o);
  ga.M = M;
  ga.N = N;
  ga.K = K;
  ga.chunk_rows = chunk_rows;
  ga.n_tiles_n = n_nt;
  // M-tile order: by the arrival position of the last chunk a tile spans,
  // ties by row (order knob 1 = plain row order).
  {
    std::vector<std::pair<int, int>> key(n_mt);
    for (int m = 0; m < n_mt; ++m) {
      const int lo = m * ts.bm, hi = std::min(M, lo + ts.bm) - 1;
      int ready = 0;
      for (int cc = lo / chunk_rows; cc <= hi / chunk_rows; ++cc) ready = std::max(ready, pos_of[cc]);
      key[m] = {o.order == 1 ? 0 : ready, m};
    }
    std::sort(key.begin(), key.end());
    for (int m = 0; m < n_mt; ++m) ga.mt_order[m] = (uint16_t)key[m].second;
  }
  const int64_t chunk_vec = (int64_t)chunk_rows * K / 8;
  const int grid_gemm = n_mt * n_nt;
  const Timeline tl = timeline(ctx, o);
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  auto copy = [&](hipStream_t s, int nwg) -> tsg_status {
    time_begin(ctx, 1, s);
    hipLaunchKernelGGL(ag_copy_kernel, dim3(nwg), dim3(256), 0, s, (const uint16_t*)a_local,
                       (const uint16_t*)a_peers, (uint16_t*)a_full, chunk_vec, R, rank, ord,
                       ctx->d_sig, ctx->d_cnt, ga.sa, o.skip_mask, tl);
    time_end(ctx, 1, s);
    return check_launch(ctx, "ag_copy_kernel");
  };
  auto gemm = [&](hipStream_t s, int wait, uint32_t arrivals, int cus) -> tsg_status {
    ga.wait = wait;
    ga.arrivals = arrivals;
    ga.per_xcd = cus / 8;
    time_begin(ctx, 0, s);
    hipError_t e = launch_gemm(tile, ga, c_dtype == TSG_BF16, grid_gemm, s);
    time_end(ctx, 0, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "ag_gemm_kernel");
    return TSG_OK;
  };

  tsg_status st = TSG_OK;
  if (mode == TSG_MODE_SERIAL) {
    const int nwg = ctx->n_cus * 2;
    st = copy(caller, nwg);
    if (st == TSG_OK) st = gemm(caller, 1, (uint32_t)nwg, ctx->n_cus);
    return st;
  }
  if (mode == TSG_MODE_COMPUTE_ONLY) return gemm(caller, 0, 0, ctx->n_cus);

  Pair pr;
  st = streams(ctx, o, &pr);
  if (st != TSG_OK) return st;
  // Copy workgroups: each release of a chunk slice costs an L2 write-back, so
  // a few wide workgroups (8 per XCD) rather than many.
  const int nwg = o.aux_cus < 0 ? 64 : std::min(64, pr.aux_cus * 4);
  st = fork(ctx, caller, pr);
  if (st != TSG_OK) return st;
  // Producer (copy) first, consumer (GEMM) second: the copy never waits, so
  // even if the two kernels were serialised the GEMM's waits would all be
  // satisfied.
  st = copy(pr.aux, nwg);
  if (st == TSG_OK && mode == TSG_MODE_OVERLAP) st = gemm(pr.main, 1, (uint32_t)nwg, pr.main_cus);
  tsg_status sj = join(ctx, caller, pr);
  return st != TSG_OK ? st : sj;
}
