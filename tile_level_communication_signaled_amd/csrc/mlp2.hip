// CTA-pipelined two-GEMM MLP on one GPU.
//
// Digest page "Resource-aware Computation-Communication Overlap for
// multi-GPU ML Workloads" (CTA-pipelining abstract): a dependent kernel runs
// concurrently with its producer, each of its CTAs starting as soon as the
// producer CTAs it depends on are done; shown on a 2-layer GEMM that stands
// for the MLP.  Here both GEMMs run on one GPU:
//
//   GEMM1 (producer): H = bf16(GELU(X W1)), tiles visited 128-row block by
//     row block.  After storing a tile, one lane arrives on the signal of each
//     128-row block the tile covers ("TileLink: Generating Efficient
//     Compute-Communication Overlapping Kernels using Tile-Centric Primitives",
//     Table 3: a consumer tile is ready once all the producer tiles it depends
//     on are done -- here the N1 / BN1 tiles of that row block).
//   GEMM2 (consumer, persistent): Y = H W2 in fp32; each tile first acquires
//     the signals of the row blocks it reads, then runs its K loop over H.
//
// GELU is the exact form 0.5 z (1 + erf(z / sqrt 2)) on the fp32 accumulator
// (erff of the device math library), rounded to bf16 (nearest even): H is the
// bf16 operand of GEMM2.  The two kernels sit on a CU split (default 192 / 64)
// or share every CU, with the persistent consumer bounded to 64 workgroups so
// that the producer always keeps most of the GPU.
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"

using namespace tsg;

namespace {

constexpr size_t kSigBase = 64;     // row-block signals of MLP2 in the context's pool
constexpr int kRowBlock = 128;
constexpr int kMaxRowBlocks = 4000;

struct Mlp1Args {
  const uint16_t* x;
  const uint16_t* w1;
  uint16_t* h;
  uint64_t* sig;
  uint32_t* cnt;
  SyncArgs sa;
  Timeline tl;
  int M, K1, N1;
  int n_tiles_n;
  int per_xcd;
  uint32_t arrivals;      // GEMM1 tiles per row block (= n_tiles_n)
  uint32_t skip_mask;     // row blocks whose signal is never completed (test hook)
};

template <class Cfg, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) mlp_gemm1_kernel(const Mlp1Args a) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  const int t = xcd_remap(blockIdx.x, gridDim.x, a.per_xcd);
  const int mt = t / a.n_tiles_n, nt = t % a.n_tiles_n;
  const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
  const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
  typename GemmTile<Cfg>::Acc acc;
  const ARowsLinear ar{a.x, a.K1, row0, a.M};
  if (DIRECT)
    GemmTile<Cfg>::run_direct(ar, a.w1, a.N1, col0, a.N1, a.K1, lds, acc);
  else
    GemmTile<Cfg>::run_regs(ar, a.w1, a.N1, col0, a.N1, a.K1, lds, acc);
  const int M = a.M, N1 = a.N1;
  uint16_t* H = a.h;
  GemmTile<Cfg>::for_each(acc, [&](int r, int c, float z) {
    const int gr = row0 + r, gc = col0 + c;
    if (gr < M && gc < N1) {
      const float g = 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
      H[(int64_t)gr * N1 + gc] = (uint16_t)f32_to_bf16(g);
    }
  });
  block_release_fence();
  if (threadIdx.x == 0) {
    for (int b = row0 / kRowBlock; b * kRowBlock < min(row0 + Cfg::BM, M); ++b) {
      if ((a.skip_mask >> (b & 31)) & 1u) continue;
      sig_arrive_counted_lane(a.cnt + b, a.sig + b, a.arrivals, a.sa.epoch);
    }
    if (a.tl.buf) timeline_put(a.tl, 5, (uint32_t)(mt << 16 | nt), t0, t0, wall_clock64());
  }
}

struct Mlp2Args {
  const uint16_t* h;
  const uint16_t* w2;
  float* y;
  const uint64_t* sig;
  SyncArgs sa;
  Timeline tl;
  int M, N1, N2;
  int n_tiles_n, n_tiles;
  int wait;
  uint32_t arrivals;
};

// Persistent: workgroup g computes tiles g, g + G, ... in row-block-major
// order, so the first tiles need the first row blocks GEMM1 completes.
template <class Cfg, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) mlp_gemm2_kernel(const Mlp2Args a) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  for (int t = blockIdx.x; t < a.n_tiles; t += gridDim.x) {
    const int mt = t / a.n_tiles_n, nt = t % a.n_tiles_n;
    const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
    const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
    if (a.wait) {
      const uint64_t target = sig_target(a.sa.epoch, a.arrivals);
      for (int b = row0 / kRowBlock; b * kRowBlock < min(row0 + Cfg::BM, a.M); ++b)
        block_wait_ge(a.sig + b, target, a.sa);
    }
    const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
    typename GemmTile<Cfg>::Acc acc;
    const ARowsLinear ar{a.h, a.N1, row0, a.M};
    if (DIRECT)
      GemmTile<Cfg>::run_direct(ar, a.w2, a.N2, col0, a.N2, a.N1, lds, acc);
    else
      GemmTile<Cfg>::run_regs(ar, a.w2, a.N2, col0, a.N2, a.N1, lds, acc);
    const int M = a.M, N2 = a.N2;
    float* Y = a.y;
    GemmTile<Cfg>::for_each(acc, [&](int r, int c, float v) {
      const int gr = row0 + r, gc = col0 + c;
      if (gr < M && gc < N2) Y[(int64_t)gr * N2 + gc] = v;
    });
    if (a.tl.buf && threadIdx.x == 0) timeline_put(a.tl, 6, (uint32_t)(mt << 16 | nt), t0, t1, wall_clock64());
    __syncthreads();  // LDS of this tile fully consumed before the next one
  }
}

using Cfg1 = TileCfg<256, 256, 2, 2>;
using Cfg3 = TileCfg<128, 128, 2, 2>;
using Cfg4 = TileCfg<256, 128, 2, 2>;
using Cfg5 = TileCfg<128, 256, 2, 2>;

struct TileShape {
  int bm, bn;
};

TileShape shape_of(int id) {
  switch (id) {
    case 1: return {256, 256};
    case 3: return {128, 128};
    case 4: return {256, 128};
    case 5: return {128, 256};
    default: return {0, 0};
  }
}

template <class Cfg>
hipError_t launch1_cfg(const Mlp1Args& a, int grid, hipStream_t s) {
  if (a.K1 % (2 * Cfg::BK) == 0)
    hipLaunchKernelGGL((mlp_gemm1_kernel<Cfg, true>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else
    hipLaunchKernelGGL((mlp_gemm1_kernel<Cfg, false>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  return hipGetLastError();
}

template <class Cfg>
hipError_t launch2_cfg(const Mlp2Args& a, int grid, hipStream_t s) {
  if (a.N1 % (2 * Cfg::BK) == 0)
    hipLaunchKernelGGL((mlp_gemm2_kernel<Cfg, true>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else
    hipLaunchKernelGGL((mlp_gemm2_kernel<Cfg, false>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch1(int id, const Mlp1Args& a, int grid, hipStream_t s) {
  switch (id) {
    case 1: return launch1_cfg<Cfg1>(a, grid, s);
    case 3: return launch1_cfg<Cfg3>(a, grid, s);
    case 4: return launch1_cfg<Cfg4>(a, grid, s);
    case 5: return launch1_cfg<Cfg5>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch2(int id, const Mlp2Args& a, int grid, hipStream_t s) {
  switch (id) {
    case 1: return launch2_cfg<Cfg1>(a, grid, s);
    case 3: return launch2_cfg<Cfg3>(a, grid, s);
    case 4: return launch2_cfg<Cfg4>(a, grid, s);
    case 5: return launch2_cfg<Cfg5>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

tsg_status tsg_op_mlp2(tsg_ctx* ctx, const void* x, const void* w1, void* h, const void* w2,
                       float* y, int M, int K1, int N1, int N2, const tsg_opts* opts, int mode,
                       void* stream) {
  using namespace tsgh;
  if (!x || !w1 || !h || !w2 || !y) return fail(ctx, TSG_E_INVALID, "mlp2_pipelined: null pointer");
  if (mode < TSG_MODE_OVERLAP || mode > TSG_MODE_COMM_ONLY) return fail(ctx, TSG_E_INVALID, "bad mode");
  if (mode == TSG_MODE_COMM_ONLY)
    return fail(ctx, TSG_E_UNSUPPORTED, "mlp2_pipelined has no communication-only part");
  if (M < 1 || K1 < 8 || N1 < 8 || N2 < 8 || K1 % 8 || N1 % 8 || N2 % 8)
    return fail(ctx, TSG_E_SHAPE, "mlp2_pipelined: bad shape M=%d K1=%d N1=%d N2=%d", M, K1, N1, N2);
  if (!aligned16(x) || !aligned16(w1) || !aligned16(h) || !aligned16(w2) || !aligned16(y))
    return fail(ctx, TSG_E_ALIGN, "mlp2_pipelined: pointers must be 16-byte aligned");
  if ((int64_t)M * K1 * 2 >= (int64_t(1) << 32) || (int64_t)M * N1 * 2 >= (int64_t(1) << 32) ||
      (int64_t)K1 * N1 * 2 >= (int64_t(1) << 32) || (int64_t)N1 * N2 * 2 >= (int64_t(1) << 32))
    return fail(ctx, TSG_E_UNSUPPORTED, "operands of 4 GiB or more are not supported");
  const int n_rb = (M + kRowBlock - 1) / kRowBlock;
  if (n_rb > kMaxRowBlocks) return fail(ctx, TSG_E_UNSUPPORTED, "M exceeds %d rows", kMaxRowBlocks * kRowBlock);

  const Opts o = resolve(opts, 64);
  const int tile1 = o.tile ? o.tile : 5;  // 128 x 256 for GEMM1
  const int tile2 = o.tile ? o.tile : 1;  // 256 x 256 for GEMM2
  const TileShape s1 = shape_of(tile1), s2 = shape_of(tile2);
  if (!s1.bm || !s2.bm) return fail(ctx, TSG_E_INVALID, "tile id %d is not available for mlp2_pipelined", o.tile);

  TSG_HIP(ctx, hipSetDevice(ctx->device));
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);

  const int n_mt1 = (M + s1.bm - 1) / s1.bm, n_nt1 = (N1 + s1.bn - 1) / s1.bn;
  const int n_mt2 = (M + s2.bm - 1) / s2.bm, n_nt2 = (N2 + s2.bn - 1) / s2.bn;
  Mlp1Args a1;
  a1.x = (const uint16_t*)x;
  a1.w1 = (const uint16_t*)w1;
  a1.h = (uint16_t*)h;
  a1.sig = ctx->d_sig + kSigBase;
  a1.cnt = ctx->d_cnt + kSigBase;
  a1.sa = sync_args(ctx, o);
  a1.tl = timeline(ctx, o);
  a1.M = M;
  a1.K1 = K1;
  a1.N1 = N1;
  a1.n_tiles_n = n_nt1;
  a1.arrivals = (uint32_t)n_nt1;
  a1.skip_mask = o.skip_mask;
  Mlp2Args a2;
  a2.h = (const uint16_t*)h;
  a2.w2 = (const uint16_t*)w2;
  a2.y = y;
  a2.sig = a1.sig;
  a2.sa = a1.sa;
  a2.tl = a1.tl;
  a2.M = M;
  a2.N1 = N1;
  a2.N2 = N2;
  a2.n_tiles_n = n_nt2;
  a2.n_tiles = n_mt2 * n_nt2;
  a2.arrivals = (uint32_t)n_nt1;
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  auto gemm1 = [&](hipStream_t s, int cus) -> tsg_status {
    a1.per_xcd = cus / 8;
    time_begin(ctx, 0, s);
    hipError_t e = launch1(tile1, a1, n_mt1 * n_nt1, s);
    time_end(ctx, 0, s);
    return e == hipSuccess ? TSG_OK : hip_fail(ctx, e, "mlp_gemm1_kernel");
  };
  auto gemm2 = [&](hipStream_t s, int nwg, int wait) -> tsg_status {
    a2.wait = wait;
    time_begin(ctx, 1, s);
    hipError_t e = launch2(tile2, a2, std::max(1, std::min(nwg, a2.n_tiles)), s);
    time_end(ctx, 1, s);
    return e == hipSuccess ? TSG_OK : hip_fail(ctx, e, "mlp_gemm2_kernel");
  };

  tsg_status st = TSG_OK;
  if (mode == TSG_MODE_SERIAL || mode == TSG_MODE_COMPUTE_ONLY) {
    st = gemm1(caller, ctx->n_cus);
    if (st == TSG_OK) st = gemm2(caller, a2.n_tiles, mode == TSG_MODE_SERIAL ? 1 : 0);
    return st;
  }
  Pair pr;
  st = streams(ctx, o, &pr);
  if (st != TSG_OK) return st;
  // The consumer is persistent with one workgroup per CU of its partition
  // (64 in shared mode), so waiting consumer workgroups can never occupy the
  // whole GPU.
  const int nwg2 = o.aux_cus < 0 ? 64 : pr.aux_cus;
  st = fork(ctx, caller, pr);
  if (st != TSG_OK) return st;
  st = gemm1(pr.main, pr.main_cus);
  if (st == TSG_OK) st = gemm2(pr.aux, nwg2, 1);
  tsg_status sj = join(ctx, caller, pr);
  return st != TSG_OK ? st : sj;
}
