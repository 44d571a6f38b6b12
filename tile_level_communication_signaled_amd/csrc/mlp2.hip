// CTA-pipelined two-GEMM MLP on one GPU.
//
// Digest page "Resource-aware Computation-Communication Overlap for
// multi-GPU ML Workloads" (CTA-pipelining abstract): a dependent kernel runs
// concurrently with its producer, each of its CTAs starting as soon as the
// producer CTAs it depends on are done; shown on a 2-layer GEMM that stands
// for the MLP.  Here both GEMMs run on one GPU:
//
//   GEMM1 (producer): H = bf16(GELU(X W1)), tiles visited row block by row
//     block (by default; a grouped order is an option).  After storing a
//     tile, one lane arrives on the signal of each 128-row block the tile
//     covers ("TileLink: Generating Efficient
//     Compute-Communication Overlapping Kernels using Tile-Centric Primitives",
//     Table 3: a consumer tile is ready once all the producer tiles it depends
//     on are done -- here the N1 / BN1 tiles of that row block).
//   GEMM2 (consumer, persistent): Y = H W2 in fp32; each tile first acquires
//     the signals of the row blocks it reads, then runs its K loop over H.
//
// GELU is the exact form 0.5 z (1 + erf(z / sqrt 2)) on the fp32 accumulator
// (erff of the device math library), rounded to bf16 (nearest even): H is the
// bf16 operand of GEMM2.  By default (shared CUs) both layers run in one
// persistent kernel fed by a ticket queue (mlp_fused_kernel); with a CU
// split the two kernels run concurrently on disjoint CU sets, GEMM2 as a
// persistent consumer.
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"

using namespace tsg;

namespace {

constexpr size_t kSigBase = 64;     // row-block signals of MLP2 in the context's pool
constexpr int kRowBlock = 128;
constexpr int kMaxRowBlocks = 4000;

// GELU, exact form, on the fp32 accumulator: 0.5 z (1 + erf(z / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

struct Mlp1Args {
  const uint16_t* x;
  const uint16_t* w1;
  uint16_t* h;
  uint64_t* sig;
  uint32_t* cnt;
  SyncArgs sa;
  Timeline tl;
  int M, K1, N1;
  int n_tiles_n, n_tiles_m;
  int group;              // tile rows per group of the grouped order
  int per_xcd;
  uint32_t arrivals;      // GEMM1 tiles per row block (= n_tiles_n)
  uint32_t skip_mask;     // row blocks whose signal is never completed (test hook)
};

template <class Cfg, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) mlp_gemm1_kernel(const Mlp1Args a) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  const int t = xcd_remap(blockIdx.x, gridDim.x, a.per_xcd);
  int mt, nt;
  grouped_tile(t, a.n_tiles_m, a.n_tiles_n, a.group, mt, nt);
  const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
  const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
  typename GemmTile<Cfg>::Acc acc;
  const ARowsLinear ar{a.x, a.K1, row0, a.M};
  if (DIRECT)
    GemmTile<Cfg>::run_direct(ar, a.w1, a.N1, col0, a.N1, a.K1, lds, acc);
  else
    GemmTile<Cfg>::run_regs(ar, a.w1, a.N1, col0, a.N1, a.K1, lds, acc);
  GemmTile<Cfg>::template store_bf16_staged<sizeof(lds), true>(
      acc, lds, a.h + (int64_t)row0 * a.N1 + col0, a.N1, a.M - row0, a.N1 - col0, gelu_erf);
  block_coherent_complete();
  if (threadIdx.x == 0) {
    for (int b = row0 / kRowBlock; b * kRowBlock < min(row0 + Cfg::BM, a.M); ++b) {
      if ((a.skip_mask >> (b & 31)) & 1u) continue;
      sig_arrive_counted_coherent(a.cnt + b, a.sig + b, a.arrivals, a.sa.epoch);
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
  int group;              // tile rows per group of the grouped order
  int per_xcd;            // consecutive tiles per XCD (0: no remap)
  int wait;
  int l1_only;            // H rows are whole 128-byte lines: acquire invalidates L1 only
  uint32_t arrivals;
};

// Persistent: workgroup g computes tiles g, g + G, ... of the tile order
// (row-block-major by default, so the first tiles need the first row blocks
// GEMM1 completes).
template <class Cfg, bool DIRECT>
__global__ void __launch_bounds__(Cfg::NT) mlp_gemm2_kernel(const Mlp2Args a) {
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  for (int tp = blockIdx.x; tp < a.n_tiles; tp += gridDim.x) {
    // with a grid that is a multiple of 8, index tp runs on XCD tp mod 8
    const int t = xcd_remap(tp, a.n_tiles, a.per_xcd);
    int mt, nt;
    grouped_tile(t, a.n_tiles / a.n_tiles_n, a.n_tiles_n, a.group, mt, nt);
    const int row0 = mt * Cfg::BM, col0 = nt * Cfg::BN;
    const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
    if (a.wait) {
      const uint64_t target = sig_target(a.sa.epoch, a.arrivals);
      for (int b = row0 / kRowBlock; b * kRowBlock < min(row0 + Cfg::BM, a.M); ++b)
        block_poll_ge(a.sig + b, target, a.sa);
      acquire_lines(a.l1_only);
    }
    const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
    typename GemmTile<Cfg>::Acc acc;
    const ARowsLinear ar{a.h, a.N1, row0, a.M};
    if (DIRECT)
      GemmTile<Cfg>::run_direct(ar, a.w2, a.N2, col0, a.N2, a.N1, lds, acc);
    else
      GemmTile<Cfg>::run_regs(ar, a.w2, a.N2, col0, a.N2, a.N1, lds, acc);
    GemmTile<Cfg>::template store_f32<false>(acc, a.y + (int64_t)row0 * a.N2 + col0, a.N2, a.M - row0, a.N2 - col0);
    if (a.tl.buf && threadIdx.x == 0) timeline_put(a.tl, 6, (uint32_t)(mt << 16 | nt), t0, t1, wall_clock64());
    __syncthreads();  // LDS of this tile fully consumed before the next one
  }
}

// Both GEMMs in one persistent kernel (overlap mode on shared CUs).
// Items are GEMM1 tiles (phase 1), then GEMM2 tiles (phase 2), each set in
// the op's tile order and cut into 8 contiguous shares, one per XCD (with the
// grouped order the tiles an XCD runs form a compact block of the tile grid
// whose operands its L2 can reuse).  A workgroup reads its XCD (XCC_ID) and takes tickets
// from its XCD's phase-1 queue, then from the other XCDs' phase-1 queues,
// and only then from the phase-2 queues, its own first.  A GEMM2 tile
// acquires the signals of its row blocks before its K loop.  No item waits
// for a later one, and a workgroup takes a phase-2 item only once every
// phase-1 item has been taken by a running workgroup that never waits, so the
// queues always drain.  The last workgroup to leave resets the counters.
struct MlpFusedArgs {
  Mlp1Args g1;
  Mlp2Args g2;
  uint32_t* queues;  // 2 phases x 8 XCD ticket counters, then an exit counter
  int n_items1;      // GEMM1 tiles
  int n_items2;      // GEMM2 tiles
  int n_mt2;         // GEMM2 tile rows
};

template <class C1, bool D1, class C2, bool D2>
__global__ void __launch_bounds__(C1::NT) mlp_fused_kernel(const MlpFusedArgs f) {
  static_assert(C1::NT == C2::NT, "both tiles use the same number of waves");
  constexpr int L1 = D1 ? C1::LDS_DIRECT : C1::LDS_REGS;
  constexpr int L2 = D2 ? C2::LDS_DIRECT : C2::LDS_REGS;
  __shared__ __attribute__((aligned(16))) char lds[L1 > L2 ? L1 : L2];
  const int my_xcd = xcd_id();
  // The ticket goes through the first word of the tile buffer, which is free
  // between items (a tile's last LDS read precedes its pipeline's final
  // barrier; the next tile writes LDS only after the second barrier here).
  // The item is made wave-uniform (readfirstlane) and the loop has a single
  // back edge through the fetch, so its barriers stay uniform.
  int phase = 0;  // phase of this workgroup's previous item (wave 0's copy)
  auto fetch = [&]() -> int {
    volatile int* s_item = (volatile int*)lds;
    if (threadIdx.x < 64) {
      const int n[2] = {f.n_items1, f.n_items2};
      const QueueItem it = xcd_queue_claim<2>(f.queues, n, my_xcd, phase);
      if (it.phase >= 0) phase = it.phase;
      if (threadIdx.x == 0) *s_item = it.phase < 0 ? -1 : (it.phase == 0 ? 0 : f.n_items1) + it.index;
    }
    __syncthreads();
    const int v = __builtin_amdgcn_readfirstlane(*s_item);
    __syncthreads();
    return v;
  };
  const Mlp1Args& a = f.g1;
  const Mlp2Args& b = f.g2;
  for (int item = fetch(); item >= 0; item = fetch()) {
    const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
    if (item < f.n_items1) {
      int mt, nt;
      grouped_tile(item, a.n_tiles_m, a.n_tiles_n, a.group, mt, nt);
      const int row0 = mt * C1::BM, col0 = nt * C1::BN;
      typename GemmTile<C1>::Acc acc;
      const ARowsLinear ar{a.x, a.K1, row0, a.M};
      if (D1)
        GemmTile<C1>::run_direct(ar, a.w1, a.N1, col0, a.N1, a.K1, lds, acc);
      else
        GemmTile<C1>::run_regs(ar, a.w1, a.N1, col0, a.N1, a.K1, lds, acc);
      GemmTile<C1>::template store_bf16_staged<sizeof(lds), true>(
          acc, lds, a.h + (int64_t)row0 * a.N1 + col0, a.N1, a.M - row0, a.N1 - col0, gelu_erf);
      block_coherent_complete();
      if (threadIdx.x == 0) {
        for (int rb = row0 / kRowBlock; rb * kRowBlock < min(row0 + C1::BM, a.M); ++rb) {
          if ((a.skip_mask >> (rb & 31)) & 1u) continue;
          sig_arrive_counted_coherent(a.cnt + rb, a.sig + rb, a.arrivals, a.sa.epoch);
        }
        if (a.tl.buf) timeline_put(a.tl, 5, (uint32_t)(mt << 16 | nt), t0, t0, wall_clock64());
      }
    } else {
      int mt, nt;
      grouped_tile(item - f.n_items1, f.n_mt2, b.n_tiles_n, b.group, mt, nt);
      const int row0 = mt * C2::BM, col0 = nt * C2::BN;
      const uint64_t target = sig_target(b.sa.epoch, b.arrivals);
      for (int rb = row0 / kRowBlock; rb * kRowBlock < min(row0 + C2::BM, b.M); ++rb)
        block_poll_ge(b.sig + rb, target, b.sa);
      acquire_lines(b.l1_only);
      const uint64_t t1 = b.tl.buf ? wall_clock64() : 0;
      typename GemmTile<C2>::Acc acc;
      const ARowsLinear ar{b.h, b.N1, row0, b.M};
      if (D2)
        GemmTile<C2>::run_direct(ar, b.w2, b.N2, col0, b.N2, b.N1, lds, acc);
      else
        GemmTile<C2>::run_regs(ar, b.w2, b.N2, col0, b.N2, b.N1, lds, acc);
      GemmTile<C2>::template store_f32<false>(acc, b.y + (int64_t)row0 * b.N2 + col0, b.N2, b.M - row0, b.N2 - col0);
      if (b.tl.buf && threadIdx.x == 0) timeline_put(b.tl, 6, (uint32_t)(mt << 16 | nt), t0, t1, wall_clock64());
    }
  }
  // last one out resets the ticket counters for the next call
  if (threadIdx.x == 0 && atomicAdd(f.queues + 16, 1u) == gridDim.x - 1)
    for (int i = 0; i <= 16; ++i) __hip_atomic_store(f.queues + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

using Cfg1 = TileCfg<256, 256, 2, 2>;
using Cfg3 = TileCfg<128, 128, 2, 2>;
using Cfg4 = TileCfg<256, 128, 2, 2>;
using Cfg5 = TileCfg<128, 256, 2, 2>;
// 16x16x32 fragments, eight waves (two per SIMD): 256 x 256 as 4 x 2 waves of
// 64 x 128, and 128 x 256 as 2 x 4 waves of 64 x 64.  Direct-to-LDS loads
// only, so the K of each GEMM must be a multiple of 128.
using Cfg6 = TileCfg<256, 256, 4, 2, 16>;
using Cfg7 = TileCfg<128, 256, 2, 4, 16>;

template <class T>
constexpr bool is_mf16() { return T::MF == 16; }

template <class C1, class C2>
hipError_t launch_fused_cfg(const MlpFusedArgs& f, int grid, hipStream_t s) {
  const bool d1 = f.g1.K1 % (2 * C1::BK) == 0, d2 = f.g2.N1 % (2 * C2::BK) == 0;
  constexpr int NT = C1::NT;
  if constexpr (is_mf16<C1>() || is_mf16<C2>()) {
    if (!d1 || !d2) return hipErrorInvalidValue;  // the host rejects these shapes first
    hipLaunchKernelGGL((mlp_fused_kernel<C1, true, C2, true>), dim3(grid), dim3(NT), 0, s, f);
  } else if (d1 && d2)
    hipLaunchKernelGGL((mlp_fused_kernel<C1, true, C2, true>), dim3(grid), dim3(NT), 0, s, f);
  else if (d1)
    hipLaunchKernelGGL((mlp_fused_kernel<C1, true, C2, false>), dim3(grid), dim3(NT), 0, s, f);
  else if (d2)
    hipLaunchKernelGGL((mlp_fused_kernel<C1, false, C2, true>), dim3(grid), dim3(NT), 0, s, f);
  else
    hipLaunchKernelGGL((mlp_fused_kernel<C1, false, C2, false>), dim3(grid), dim3(NT), 0, s, f);
  return hipGetLastError();
}

// Tile pairs the fused kernel is built for: (GEMM1 tile, GEMM2 tile).
bool fused_supported(int t1, int t2) {
  return (t1 == 5 && t2 == 1) || (t1 == 5 && t2 == 5) || (t1 == 3 && t2 == 3) || (t1 == 7 && t2 == 6) ||
         (t1 == 7 && t2 == 7);
}

hipError_t launch_fused(int t1, int t2, const MlpFusedArgs& f, int grid, hipStream_t s) {
  if (t1 == 5 && t2 == 1) return launch_fused_cfg<Cfg5, Cfg1>(f, grid, s);
  if (t1 == 5 && t2 == 5) return launch_fused_cfg<Cfg5, Cfg5>(f, grid, s);
  if (t1 == 3 && t2 == 3) return launch_fused_cfg<Cfg3, Cfg3>(f, grid, s);
  if (t1 == 7 && t2 == 6) return launch_fused_cfg<Cfg7, Cfg6>(f, grid, s);
  if (t1 == 7 && t2 == 7) return launch_fused_cfg<Cfg7, Cfg7>(f, grid, s);
  return hipErrorInvalidValue;
}

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
    case 7: return {128, 256};
    default: return {0, 0};
  }
}

template <class Cfg>
hipError_t launch1_cfg(const Mlp1Args& a, int grid, hipStream_t s) {
  if (is_mf16<Cfg>() && a.K1 % (2 * Cfg::BK)) return hipErrorInvalidValue;  // rejected by the host first
  if (a.K1 % (2 * Cfg::BK) == 0)
    hipLaunchKernelGGL((mlp_gemm1_kernel<Cfg, true>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  else
    hipLaunchKernelGGL((mlp_gemm1_kernel<Cfg, false>), dim3(grid), dim3(Cfg::NT), 0, s, a);
  return hipGetLastError();
}

template <class Cfg>
hipError_t launch2_cfg(const Mlp2Args& a, int grid, hipStream_t s) {
  if (is_mf16<Cfg>() && a.N1 % (2 * Cfg::BK)) return hipErrorInvalidValue;  // rejected by the host first
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
    case 6: return launch1_cfg<Cfg6>(a, grid, s);
    case 7: return launch1_cfg<Cfg7>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch2(int id, const Mlp2Args& a, int grid, hipStream_t s) {
  switch (id) {
    case 1: return launch2_cfg<Cfg1>(a, grid, s);
    case 3: return launch2_cfg<Cfg3>(a, grid, s);
    case 4: return launch2_cfg<Cfg4>(a, grid, s);
    case 5: return launch2_cfg<Cfg5>(a, grid, s);
    case 6: return launch2_cfg<Cfg6>(a, grid, s);
    case 7: return launch2_cfg<Cfg7>(a, grid, s);
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

  const Opts o = resolve(opts, -1);
  const bool small = M < 1024 || N1 < 1024 || N2 < 1024;
  // Tile 6 names a pair of eight-wave tiles on 16x16x32 fragments: 128 x 256
  // (2 x 4 waves) for GEMM1 and 256 x 256 (4 x 2 waves) for GEMM2.  It is the
  // default when both K dimensions allow direct-to-LDS loads; otherwise
  // GEMM1 takes 128 x 256 and GEMM2 256 x 256 on four waves of 32x32x16.
  const bool eight = !small && K1 % 128 == 0 && N1 % 128 == 0;
  const int tile1 = o.tile == 6 ? 7 : o.tile ? o.tile : small ? 3 : eight ? 7 : 5;
  const int tile2 = o.tile ? o.tile : small ? 3 : eight ? 6 : 1;
  if (o.order != 0 && o.order != 1) return fail(ctx, TSG_E_INVALID, "mlp2_pipelined: order must be 0 or 1");
  // Tile order of both GEMMs: 0 = row-block-major (a GEMM2 tile needs whole
  // row blocks of H, so GEMM1 finishes them one after another and GEMM2's
  // first tiles read the first ones); 1 = groups of 8 tile rows walked
  // column by column, which keeps an XCD's operands in its L2 when all
  // tiles run at once.
  const int group = o.order == 1 ? 8 : 1;
  const TileShape s1 = shape_of(tile1), s2 = shape_of(tile2);
  if (!s1.bm || !s2.bm) return fail(ctx, TSG_E_INVALID, "tile id %d is not available for mlp2_pipelined", o.tile);
  if ((tile1 >= 6 && K1 % 128) || (tile2 >= 6 && N1 % 128))
    return fail(ctx, TSG_E_UNSUPPORTED, "tile %d needs K1 and N1 multiples of 128 (direct-to-LDS loads only)", o.tile);

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
  a1.n_tiles_m = n_mt1;
  a1.group = group;
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
  a2.group = group;
  a2.arrivals = (uint32_t)n_nt1;
  a2.l1_only = ((uintptr_t)h % 128 == 0 && ((int64_t)N1 * 2) % 128 == 0) ? 1 : 0;
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
    nwg = std::max(1, std::min(nwg, a2.n_tiles));
    a2.per_xcd = nwg % 8 == 0 ? nwg / 8 : 0;
    time_begin(ctx, 1, s);
    hipError_t e = launch2(tile2, a2, nwg, s);
    time_end(ctx, 1, s);
    return e == hipSuccess ? TSG_OK : hip_fail(ctx, e, "mlp_gemm2_kernel");
  };

  tsg_status st = TSG_OK;
  if (mode == TSG_MODE_SERIAL || mode == TSG_MODE_COMPUTE_ONLY) {
    st = gemm1(caller, ctx->n_cus);
    if (st == TSG_OK) st = gemm2(caller, a2.n_tiles, mode == TSG_MODE_SERIAL ? 1 : 0);
    return st;
  }
  if (o.aux_cus < 0 && fused_supported(tile1, tile2)) {
    // Shared CUs: both layers in one persistent kernel on the caller's stream.
    MlpFusedArgs f;
    f.g1 = a1;
    f.g2 = a2;
    f.g2.wait = 1;
    f.g2.per_xcd = 0;
    f.g1.per_xcd = 0;
    f.n_items1 = n_mt1 * n_nt1;
    f.n_items2 = a2.n_tiles;
    f.n_mt2 = n_mt2;
    const int nwg = o.aux_wgs > 0 ? o.aux_wgs : ctx->n_cus;
    f.queues = ctx->d_queue + 16;
    time_begin(ctx, 0, caller);
    hipError_t e = launch_fused(tile1, tile2, f, nwg, caller);
    time_end(ctx, 0, caller);
    return e == hipSuccess ? TSG_OK : hip_fail(ctx, e, "mlp_fused_kernel");
  }
  Pair pr;
  st = streams(ctx, o, &pr);
  if (st != TSG_OK) return st;
  // The consumer is persistent with one workgroup per CU of its partition
  // (64 in shared mode), so waiting consumer workgroups can never occupy the
  // whole GPU.
  const int nwg2 = o.aux_wgs > 0 ? o.aux_wgs : (o.aux_cus < 0 ? 64 : pr.aux_cus);
  st = fork(ctx, caller, pr);
  if (st != TSG_OK) return st;
  st = gemm1(pr.main, pr.main_cus);
  if (st == TSG_OK) st = gemm2(pr.aux, nwg2, 1);
  tsg_status sj = join(ctx, caller, pr);
  return st != TSG_OK ? st : sj;
}
