// AllGather + gather + grouped GEMM: the gather side of a tensor-parallel
// MoE layer at one rank's share.
//
// "TileLink: Generating Efficient Compute-Communication Overlapping Kernels
// using Tile-Centric Primitives", section 5 (AllGather + MoE: dynamic routing
// decides which tokens every tile needs, so the shape, rank and channel
// mappings of a tile are lookup tables filled at run time, and the tile's
// loads gather its tokens through them), section 7.2 (MoE layer, first
// part: AG + Gather + GroupGEMM) and section 4.1 (dynamic mapping).
// "Triton-distributed: Programming Overlapping Kernels on Distributed AI
// Systems with the Triton Compiler", section 3.2, Algorithm 2 (pull-mode
// AllGather: the local chunk first, then one copy and one signal per peer).
//
// The T tokens are sharded over R ranks along T (chunk c = tokens
// [c T/R, (c+1) T/R) of rank c).  One call:
//   1. moe_count_kernel / moe_place_kernel (shared with the expert-compute
//      path): expert_counts, sorted_ids and the padded row tables, plus the
//      rank mask of every row block (bit c: a row of the block gathers a
//      token of chunk c) -- the dynamic rank mapping f_R of the block.
//   2. moe_rb_order_kernel (one workgroup): orders the row blocks by the
//      arrival position of the last chunk they need (stable), so tiles
//      whose tokens arrive first run first -- the tile order follows the
//      arrival order, as in the AllGather GEMM's swizzle, but read from the
//      runtime tables.
//   3. moe_ag_kernel (persistent, per-XCD phased queues): first the copy
//      units that stand in for the peers' arrival (the AllGather copy's
//      units: column slabs of each chunk, the local chunk first, counted
//      signals), then the up tiles in that order, all column tiles of a row
//      block together; each XCD takes a contiguous share of the tiles, so
//      the column tiles of a row block, which gather the same tokens, and
//      the blocks of one expert, which read the same weights, meet in its
//      L2.  A tile waits for every slab signal
//      of every chunk in its block's rank mask, gathers its tokens' rows of
//      x_full through the row -> token table, multiplies them by w_up[e]
//      (bf16 MFMA, fp32 accumulation), applies SiLU and stores bf16 rows to
//      h in pair order through the row -> pair table.  Copy units never
//      wait, and a workgroup reaches the tiles only once every copy unit
//      has been taken by a running workgroup: the queues always drain.
#include "tsg_copy.hpp"
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"
#include "tsg_moe_route.hpp"

using namespace tsg;

namespace {

constexpr int BM = 256;  // row block: tile rows and the per-expert padding unit
constexpr int BN = 224;
constexpr int kMaxRowBlocks = 4096;
static_assert(kMaxRowBlocks <= kRouteMaskBlocks, "the placement kernel gathers every block's rank mask in LDS");
constexpr size_t kSigBase = size_t(1) << 17;  // chunk slab signals in the context's pool
constexpr size_t kSigCap = size_t(1) << 16;
constexpr int kQueueSlot = 96;                // 2 phases x 8 XCD tickets, exit counter

// Main path (H a multiple of 128): 16x16x32 fragments, four by two waves of
// 64 x 112; otherwise the register-staged path with 32x32x16 fragments,
// eight waves of 32 x 224.
template <bool DIRECT>
using CfgOf = std::conditional_t<DIRECT, TileCfg<BM, BN, 4, 2, 16>, TileCfg<BM, BN, 8, 1>>;
constexpr int kThreads = CfgOf<true>::NT;
static_assert(CfgOf<false>::NT == kThreads, "both paths use one workgroup size");

struct Layout {
  size_t meta, offs, poffs, rb_expert, row_pair, row_token, pair_row, blk, rb_mask, rb_order, total;
  int64_t n_rb_max, rows_max, G;
};

inline size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

Layout layout(int64_t T, int64_t E, int64_t k) {
  Layout L;
  const int64_t pairs = T * k;
  L.n_rb_max = (pairs + E * (BM - 1) + BM - 1) / BM;
  L.rows_max = L.n_rb_max * BM;
  L.G = (pairs + 255) / 256;
  size_t o = 0;
  L.meta = o;      o += up256(64 * 4);
  L.offs = o;      o += up256((E + 1) * 4);
  L.poffs = o;     o += up256((E + 1) * 4);
  L.rb_expert = o; o += up256(L.n_rb_max * 4);
  L.row_pair = o;  o += up256(L.rows_max * 4);
  L.row_token = o; o += up256(L.rows_max * 4);
  L.pair_row = o;  o += up256(pairs * 4);
  L.blk = o;       o += up256(L.G * E * 4);
  L.rb_mask = o;   o += up256(L.n_rb_max * 4);
  L.rb_order = o;  o += up256(L.n_rb_max * 4);
  L.total = o;
  return L;
}

struct AgMoeArgs {
  const uint16_t* x_full;
  const uint16_t* w_up;
  uint16_t* h;
  MoeTables tab;
  const uint32_t* rb_mask;
  const int* rb_order;
  const uint64_t* sig;    // slab signals of the chunks, c * n_slab + s
  uint32_t* queue;        // 2 phases x 8 XCD ticket counters, exit counter (zero between calls)
  SyncArgs sa;
  Timeline tl;
  CopyArgs copy;
  int n_copy;             // copy units at the head of the queue (0: no copy)
  int n_tiles;            // row blocks (at most n_rb_max) x column tiles
  int n_nt;
  int H, I;
  int n_slab;
  int wait;
  int l1_only;            // x_full slabs are whole 128-byte lines
};

template <bool DIRECT>
__global__ void __launch_bounds__(kThreads) moe_ag_kernel(const AgMoeArgs a) {
  using Cfg = CfgOf<DIRECT>;
  __shared__ __attribute__((aligned(16))) char lds[DIRECT ? Cfg::LDS_DIRECT : Cfg::LDS_REGS];
  const int n_rb = __builtin_amdgcn_readfirstlane(a.tab.meta[0]);
  // tiles of the row blocks in use (n_tiles is the bound for n_rb_max blocks)
  const int n_ph[2] = {a.n_copy, a.n_tiles > 0 ? min(n_rb * a.n_nt, a.n_tiles) : 0};
  const int my_xcd = xcd_id();
  int phase = 0;
  // Next item, identical in every thread: wave 0 claims it and passes it on
  // through the first words of the tile buffer, which are free between items
  // (a tile's last LDS access precedes a barrier: the K loop's last one, or
  // the staged epilogue's wave-local reads, which wave 0 finishes before
  // its lane 0 writes).
  auto fetch = [&]() -> QueueItem {
    volatile int* s_item = (volatile int*)lds;
    if (threadIdx.x < 64) {
      const QueueItem it = xcd_queue_claim<2>(a.queue, n_ph, my_xcd, phase);
      if (threadIdx.x == 0) {
        s_item[0] = it.phase;
        s_item[1] = it.index;
      }
    }
    __syncthreads();
    const QueueItem it{__builtin_amdgcn_readfirstlane(s_item[0]), __builtin_amdgcn_readfirstlane(s_item[1])};
    __syncthreads();
    return it;
  };
  for (QueueItem it = fetch(); it.phase >= 0; it = fetch()) {
    phase = it.phase;
    if (it.phase == 0) {
      copy_unit<kThreads>(a.copy, it.index);
      __syncthreads();
    } else {
      const int ti = it.index;
      const int ord = ti / a.n_nt, nt = ti - ord * a.n_nt;
      if (ord < n_rb) {
        const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
        const int rb = __builtin_amdgcn_readfirstlane(a.rb_order[ord]);
        const int e = __builtin_amdgcn_readfirstlane(a.tab.rb_expert[rb]);
        if (a.wait) {
          // dynamic rank mapping: the chunks this block's tokens come from
          uint32_t m = __builtin_amdgcn_readfirstlane(a.rb_mask[rb]);
          const uint64_t target = sig_target(a.sa.epoch, 1);
          while (m) {
            const int c = (int)__builtin_ctz(m);
            m &= m - 1;
            for (int s = 0; s < a.n_slab; ++s) block_poll_ge(a.sig + (size_t)c * a.n_slab + s, target, a.sa);
          }
          acquire_lines(a.l1_only != 0);
        }
        const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
        const int col0 = nt * BN;
        typename GemmTile<Cfg>::Acc acc;
        // padding rows read the block's first row, a token the tile waited for
        const int first = __builtin_amdgcn_readfirstlane(a.tab.row_token[(int64_t)rb * BM]);
        const ARowsGather ar{a.x_full, a.H, a.tab.row_token + (int64_t)rb * BM, first};
        const uint16_t* B = a.w_up + (int64_t)e * a.H * a.I;
        // rows past the expert's last pair are padding (whole waves of them
        // skip their matrix work)
        const int valid = __builtin_amdgcn_readfirstlane(
            min(BM, a.tab.offs[e + 1] - a.tab.offs[e] - (rb * BM - a.tab.poffs[e])));
        if (DIRECT)
          GemmTile<Cfg>::run_direct(ar, B, a.I, col0, a.I, a.H, lds, acc, NoHook(), valid);
        else
          GemmTile<Cfg>::run_regs(ar, B, a.I, col0, a.I, a.H, lds, acc);
        // h[pair] = bf16(SiLU(u)), SiLU(u) = u / (1 + e^-u), rows scattered
        // to pair order (padding rows have no pair and are not stored)
        GemmTile<Cfg>::template store_bf16_rows<sizeof(lds)>(
            acc, lds, a.h + col0, a.I, a.tab.row_pair + (int64_t)rb * BM, a.I - col0,
            [](float u) { return u / (1.0f + expf(-u)); });
        if (a.tl.buf && threadIdx.x == 0) timeline_put(a.tl, 10, (uint32_t)(rb << 16 | nt), t0, t1, wall_clock64());
        __syncthreads();  // staging region read back before the next item
      }
    }
  }
  // the last workgroup to leave resets the ticket and exit counters
  if (threadIdx.x == 0 && atomicAdd(a.queue + 16, 1u) == gridDim.x - 1)
    for (int i = 0; i <= 16; ++i) __hip_atomic_store(a.queue + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t tsg_moe_ag_workspace(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  if (T < 1 || H < 8 || I < 8 || E < 1 || E > kMaxExperts || k != 2) return 0;
  return layout(T, E, k).total;
}

tsg_status tsg_op_moe_ag(tsg_ctx* ctx, const void* x_local, const void* x_peers, void* x_full,
                         const int32_t* topk_ids, const void* w_up, void* h, int32_t* expert_counts,
                         int32_t* sorted_ids, void* workspace, size_t workspace_bytes, int T, int H, int I,
                         int E, int k, int R, int rank, const int* arrival_order, const tsg_opts* opts,
                         int mode, void* stream) {
  using namespace tsgh;
  if (!x_local || !x_full || !topk_ids || !w_up || !h || !expert_counts || !sorted_ids || (R > 1 && !x_peers))
    return fail(ctx, TSG_E_INVALID, "moe_ag_group_gemm: null pointer");
  if (mode < TSG_MODE_OVERLAP || mode > TSG_MODE_COMM_ONLY) return fail(ctx, TSG_E_INVALID, "bad mode");
  if (k != 2) return fail(ctx, TSG_E_UNSUPPORTED, "moe_ag_group_gemm supports k == 2 only");
  if (R < 1 || R > kMaxRanks || rank < 0 || rank >= R)
    return fail(ctx, TSG_E_SHAPE, "need 1 <= R <= %d and 0 <= rank < R", kMaxRanks);
  if (T < R || T % R || E < 1 || E > kMaxExperts || H < 8 || I < 8 || H % 8 || I % 8)
    return fail(ctx, TSG_E_SHAPE, "moe_ag_group_gemm: bad shape T=%d H=%d I=%d E=%d R=%d", T, H, I, E, R);
  if ((int64_t)T * k > 65535)
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_ag_group_gemm: T * k above 65535 routed pairs");
  if (!aligned16(x_local) || (x_peers && !aligned16(x_peers)) || !aligned16(x_full) || !aligned16(topk_ids) ||
      !aligned16(w_up) || !aligned16(h) || !aligned16(workspace))
    return fail(ctx, TSG_E_ALIGN, "moe_ag_group_gemm: pointers must be 16-byte aligned");
  const Layout L = layout(T, E, k);
  if (!workspace || workspace_bytes < L.total)
    return fail(ctx, TSG_E_WORKSPACE, "workspace of %zu bytes needed", L.total);
  if (L.n_rb_max > kMaxRowBlocks)
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_ag_group_gemm: more than %d row blocks", kMaxRowBlocks);
  if ((int64_t)T * H * 2 >= (int64_t(1) << 31) || (int64_t)H * I * 2 >= (int64_t(1) << 32))
    return fail(ctx, TSG_E_UNSUPPORTED, "operands of 2 GiB or more are not supported");

  // arrival order: the local chunk first ([TD] Algorithm 2), then the given
  // peers (or the ring rank+1, rank+2, ...)
  int pos_of[kMaxRanks];
  ChunkOrder co;
  for (int i = 0; i < kMaxRanks; ++i) {
    pos_of[i] = -1;
    co.chunk[i] = 0;
  }
  co.chunk[0] = (int8_t)rank;
  pos_of[rank] = 0;
  for (int p = 1; p < R; ++p) {
    const int cc = arrival_order ? arrival_order[p - 1] : (rank + p) % R;
    if (cc < 0 || cc >= R || pos_of[cc] >= 0)
      return fail(ctx, TSG_E_INVALID, "arrival_order must be a permutation of the peer ranks");
    co.chunk[p] = (int8_t)cc;
    pos_of[cc] = p;
  }

  const Opts o = resolve(opts, -1);
  if (o.aux_cus > 0) return fail(ctx, TSG_E_UNSUPPORTED, "moe_ag_group_gemm runs on shared CUs only");
  int slab = o.comm_tile ? o.comm_tile : 2048;
  if (slab < 64 || (slab & (slab - 1)))
    return fail(ctx, TSG_E_INVALID, "comm_tile must be a power of two >= 64 (got %d)", slab);
  int k_pow2 = 64;
  while (k_pow2 < H) k_pow2 *= 2;
  slab = std::min(std::min(slab, k_pow2), 2048);
  int slab_log2 = 0;
  while ((1 << slab_log2) < slab) ++slab_log2;
  const int n_slab = (H + slab - 1) / slab;
  if ((size_t)R * n_slab > kSigCap) return fail(ctx, TSG_E_UNSUPPORTED, "too many chunk signals");
  const int chunk_rows = T / R;
  const int nwg = ctx->n_cus;
  int np[kHead + 1], ustart[kHead + 1];
  int64_t n_units = 0;
  if (!copy_plan(R, 1, chunk_rows, H, n_slab, slab_log2 - 3, nwg, np, ustart, &n_units))
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_ag_group_gemm: the copy's offsets would overflow");

  TSG_HIP(ctx, hipSetDevice(ctx->device));
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);
  const SyncArgs sa = sync_args(ctx, o);
  const Timeline tl = timeline(ctx, o);
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  char* base = (char*)workspace;
  MoeTables tab;
  tab.meta = (int*)(base + L.meta);
  tab.offs = (int*)(base + L.offs);
  tab.poffs = (int*)(base + L.poffs);
  tab.rb_expert = (int*)(base + L.rb_expert);
  tab.row_pair = (int*)(base + L.row_pair);
  tab.row_token = (int*)(base + L.row_token);
  tab.pair_row = (int*)(base + L.pair_row);
  uint32_t* rb_mask = (uint32_t*)(base + L.rb_mask);
  int* rb_order = (int*)(base + L.rb_order);

  RouteArgs ra;
  ra.ids = topk_ids;
  ra.counts = expert_counts;
  ra.sorted_ids = sorted_ids;
  ra.ws = tab;
  ra.blk = (int*)(base + L.blk);
  ra.status = ctx->d_status;
  ra.P = T * k;
  ra.E = E;
  ra.k = k;
  ra.G = (int)L.G;
  ra.rows_max = L.rows_max;
  ra.n_rb_max = L.n_rb_max;
  ra.rb_mask = rb_mask;
  ra.tokens_per_rank = chunk_rows;

  RbOrderArgs oa;
  oa.meta = tab.meta;
  oa.rb_mask = rb_mask;
  oa.rb_order = rb_order;
  for (int i = 0; i < kRouteMaxRanks; ++i) oa.key_of[i] = i < kMaxRanks && pos_of[i] >= 0 ? pos_of[i] : 0;
  oa.min_key = 0;
  oa.R = R;

  CopyArgs ca;
  ca.a_local = (const u32x4_t*)x_local;
  ca.a_peers = (const u32x4_t*)x_peers;
  ca.a_full = (u32x4_t*)x_full;
  ca.sig = ctx->d_sig + kSigBase;
  ca.cnt = ctx->d_cnt + kSigBase;
  ca.sa = sa;
  ca.tl = tl;  // copy units: kind 1
  ca.ord = co;
  ca.k8 = H / 8;
  ca.chunk_rows = chunk_rows;
  ca.R = R;
  ca.rank = rank;
  ca.C = 1;
  ca.ch_rows = chunk_rows;
  ca.n_slab = n_slab;
  ca.vpr_log2 = slab_log2 - 3;
  for (int i = 0; i <= kHead; ++i) {
    ca.np[i] = np[i];
    ca.ustart[i] = ustart[i];
  }
  ca.n_units = (int)n_units;
  ca.skip_mask = o.skip_mask;
  ca.queue = nullptr;  // not used: units come from the kernel's own queues
  ca.n_workers = 0;
  ca.pace_word = nullptr;
  ca.pace_ticks = 0.f;
  ca.unit_base = 0;

  AgMoeArgs ka;
  ka.x_full = (const uint16_t*)x_full;
  ka.w_up = (const uint16_t*)w_up;
  ka.h = (uint16_t*)h;
  ka.tab = tab;
  ka.rb_mask = rb_mask;
  ka.rb_order = rb_order;
  ka.sig = ctx->d_sig + kSigBase;
  ka.queue = ctx->d_queue + kQueueSlot;
  ka.sa = sa;
  ka.tl = tl;
  ka.copy = ca;
  ka.n_nt = (I + BN - 1) / BN;
  ka.H = H;
  ka.I = I;
  ka.n_slab = n_slab;
  ka.l1_only = ((uintptr_t)x_full % 128 == 0 && H % 64 == 0 && slab >= 64) ? 1 : 0;
  const bool direct = H % (2 * CfgOf<true>::BK) == 0;

  auto launch = [&](int n_copy, int n_tiles, int wait, int which) -> tsg_status {
    ka.n_copy = n_copy;
    ka.n_tiles = n_tiles;
    ka.wait = wait;
    time_begin(ctx, which, caller);
    if (direct)
      hipLaunchKernelGGL(moe_ag_kernel<true>, dim3(nwg), dim3(kThreads), 0, caller, ka);
    else
      hipLaunchKernelGGL(moe_ag_kernel<false>, dim3(nwg), dim3(kThreads), 0, caller, ka);
    time_end(ctx, which, caller);
    return check_launch(ctx, "moe_ag_kernel");
  };
  const int n_tiles = (int)L.n_rb_max * ka.n_nt;
  if (mode != TSG_MODE_COMM_ONLY) {
    hipLaunchKernelGGL(moe_count_kernel<BM>, dim3(ra.G), dim3(256), 0, caller, ra);
    tsg_status st = check_launch(ctx, "moe_count_kernel");
    if (st != TSG_OK) return st;
    hipLaunchKernelGGL(moe_place_kernel<BM>, dim3(ra.G), dim3(256), 0, caller, ra);
    if ((st = check_launch(ctx, "moe_place_kernel")) != TSG_OK) return st;
    hipLaunchKernelGGL(moe_rb_order_kernel<>, dim3(1), dim3(256), 0, caller, oa);
    if ((st = check_launch(ctx, "moe_rb_order_kernel")) != TSG_OK) return st;
  }
  switch (mode) {
    case TSG_MODE_OVERLAP: return launch((int)n_units, n_tiles, 1, 0);
    case TSG_MODE_SERIAL: {
      tsg_status st = launch((int)n_units, 0, 0, 1);
      return st != TSG_OK ? st : launch(0, n_tiles, 1, 0);
    }
    case TSG_MODE_COMPUTE_ONLY: return launch(0, n_tiles, 0, 0);
    default: return launch((int)n_units, 0, 0, 1);
  }
}
