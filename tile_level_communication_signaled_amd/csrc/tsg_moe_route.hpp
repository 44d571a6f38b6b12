// Routing bookkeeping of the MoE paths: a stable counting sort of the
// routed pairs by expert and the lookup tables of the padded row layout
// ("TileLink: Generating Efficient Compute-Communication Overlapping Kernels
// using Tile-Centric Primitives", section 4.1, dynamic mapping: lookup
// tables filled at run time from the routing, mapping a row tile to its
// expert and rows, and rows to tokens).  Shared by the expert-compute +
// combine path and the AllGather + gather + grouped-GEMM path.
#pragma once

#include "tsg_device.hpp"

namespace tsg {

constexpr int kMaxExperts = 256;

// Lookup tables in the caller's workspace.
struct MoeTables {
  int* meta;        // [0] = number of row blocks in use, [1] = valid pairs
  int* offs;        // [E+1] exclusive prefix of the expert counts
  int* poffs;       // [E+1] first padded row of each expert
  int* rb_expert;   // expert of each row block, -1 past the last
  int* row_pair;    // pair of each padded row, -1 for padding
  int* row_token;   // token of each padded row, -1 for padding
  int* pair_row;    // padded row of each pair, -1 for a dropped pair
};

// ------------------------------------------------------------------ route
// Two kernels over blocks of 256 pairs, one pair per thread (P = T k <=
// 65535 pairs, so at most 256 blocks).
//   moe_count_kernel: each block counts its pairs per expert (wave ballots
//     into LDS) and stores the G x E block counts.
//   moe_place_kernel: each block loads all G x E counts into LDS and takes
//     from them the expert totals, offsets, padded offsets and its own
//     per-expert prefix over the earlier blocks.  A pair's rank among its
//     block's pairs of the same expert (wave ballots, then the earlier
//     waves' counts) then gives its place: position offs[e] + pre_b[e] +
//     rank in sorted_ids, row poffs[e] + pre_b[e] + rank.  The same kernel
//     marks padding rows, unused rows and the sorted_ids of dropped pairs
//     with -1; block 0 writes the counts, offsets and row-block table.
// Stable: pairs of one expert keep their order, so sorted_ids is ordered by
// (expert, token, slot).
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteMaxPairs = 65535;
constexpr int kRouteLdsCounts = 4096;  // G x E counts kept in LDS (larger: read from memory)
constexpr int kRouteMaskBlocks = 4096; // row blocks whose rank masks a block gathers in LDS

struct RouteArgs {
  const int32_t* ids;
  int32_t* counts;
  int32_t* sorted_ids;
  MoeTables ws;
  int* blk;             // [G][E] per-block counts (scratch)
  uint32_t* status;
  int P, E, k, G;
  int64_t rows_max, n_rb_max;
  // Optional (AllGather + MoE): rb_mask[rb] receives bit c for every chunk c
  // = token / tokens_per_rank that a row of block rb gathers from.  Each
  // placement block ORs its pairs' bits in LDS first and then ORs every
  // nonzero word into rb_mask once (n_rb_max <= kRouteMaskBlocks): a block's
  // pairs of one expert fill consecutive rows, so it touches few row blocks,
  // and the global atomics per word drop from one per pair to one per block.
  uint32_t* rb_mask;
  int tokens_per_rank;
};

// Padded offsets in LDS -> expert of padded row r (binary search), or -1
// past the last expert's rows.
__device__ __forceinline__ int expert_of_row(const int* s_poffs, int E, int64_t r) {
  if (r >= s_poffs[E]) return -1;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_poffs[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Ranks each lane's expert id among the lanes of its wave with the same id
// (lower lanes first) and stores the count of every id present into cnt[id]
// (LDS).  Lanes with ok == false take part in no group.
__device__ __forceinline__ int wave_rank(int e, bool ok, int* cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  int rank = 0;
  uint64_t todo = __ballot(ok);
  while (todo) {
    const int l = (int)__builtin_ctzll(todo);
    const int el = __builtin_amdgcn_readlane(e, l);
    const uint64_t m = __ballot(ok && e == el);
    if (ok && e == el) rank = __popcll(m & below);
    if (lane == l) cnt[el] = __popcll(m);
    todo &= ~m;
  }
  return rank;
}

template <int BM>
__global__ void __launch_bounds__(kRouteThreads) moe_count_kernel(const RouteArgs a) {
  __shared__ int s_cnt[kRouteWaves][kMaxExperts];
  const int b = blockIdx.x, t = threadIdx.x, wave = t >> 6;
  const int E = a.E;
  for (int i = t; i < kRouteWaves * kMaxExperts; i += kRouteThreads) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const int p = b * kRouteThreads + t;
  const int e = p < a.P ? a.ids[p] : 0;
  const bool ok = p < a.P && e >= 0 && e < E;
  (void)wave_rank(e, ok, s_cnt[wave]);
  if (__ballot(p < a.P && !ok) && (t & 63) == 0)
    __hip_atomic_fetch_or(a.status, ERR_BAD_EXPERT, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  __syncthreads();
  for (int x = t; x < E; x += kRouteThreads) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) c += s_cnt[w][x];
    a.blk[(int64_t)b * E + x] = c;
  }
  if (a.rb_mask)  // cleared here, filled by the placement kernel
    for (int64_t rb = p; rb < a.n_rb_max; rb += (int64_t)a.G * kRouteThreads) a.rb_mask[rb] = 0u;
}

template <int BM>
__global__ void __launch_bounds__(kRouteThreads) moe_place_kernel(const RouteArgs a) {
  __shared__ int s_cnt[kRouteWaves][kMaxExperts];
  __shared__ int s_blk[kRouteLdsCounts];
  __shared__ int s_offs[kMaxExperts + 1], s_poffs[kMaxExperts + 1], s_pre[kMaxExperts];
  __shared__ uint32_t s_mask[kRouteMaskBlocks];
  const int b = blockIdx.x, t = threadIdx.x, wave = t >> 6;
  const int E = a.E, G = a.G;
  const bool in_lds = G * E <= kRouteLdsCounts;
  const bool mask_lds = a.rb_mask && a.n_rb_max <= kRouteMaskBlocks;
  if (mask_lds)
    for (int i = t; i < a.n_rb_max; i += kRouteThreads) s_mask[i] = 0u;
  const int p = b * kRouteThreads + t;
  const int e = p < a.P ? a.ids[p] : 0;
  if (in_lds)
    for (int i = t; i < G * E; i += kRouteThreads) s_blk[i] = a.blk[i];
  for (int i = t; i < kRouteWaves * kMaxExperts; i += kRouteThreads) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  // per expert: prefix over the blocks before b, and the total
  for (int x = t; x < E; x += kRouteThreads) {
    int pre = 0, tot = 0;
    for (int bb = 0; bb < G; ++bb) {
      const int c = in_lds ? s_blk[bb * E + x] : a.blk[(int64_t)bb * E + x];
      pre += bb < b ? c : 0;
      tot += c;
    }
    s_pre[x] = pre;
    s_offs[x + 1] = tot;  // scanned below
  }
  __syncthreads();
  if (t == 0) {
    int o = 0, po = 0;
    for (int x = 0; x < E; ++x) {
      const int c = s_offs[x + 1];
      s_offs[x] = o;
      s_poffs[x] = po;
      o += c;
      po += (c + BM - 1) / BM * BM;
    }
    s_offs[E] = o;
    s_poffs[E] = po;
  }
  __syncthreads();
  if (b == 0) {
    for (int x = t; x <= E; x += kRouteThreads) {
      if (x < E) a.counts[x] = s_offs[x + 1] - s_offs[x];
      a.ws.offs[x] = s_offs[x];
      a.ws.poffs[x] = s_poffs[x];
    }
    if (t == 0) {
      a.ws.meta[0] = s_poffs[E] / BM;
      a.ws.meta[1] = s_offs[E];
    }
    for (int64_t rb = t; rb < a.n_rb_max; rb += kRouteThreads)
      a.ws.rb_expert[rb] = expert_of_row(s_poffs, E, rb * BM);
  }
  const bool ok = p < a.P && e >= 0 && e < E;
  int rank = wave_rank(e, ok, s_cnt[wave]);
  __syncthreads();
  if (ok) {
    for (int w = 0; w < wave; ++w) rank += s_cnt[w][e];
    rank += s_pre[e];
    const int row = s_poffs[e] + rank;
    a.sorted_ids[s_offs[e] + rank] = p;
    a.ws.pair_row[p] = row;
    a.ws.row_pair[row] = p;
    a.ws.row_token[row] = p / a.k;
    if (a.rb_mask) {
      const uint32_t bit = 1u << ((p / a.k) / a.tokens_per_rank);
      if (mask_lds)
        atomicOr(s_mask + row / BM, bit);
      else
        atomicOr(a.rb_mask + row / BM, bit);
    }
  } else if (p < a.P) {
    a.ws.pair_row[p] = -1;  // dropped pair (bad expert id)
  }
  if (mask_lds) {
    __syncthreads();
    for (int i = t; i < a.n_rb_max; i += kRouteThreads)
      if (s_mask[i]) atomicOr(a.rb_mask + i, s_mask[i]);
  }
  // rows that hold no pair: padding after each expert's pairs, and rows
  // past the last expert's
  const int64_t stride = (int64_t)G * kRouteThreads;
  for (int64_t r = p; r < a.rows_max; r += stride) {
    const int x = expert_of_row(s_poffs, E, r);
    if (x < 0 || r - s_poffs[x] >= s_offs[x + 1] - s_offs[x]) {
      a.ws.row_pair[r] = -1;
      a.ws.row_token[r] = -1;
    }
  }
  // sorted_ids past the kept pairs (only when pairs were dropped)
  for (int64_t q = (int64_t)s_offs[E] + p; q < a.P; q += stride) a.sorted_ids[q] = -1;
}

// ------------------------------------------------------------ block order
// The row blocks in use (meta[0] of them), ordered by a key taken from each
// block's rank mask: key(rb) = the largest (smallest, with min_key) of
// key_of[c] over the ranks c in rb_mask[rb], ties by block index (a stable
// counting sort).  The AllGather + MoE path keys a block by the arrival
// position of the last chunk it gathers from; the expert-compute path puts
// the blocks holding any token of another rank first.  One workgroup; at
// most kRouteMaskBlocks blocks, keys in [0, kRouteMaxRanks).
constexpr int kRouteMaxRanks = 32;

struct RbOrderArgs {
  const int* meta;
  const uint32_t* rb_mask;
  int* rb_order;
  int key_of[kRouteMaxRanks];
  int R;
  int min_key;
};

// (a template, like the routing kernels, so that every translation unit
// including this header may instantiate it)
template <int MAX_BLOCKS = kRouteMaskBlocks>
__global__ void __launch_bounds__(256) moe_rb_order_kernel(const RbOrderArgs a) {
  __shared__ int s_hist[kRouteMaxRanks + 1];
  __shared__ int s_key[MAX_BLOCKS];
  const int n_rb = min(a.meta[0], MAX_BLOCKS);
  const int t = threadIdx.x;
  if (t <= kRouteMaxRanks) s_hist[t] = 0;
  __syncthreads();
  for (int rb = t; rb < n_rb; rb += 256) {
    const uint32_t m = a.rb_mask[rb];
    int key = a.min_key ? kRouteMaxRanks - 1 : 0;
    for (int c = 0; c < a.R; ++c)
      if ((m >> c) & 1u) key = a.min_key ? min(key, a.key_of[c]) : max(key, a.key_of[c]);
    key = min(max(key, 0), kRouteMaxRanks - 1);
    s_key[rb] = key;
    atomicAdd(&s_hist[key], 1);
  }
  __syncthreads();
  if (t == 0) {  // exclusive scan over the keys, then a stable placement
    int run = 0;
    for (int key = 0; key < kRouteMaxRanks; ++key) {
      const int c = s_hist[key];
      s_hist[key] = run;
      run += c;
    }
    for (int rb = 0; rb < n_rb; ++rb) a.rb_order[s_hist[s_key[rb]]++] = rb;
  }
}

}  // namespace tsg
