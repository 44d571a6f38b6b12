// AllGather of the KV context + self-attention (sequence parallel), one
// rank's share.
//
// "TileLink: Generating Efficient Compute-Communication Overlapping Kernels
// using Tile-Centric Primitives", section 2.1 (sequence-parallel attention:
// the key/value context is sharded across ranks and gathered before the
// attention), section 5 (AllGather KV + self-attention: the communication
// tile is one rank's share of the sequence, S / R rows, the computation
// tile differs, and tile-centric mapping keeps the barriers between the two
// correct) and section 7.2 (self-attention layer: two batched GEMMs and a
// softmax fused in the Flash-Attention manner).
//
// The S tokens are sharded over R ranks along the sequence (chunk c = rows
// [c S/R, (c+1) S/R) of rank c).  K and V are [S x heads x D] row-major
// (one row per token, heads side by side), Q and out [S/R x heads x D] (this
// rank's tokens).  For each head h and local query q:
//     out[q, h] = sum_j softmax_j(Q[q, h] . K[j, h] / sqrt(D)) V[j, h]
// over all S keys j (no mask).
//
// One persistent kernel, one ticket queue: first the copy units that stand
// in for the peers' arrival (the AllGather copy's units over K, then V, as
// [S x heads D] matrices: column slabs of each chunk, peers in arrival order,
// the local chunk last, every (chunk, slab) counted on its signal), then the
// attention tiles (head, 128 queries).  A tile takes the chunks in arrival
// order, its own chunk first, read in place from k_local / v_local without
// waiting; before a peer chunk it waits for the K and V signals of the slabs
// holding its head's columns.  Inside a chunk, 64 keys at a time:
//   S = Q K^T (v_mfma_f32_32x32x16_bf16; Q fragments in registers, K staged
//   in LDS), online softmax per query row (running max and sum, exp2 of the
//   scaled scores), P rounded to bf16 through a per-wave LDS region, then
//   O += P V (V staged in LDS and read with transpose reads).  The next
//   block's K and V are loaded into registers while this one is computed.
// out = O / (row sum), rounded to bf16.
#include "tsg_copy.hpp"
#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"

using namespace tsg;

namespace {

constexpr int D = 128;      // head dimension
constexpr int BQ = 128;     // queries per tile: 4 waves x 32
constexpr int BKV = 64;     // keys per block
constexpr int NT = 256;
constexpr size_t kSigBase = (size_t(1) << 17) + 65536;  // K then V slab signals in the context's pool
constexpr size_t kSigCap = 65536;
constexpr int kQueueSlot = 52;

// V blocks are staged as the B operand of a GEMM whose k dimension is the
// key (64 rows) and whose n dimension is the head dimension (128 columns):
// the transpose reads of the GEMM engine then hand out P V's B fragments.
using CfgV = TileCfg<BQ, D, 4, 1>;
using TileV = GemmTile<CfgV>;

constexpr int K_BYTES = BKV * D * 2;     // 16 KB, two halves of 64 columns
constexpr int V_BYTES = BKV * D * 2;     // 16 KB
constexpr int P_BYTES = 32 * BKV * 2;    // per wave, 4 KB
constexpr int LDS_BYTES = K_BYTES + V_BYTES + 4 * P_BYTES;
static_assert(CfgV::B_STAGE == V_BYTES, "V block is one B stage");

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_local;
  const uint16_t* v_local;
  const uint16_t* k_full;
  const uint16_t* v_full;
  uint16_t* out;
  const uint64_t* sig_k;  // chunk c, slab s at c * n_slab + s
  const uint64_t* sig_v;
  uint32_t* queue;        // ticket, exit counter (zero between calls)
  SyncArgs sa;
  Timeline tl;
  CopyArgs copy_k, copy_v;
  int n_copy_k, n_copy_v;
  int n_tiles;            // heads x query blocks
  int n_qb;
  int heads, S_loc, R, rank;
  int8_t order[kMaxRanks];  // chunk at arrival position p (p = 0: own chunk)
  int n_slab, slab_log2;
  int wait;
  int l1_only;
  float scale_log2;       // log2(e) / sqrt(D)
};

// Global -> register loads of one 64-key block of K or V (64 rows x 256 B):
// 1024 pieces of 16 B, four per thread; piece i = t + 256 it is row i / 16,
// 16-byte column chunk i % 16.
struct BlockRegs {
  u32x4_t k[4], v[4];
};

__device__ __forceinline__ void load_block(BlockRegs& br, const uint16_t* kb, const uint16_t* vb, int64_t ld) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = threadIdx.x + NT * it;
    const int r = i >> 4, gc = i & 15;
    br.k[it] = *(const u32x4_t*)(kb + (int64_t)r * ld + gc * 8);
    br.v[it] = *(const u32x4_t*)(vb + (int64_t)r * ld + gc * 8);
  }
}

// Register -> LDS.  K: two halves of 64 columns, each in the engine's A-stage
// layout (rows of 128 bytes, chunk c of row r at position c ^ (r / 2 mod 8)).
// V: one B stage, row-major, chunk c of row r at position c ^ b_swz(r).
__device__ __forceinline__ void store_block(const BlockRegs& br, char* lk, char* lv) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = threadIdx.x + NT * it;
    const int r = i >> 4, gc = i & 15;
    *(u32x4_t*)(lk + (gc >> 3) * (BKV * 128) + lds_swz(r, gc & 7)) = br.k[it];
    *(u32x4_t*)(lv + r * (D * 2) + ((gc ^ TileV::b_swz(r)) << 4)) = br.v[it];
  }
}

__device__ __forceinline__ float wave_half_max(float x) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_half_sum(float x) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One attention tile: head h, queries [qb * BQ, qb * BQ + BQ) of this rank.
// Returns the wall-clock ticks spent waiting for signals.
__device__ __forceinline__ uint64_t attn_tile(const AttnArgs& a, int h, int qb, char* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  char* lk = lds;
  char* lv = lds + K_BYTES;
  char* lp = lds + K_BYTES + V_BYTES + wave * P_BYTES;
  const int64_t ld = (int64_t)a.heads * D;  // elements per token row

  // Q fragments: lane row = wave * 32 + l32, k16 step ks: columns 16 ks + 8 hi .. + 7
  bf16x8_t qa[D / 16];
  {
    int row = qb * BQ + wave * 32 + l32;
    if (row >= a.S_loc) row = a.S_loc - 1;  // never stored
    const uint16_t* qr = a.q + (int64_t)row * ld + h * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qa[ks] = *(const bf16x8_t*)(qr + 16 * ks);
  }
  f32x16_t o[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[j][v] = 0.f;
  // per lane: 16 query rows (8 (v / 4) + 4 hi + v mod 4), running max (in
  // log2 units) and sum
  float m[16], l[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    m[v] = -INFINITY;
    l[v] = 0.f;
  }
  uint32_t tr_off[CfgV::FN];
  TileV::tr_lane_offsets(0, tr_off);
  const int s_lo = (h * D) >> a.slab_log2, s_hi = (h * D + D - 1) >> a.slab_log2;
  const int n_blk = a.S_loc / BKV;
  uint64_t waited = 0;

  for (int p = 0; p < a.R; ++p) {
    const int c = a.order[p];
    const bool own = c == a.rank;
    if (!own && a.wait) {
      const uint64_t t = wall_clock64();
      const uint64_t target = sig_target(a.sa.epoch, 1);
      for (int s = s_lo; s <= s_hi; ++s) {
        block_poll_ge(a.sig_k + (size_t)c * a.n_slab + s, target, a.sa);
        block_poll_ge(a.sig_v + (size_t)c * a.n_slab + s, target, a.sa);
      }
      acquire_lines(a.l1_only != 0);
      waited += wall_clock64() - t;
    }
    const uint16_t* kc = own ? a.k_local : a.k_full + (int64_t)c * a.S_loc * ld;
    const uint16_t* vc = own ? a.v_local : a.v_full + (int64_t)c * a.S_loc * ld;
    kc += h * D;
    vc += h * D;
    BlockRegs br;
    load_block(br, kc, vc, ld);
    for (int b = 0; b < n_blk; ++b) {
      __syncthreads();  // the previous block's LDS reads are done
      store_block(br, lk, lv);
      __syncthreads();
      if (b + 1 < n_blk) load_block(br, kc + (int64_t)(b + 1) * BKV * ld, vc + (int64_t)(b + 1) * BKV * ld, ld);
      // S = Q K^T, two fragments of 32 keys
      f32x16_t s[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[j][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const char* half = lk + (ks >> 2) * (BKV * 128);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_t kb = *(const bf16x8_t*)(half + lds_swz(32 * j + l32, 2 * (ks & 3) + hi));
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kb, s[j], 0, 0, 0);
        }
      }
      // online softmax over the block's 64 keys, per query row
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x0 = s[0][v] * a.scale_log2, x1 = s[1][v] * a.scale_log2;
        const float mn = fmaxf(m[v], wave_half_max(fmaxf(x0, x1)));
        const float alpha = exp2f(m[v] - mn);
        const float p0 = exp2f(x0 - mn), p1 = exp2f(x1 - mn);
        l[v] = l[v] * alpha + wave_half_sum(p0 + p1);
        m[v] = mn;
#pragma unroll
        for (int j = 0; j < D / 32; ++j) o[j][v] *= alpha;
        // P in bf16, row r of the wave's region, keys l32 and 32 + l32
        const int r = 8 * (v >> 2) + 4 * hi + (v & 3);
        *(uint16_t*)(lp + lds_swz(r, l32 >> 3) + (l32 & 7) * 2) = (uint16_t)f32_to_bf16(p0);
        *(uint16_t*)(lp + lds_swz(r, 4 + (l32 >> 3)) + (l32 & 7) * 2) = (uint16_t)f32_to_bf16(p1);
      }
      // the wave's P region is its own: its writes complete before its reads
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // O += P V, four k16 steps of 16 keys
#pragma unroll
      for (int kk = 0; kk < BKV / 16; ++kk) {
        const bf16x8_t pa = *(const bf16x8_t*)(lp + lds_swz(l32, 2 * kk + hi));
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
          o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, TileV::read_b_tr(lv, tr_off[j], kk), o[j], 0, 0, 0);
      }
    }
  }
  // out = O / l, bf16
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = qb * BQ + wave * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
    if (row < a.S_loc) {
      const float inv = 1.0f / l[v];
      uint16_t* orow = a.out + (int64_t)row * ld + h * D + l32;
#pragma unroll
      for (int j = 0; j < D / 32; ++j) orow[32 * j] = (uint16_t)f32_to_bf16(o[j][v] * inv);
    }
  }
  return waited;
}

__global__ void __launch_bounds__(NT) ag_attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int n_items = a.n_copy_k + a.n_copy_v + a.n_tiles;
  // Next item, identical in every thread; the ticket goes through the first
  // word of the LDS, which is free between items (every item ends with a
  // barrier).
  auto fetch = [&]() -> int {
    volatile int* s_item = (volatile int*)lds;
    if (threadIdx.x == 0) *s_item = (int)atomicAdd(a.queue, 1u);
    __syncthreads();
    const int v = __builtin_amdgcn_readfirstlane(*s_item);
    __syncthreads();
    return v;
  };
  for (int item = fetch(); item < n_items; item = fetch()) {
    if (item < a.n_copy_k) {
      copy_unit<NT>(a.copy_k, item);
    } else if (item < a.n_copy_k + a.n_copy_v) {
      copy_unit<NT>(a.copy_v, item - a.n_copy_k);
    } else {
      const int t = item - a.n_copy_k - a.n_copy_v;
      const int h = t / a.n_qb, qb = t - h * a.n_qb;
      const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
      const uint64_t waited = attn_tile(a, h, qb, lds);
      if (a.tl.buf && threadIdx.x == 0)
        timeline_put(a.tl, 11, (uint32_t)(h << 16 | qb), t0, t0 + waited, wall_clock64());
    }
    __syncthreads();
  }
  // the last workgroup to leave resets the ticket and exit counters
  if (threadIdx.x == 0 && atomicAdd(a.queue + 1, 1u) == gridDim.x - 1) {
    __hip_atomic_store(a.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.queue + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

tsg_status tsg_op_attn(tsg_ctx* ctx, const void* q, const void* k_local, const void* k_peers, const void* v_local,
                       const void* v_peers, void* k_full, void* v_full, void* out, int S, int heads, int head_dim,
                       int R, int rank, const int* arrival_order, const tsg_opts* opts, int mode, void* stream) {
  using namespace tsgh;
  if (!q || !k_local || !v_local || !k_full || !v_full || !out || (R > 1 && (!k_peers || !v_peers)))
    return fail(ctx, TSG_E_INVALID, "ag_kv_attention: null pointer");
  if (mode < TSG_MODE_OVERLAP || mode > TSG_MODE_COMM_ONLY) return fail(ctx, TSG_E_INVALID, "bad mode");
  if (head_dim != D) return fail(ctx, TSG_E_UNSUPPORTED, "ag_kv_attention supports head_dim %d only", D);
  if (R < 1 || R > kMaxRanks || rank < 0 || rank >= R)
    return fail(ctx, TSG_E_SHAPE, "need 1 <= R <= %d and 0 <= rank < R", kMaxRanks);
  if (heads < 1 || S < R * BKV || S % (R * BKV))
    return fail(ctx, TSG_E_SHAPE, "ag_kv_attention: S must be a positive multiple of %d R (S=%d R=%d)", BKV, S, R);
  if ((int64_t)S * heads * D * 2 >= (int64_t(1) << 31))
    return fail(ctx, TSG_E_UNSUPPORTED, "operands of 2 GiB or more are not supported");
  if (!aligned16(q) || !aligned16(k_local) || !aligned16(v_local) || !aligned16(k_full) || !aligned16(v_full) ||
      !aligned16(out) || (k_peers && !aligned16(k_peers)) || (v_peers && !aligned16(v_peers)))
    return fail(ctx, TSG_E_ALIGN, "ag_kv_attention: pointers must be 16-byte aligned");

  // tile order of the chunks: own chunk first, then the peers in arrival
  // order; the copy moves the peers in that order and the own chunk last
  int pos_of[kMaxRanks];
  for (int i = 0; i < kMaxRanks; ++i) pos_of[i] = -1;
  int8_t ord[kMaxRanks] = {};
  ord[0] = (int8_t)rank;
  pos_of[rank] = 0;
  for (int p = 1; p < R; ++p) {
    const int cc = arrival_order ? arrival_order[p - 1] : (rank + p) % R;
    if (cc < 0 || cc >= R || pos_of[cc] >= 0)
      return fail(ctx, TSG_E_INVALID, "arrival_order must be a permutation of the peer ranks");
    ord[p] = (int8_t)cc;
    pos_of[cc] = p;
  }
  const Opts o = resolve(opts, -1);
  if (o.aux_cus > 0) return fail(ctx, TSG_E_UNSUPPORTED, "ag_kv_attention runs on shared CUs only");
  // slab: the columns of one head by default (comm_tile: any power of two
  // from 64 to 2048)
  int slab = o.comm_tile ? o.comm_tile : D;
  if (slab < 64 || slab > 2048 || (slab & (slab - 1)))
    return fail(ctx, TSG_E_INVALID, "comm_tile must be a power of two in [64, 2048] (got %d)", slab);
  const int HD = heads * D;
  int slab_log2 = 0;
  while ((1 << slab_log2) < slab) ++slab_log2;
  const int n_slab = (HD + slab - 1) / slab;
  if ((size_t)2 * R * n_slab > kSigCap) return fail(ctx, TSG_E_UNSUPPORTED, "too many slab signals");
  const int S_loc = S / R;
  const int nwg = ctx->n_cus;  // one workgroup per CU (its registers allow one wave per SIMD)
  int np[kHead + 1], ustart[kHead + 1];
  int64_t n_units = 0;
  if (!copy_plan(R, 1, S_loc, HD, n_slab, slab_log2 - 3, nwg, np, ustart, &n_units))
    return fail(ctx, TSG_E_UNSUPPORTED, "ag_kv_attention: the copy's offsets would overflow");

  TSG_HIP(ctx, hipSetDevice(ctx->device));
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);
  const SyncArgs sa = sync_args(ctx, o);
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  CopyArgs ck;
  ck.a_local = (const u32x4_t*)k_local;
  ck.a_peers = (const u32x4_t*)k_peers;
  ck.a_full = (u32x4_t*)k_full;
  ck.sig = ctx->d_sig + kSigBase;
  ck.cnt = ctx->d_cnt + kSigBase;
  ck.sa = sa;
  ck.tl = Timeline{nullptr, nullptr, 0};
  for (int p = 0; p < kMaxRanks; ++p) ck.ord.chunk[p] = 0;
  for (int p = 1; p < R; ++p) ck.ord.chunk[p - 1] = ord[p];
  ck.ord.chunk[R - 1] = (int8_t)rank;
  ck.k8 = HD / 8;
  ck.chunk_rows = S_loc;
  ck.R = R;
  ck.rank = rank;
  ck.C = 1;
  ck.ch_rows = S_loc;
  ck.n_slab = n_slab;
  ck.vpr_log2 = slab_log2 - 3;
  for (int i = 0; i <= kHead; ++i) {
    ck.np[i] = np[i];
    ck.ustart[i] = ustart[i];
  }
  ck.n_units = (int)n_units;
  ck.skip_mask = o.skip_mask;
  ck.queue = nullptr;
  ck.n_workers = 0;
  ck.pace_word = nullptr;
  ck.pace_ticks = 0.f;
  CopyArgs cv = ck;
  cv.a_local = (const u32x4_t*)v_local;
  cv.a_peers = (const u32x4_t*)v_peers;
  cv.a_full = (u32x4_t*)v_full;
  cv.sig = ctx->d_sig + kSigBase + (size_t)R * n_slab;
  cv.cnt = ctx->d_cnt + kSigBase + (size_t)R * n_slab;

  AttnArgs ka;
  ka.q = (const uint16_t*)q;
  ka.k_local = (const uint16_t*)k_local;
  ka.v_local = (const uint16_t*)v_local;
  ka.k_full = (const uint16_t*)k_full;
  ka.v_full = (const uint16_t*)v_full;
  ka.out = (uint16_t*)out;
  ka.sig_k = ck.sig;
  ka.sig_v = cv.sig;
  ka.queue = ctx->d_queue + kQueueSlot;
  ka.sa = sa;
  ka.tl = timeline(ctx, o);
  ka.copy_k = ck;
  ka.copy_v = cv;
  ka.n_qb = (S_loc + BQ - 1) / BQ;
  ka.heads = heads;
  ka.S_loc = S_loc;
  ka.R = R;
  ka.rank = rank;
  for (int p = 0; p < kMaxRanks; ++p) ka.order[p] = ord[p];
  ka.n_slab = n_slab;
  ka.slab_log2 = slab_log2;
  ka.l1_only = ((uintptr_t)k_full % 128 == 0 && (uintptr_t)v_full % 128 == 0 && slab >= 64) ? 1 : 0;
  ka.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int n_tiles = heads * ka.n_qb;

  auto launch = [&](int n_copy, int tiles, int wait, int which) -> tsg_status {
    ka.n_copy_k = n_copy;
    ka.n_copy_v = n_copy;
    ka.n_tiles = tiles;
    ka.wait = wait;
    time_begin(ctx, which, caller);
    hipLaunchKernelGGL(ag_attn_kernel, dim3(nwg), dim3(NT), 0, caller, ka);
    time_end(ctx, which, caller);
    return check_launch(ctx, "ag_attn_kernel");
  };
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
