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
// The copy that stands in for the peers' arrival is the AllGather copy's
// units over K and V as [S x heads D] matrices: column slabs of each chunk,
// peers in arrival order, the local chunk last, every (chunk, slab) counted
// on its signal.  Overlapped, it runs as a small kernel of its own beside the
// attention kernel, on the same CUs (one copy wave per SIMD fits beside two
// attention waves), arrival position by position; or, with opts.pull_units > 0, as the first items of the attention
// kernel's own ticket queue.  The attention tiles (head, 128 queries) take
// the chunks in arrival order, their own chunk first, read in place from
// k_local / v_local without waiting; before a peer chunk a tile waits for the
// K and V signals of the slabs holding its head's columns.  Inside a chunk,
// 64 keys at a time:
//   S^T = K Q^T (v_mfma_f32_32x32x16_bf16; Q fragments in registers, K
//   staged in LDS), online softmax per query (running max and sum, exp2 of
//   the scaled scores), then O^T += V^T P^T with P^T taken from the S^T
//   registers rounded to bf16 and V staged in LDS and read with transpose
//   reads.  The next block's K and V are loaded into the other LDS stage
//   while this one is computed.
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
constexpr int kQueueSlot = 64;       // attention kernel: 2 phases x 8 XCD tickets, exit counter
constexpr int kCopyQueueSlot = 54;   // copy kernel: ticket, exit counter (56-57: a copy the call joins)

// V blocks are staged like a B stage of the GEMM engine (64 key rows of 128
// head-dimension columns, row-major, 16-byte chunks permuted per row by
// b_swz so that transpose reads are free of bank conflicts).
using CfgV = TileCfg<BQ, D, 4, 1>;
using TileV = GemmTile<CfgV>;

constexpr int K_BYTES = BKV * D * 2;     // 16 KB, two halves of 64 columns
constexpr int V_BYTES = BKV * D * 2;     // 16 KB
constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;  // two stages: block b + 1 lands while block b is computed
static_assert(CfgV::B_STAGE == V_BYTES, "V block is one B stage");
static_assert(BKV == 64 && D == 128, "the load-block mapping below assumes 64 x 128 blocks");

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_local;
  const uint16_t* v_local;
  const uint16_t* k_full;
  const uint16_t* v_full;
  uint16_t* out;
  const uint64_t* sig_k;  // chunk c, slab s at c * n_slab + s
  const uint64_t* sig_v;
  uint32_t* queue;        // 2 phases x 8 XCD ticket counters, exit counter (zero between calls)
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
  int wait_own_end;       // after its stores a tile waits for its own chunk's K and V slabs
  int l1_only;
  float scale_log2;       // log2(e) / sqrt(D)
};

// A 64-key block of K or V is 16 KB of LDS, moved from global memory by
// global_load_lds (16 bytes a lane, 1 KB a wave instruction, no registers):
// load block t = w + 4 i (i = 0..3) of wave w.  Lane l fills byte 16 l of the
// load block, which fixes the global piece it fetches:
//   K: two halves of 64 columns in the engine's A-stage layout (rows of 128
//      bytes, chunk c of row r at position lds_pos(r, c), its own inverse);
//      load block t is rows 8 (t mod 8) .. + 7 of half t / 8, and lane l
//      takes row 8 (t mod 8) + l / 8, logical chunk lds_pos(row, l mod 8);
//   V: one B stage, row-major, column chunk c of row r at position
//      c ^ b_swz(r); load block t is rows 4 t .. 4 t + 3, and lane l takes
//      row 4 t + l / 16, column chunk (l mod 16) ^ b_swz(row).
// The offsets are in bytes from the block's first row in global memory.
struct LoadOffsets {
  uint32_t k[4], v[4];
};

__device__ __forceinline__ void load_offsets(LoadOffsets& lo, int64_t ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = wave + 4 * i;
    const int kr = 8 * (t & 7) + (lane >> 3);
    const int kcol = 64 * (t >> 3) + 8 * (int)lds_pos(kr, lane & 7);
    lo.k[i] = (uint32_t)((kr * ld + kcol) * 2);
    const int vr = 4 * t + (lane >> 4);
    const int vcol = 8 * ((lane & 15) ^ TileV::b_swz(vr));
    lo.v[i] = (uint32_t)((vr * ld + vcol) * 2);
  }
}

// Issue the loads of one block (its first rows at kb and vb) into a stage.
__device__ __forceinline__ void issue_block(const LoadOffsets& lo, const uint16_t* kb, const uint16_t* vb,
                                            char* stage) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = wave + 4 * i;
    __builtin_amdgcn_global_load_lds((const void*)((const char*)kb + lo.k[i]),
                                     (__attribute__((address_space(3))) void*)(stage + t * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)((const char*)vb + lo.v[i]),
                                     (__attribute__((address_space(3))) void*)(stage + K_BYTES + t * 1024),
                                     16, 0, 0);
  }
}

// LDS byte offset of this lane's transpose reads of V for the A operand of
// O^T += V^T P^T: lane l takes column d = 32 j + (l mod 32) of V and, in a
// 16-key step, the keys 4 (l / 32) + 0..3 (first read) and 8 + 4 (l / 32)
// + 0..3 (second read, 8 rows further) -- the same keys, in the same order,
// as the scores this lane holds in registers 0..7 (or 8..15) of S^T, which
// makes those registers the B operand P^T directly.  In each group of 16
// lanes, lane 4 i + q points at row i, columns 4 q .. 4 q + 3 of a 4-row,
// 16-column block.
__device__ __forceinline__ void v_lane_offsets(uint32_t (&off)[D / 32]) {
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5, g = lane >> 4, sl = lane & 15;
  const int row = 4 * hi + (sl >> 2);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const int col = 32 * j + 16 * (g & 1) + 4 * (sl & 3);
    const int chunk = (col >> 3) ^ TileV::b_swz(row);
    off[j] = (uint32_t)((row * D + chunk * 8 + (col & 7)) * 2);
  }
}

__device__ __forceinline__ bf16x8_t read_v(const char* lv, uint32_t off, int kk) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const char* p = lv + off + kk * 16 * D * 2;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 8 * D * 2));
  const v8i16 w = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, w);
}

// Eight fp32 values as the bf16x8 operand, rounded to nearest even
// (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16x8_t pack_bf16x8(const f32x16_t& x, int base) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 f = {x[base + 2 * i], x[base + 2 * i + 1]};
    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  const u32x4_t v = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Rescale threshold of the running maximum, in log2 units: the reference
// maximum m of a query moves only when a block's maximum exceeds it by more
// than this, so that exp2(score - m) stays below 2^8 and the rescale of O
// and l is skipped for most blocks (softmax does not depend on m).
constexpr float kRescaleLog2 = 8.0f;

// One attention tile: head h, queries [qb * BQ, qb * BQ + BQ) of this rank;
// wave w owns queries qb * BQ + 32 w .. + 31, one per lane pair (l, l + 32).
// Transposed products: S^T = K Q^T and O^T += V^T P^T, so that a lane holds
// scores and outputs of a single query (its l mod 32): the softmax max and
// sum reduce in registers and across the two lane halves only, the running
// rescale is per lane, and the probabilities go from the S^T accumulators
// straight into the B operand of the second product.
// Returns the wall-clock ticks spent waiting for signals.
__device__ __forceinline__ uint64_t attn_tile(const AttnArgs& a, int h, int qb, char* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const int64_t ld = (int64_t)a.heads * D;  // elements per token row
  const int qrow = qb * BQ + wave * 32 + l32;

  // Q^T fragments (B operand): lane column = query qrow, k16 step ks:
  // head-dimension 16 ks + 8 hi .. + 7
  bf16x8_t qa[D / 16];
  {
    const int row = qrow < a.S_loc ? qrow : a.S_loc - 1;  // never stored
    const uint16_t* qr = a.q + (int64_t)row * ld + h * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qa[ks] = *(const bf16x8_t*)(qr + 16 * ks);
  }
  // O^T: fragment j holds head-dimension rows 32 j + 8 (v / 4) + 4 hi +
  // v mod 4 (register v) of this lane's query
  f32x16_t o[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[j][v] = 0.f;
  float m = -INFINITY, l = 0.f;  // reference max (log2 units) and sum of this lane's query
  uint32_t v_off[D / 32];
  v_lane_offsets(v_off);
  const int s_lo = (h * D) >> a.slab_log2, s_hi = (h * D + D - 1) >> a.slab_log2;
  const int n_blk = a.S_loc / BKV;
  uint64_t waited = 0;

  LoadOffsets lo;
  load_offsets(lo, ld);
  // chunk base pointers (this head's columns) of arrival position p; before
  // a peer chunk's first block is loaded, the K and V signals of the slabs
  // holding the head's columns are waited for
  auto chunk_base = [&](int p, const uint16_t*& kc, const uint16_t*& vc) {
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
    kc = (own ? a.k_local : a.k_full + (int64_t)c * a.S_loc * ld) + h * D;
    vc = (own ? a.v_local : a.v_full + (int64_t)c * a.S_loc * ld) + h * D;
  };
  const uint16_t *kc, *vc;
  chunk_base(0, kc, vc);
  issue_block(lo, kc, vc, lds);
  // blocks g = p n_blk + b in arrival order; block g is in stage g mod 2
  const int n_all = a.R * n_blk;
  for (int g = 0, b = 0, p = 0; g < n_all; ++g) {
    // block g has landed (this wave's loads, then every wave's), and every
    // wave is done reading the other stage (block g - 1)
    wait_vmcnt<0>();
    lds_barrier();
    const char* lk = lds + (g & 1) * STAGE_BYTES;
    const char* lv = lk + K_BYTES;
    if (++b == n_blk) {
      b = 0;
      if (++p < a.R) chunk_base(p, kc, vc);
    }
    if (g + 1 < n_all)
      issue_block(lo, kc + (int64_t)b * BKV * ld, vc + (int64_t)b * BKV * ld, lds + ((g + 1) & 1) * STAGE_BYTES);
    // S^T = K Q^T: fragment j holds keys 32 j + 8 (v / 4) + 4 hi + v mod 4
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
        const bf16x8_t kf = *(const bf16x8_t*)(half + lds_swz(32 * j + l32, 2 * (ks & 3) + hi));
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qa[ks], s[j], 0, 0, 0);
      }
    }
    // online softmax of this lane's query over the block's 64 keys: 32 in
    // this lane, 32 in lane l ^ 32 (scores in log2 units: raw x scale)
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[j][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
    if (__any(mx > m + kRescaleLog2)) {  // wave-uniform
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      m = mn;
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[j][v] *= alpha;
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[j][v] = __builtin_amdgcn_exp2f(fmaf(s[j][v], a.scale_log2, -m));
        sum += s[j][v];
      }
    l += sum + __shfl_xor(sum, 32, 64);
    // O^T += V^T P^T, four 16-key steps: P^T from registers 8 (kk mod 2)
    // .. + 7 of S^T fragment kk / 2, rounded to bf16
#pragma unroll
    for (int kk = 0; kk < BKV / 16; ++kk) {
      const bf16x8_t pb = pack_bf16x8(s[kk >> 1], 8 * (kk & 1));
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(lv, v_off[j], kk), pb, o[j], 0, 0, 0);
    }
  }
  lds_barrier();  // every wave is done with the stages before the LDS is reused
  // out = O / l in bf16: four consecutive head-dimension values per
  // (fragment, register group), one 8-byte store each
  if (qrow < a.S_loc) {
    const float inv = 1.0f / l;
    uint16_t* orow = a.out + (int64_t)qrow * ld + h * D + 4 * hi;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint64_t w = (uint64_t)f32_to_bf16(o[j][4 * g] * inv) |
                           ((uint64_t)f32_to_bf16(o[j][4 * g + 1] * inv) << 16) |
                           ((uint64_t)f32_to_bf16(o[j][4 * g + 2] * inv) << 32) |
                           ((uint64_t)f32_to_bf16(o[j][4 * g + 3] * inv) << 48);
        *(uint64_t*)(orow + 32 * j + 8 * g) = w;
      }
  }
  // When the caller's stream does not wait for the copy kernel, the
  // attention kernel's end must imply the whole gather: a tile waited for
  // every peer chunk of its head, and the own chunk, moved last and read in
  // place, is waited for here (long complete in practice).
  if (a.wait_own_end) {
    const uint64_t target = sig_target(a.sa.epoch, 1);
    for (int s = s_lo; s <= s_hi; ++s) {
      block_poll_ge(a.sig_k + (size_t)a.rank * a.n_slab + s, target, a.sa);
      block_poll_ge(a.sig_v + (size_t)a.rank * a.n_slab + s, target, a.sa);
    }
  }
  return waited;
}

// Items come from per-XCD phased queues: phase 0 the copy units (K, then
// V), phase 1 the tiles, head-major (tile t = head t / n_qb, query block
// t mod n_qb), so that each XCD runs a contiguous share of heads and the
// query blocks of a head, which stream the same keys and values, share its
// L2.
__global__ void __launch_bounds__(NT, 2) ag_attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int n_ph[2] = {a.n_copy_k + a.n_copy_v, a.n_tiles};
  const int my_xcd = xcd_id();
  int phase = 0;
  // Next item, identical in every thread: wave 0 claims it and passes it on
  // through the first words of the LDS, which are free between items (every
  // item ends with a barrier).
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
      if (it.index < a.n_copy_k)
        copy_unit<NT>(a.copy_k, it.index);
      else
        copy_unit<NT>(a.copy_v, it.index - a.n_copy_k);
    } else {
      const int h = it.index / a.n_qb, qb = it.index - h * a.n_qb;
      const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
      const uint64_t waited = attn_tile(a, h, qb, lds);
      if (a.tl.buf && threadIdx.x == 0)
        timeline_put(a.tl, 11, (uint32_t)(h << 16 | qb), t0, t0 + waited, wall_clock64());
    }
    __syncthreads();
  }
  // the last workgroup to leave resets the ticket and exit counters
  if (threadIdx.x == 0 && atomicAdd(a.queue + 16, 1u) == gridDim.x - 1)
    for (int i = 0; i <= 16; ++i) __hip_atomic_store(a.queue + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy kernel of the overlapped form: units from its own queue, arrival
// position by position (all slabs of the first peer's K and V, then the
// next peer's, ...), until none is left.  It never
// waits, so it always drains the queue.  Capped at 48 registers (the
// attribute counts half the unified register file): one copy wave fits on
// each SIMD beside two attention waves of 200.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(24)))
    ag_attn_copy_kernel(const CopyArgs ck, const CopyArgs cv) {
  __shared__ int slot;
  // every slab has npc pieces a chunk, and unit u = (s R + p) npc + j;
  // ticket w takes arrival position p = (w / 2) / (n_slab npc) first, then
  // slab, piece, and K (w even) or V (w odd)
  const int npc = ck.np[kHead];
  const int per_pos = ck.n_slab * npc;
  const int n = ck.n_units + cv.n_units;
  for (int w = claim_unit(ck, &slot); w < n; w = claim_unit(ck, &slot)) {
    const int w2 = w >> 1;
    const int p = w2 / per_pos;
    const int r = w2 - p * per_pos;
    const int sl = r / npc;
    const int u = (sl * ck.R + p) * npc + (r - sl * npc);
    if (w & 1)
      copy_unit<256>(cv, u);
    else
      copy_unit<256>(ck, u);
  }
  if (threadIdx.x == 0) leave_queue(ck);
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
  // two workgroups per CU: with at most 256 registers a wave, two waves share
  // each SIMD, so one's softmax runs while the other's MFMAs do
  const int nwg = 2 * ctx->n_cus;
  int np[kHead + 1], ustart[kHead + 1];
  int64_t n_units = 0;
  if (!copy_plan(R, 1, S_loc, HD, n_slab, slab_log2 - 3, nwg, np, ustart, &n_units))
    return fail(ctx, TSG_E_UNSUPPORTED, "ag_kv_attention: the copy's offsets would overflow");
  // one piece count for every slab (every tile needs whole chunks of its
  // head, so no slab comes first): unit u = (s R + p) npc + j
  {
    const int npc = np[kHead];
    for (int i = 0; i <= kHead; ++i) {
      np[i] = npc;
      ustart[i] = std::min(i, n_slab) * R * npc;
    }
    n_units = (int64_t)n_slab * R * npc;
  }

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
  ck.tl = timeline(ctx, o);  // copy units: kind 1
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
  ck.unit_base = 0;
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
  ka.wait_own_end = 0;
  ka.l1_only = ((uintptr_t)k_full % 128 == 0 && (uintptr_t)v_full % 128 == 0 && slab >= 64) ? 1 : 0;
  ka.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int n_tiles = heads * ka.n_qb;

  auto launch = [&](hipStream_t st, int n_copy, int tiles, int wait, int which) -> tsg_status {
    ka.n_copy_k = n_copy;
    ka.n_copy_v = n_copy;
    ka.n_tiles = tiles;
    ka.wait = wait;
    time_begin(ctx, which, st);
    hipLaunchKernelGGL(ag_attn_kernel, dim3(nwg), dim3(NT), 0, st, ka);
    time_end(ctx, which, st);
    return check_launch(ctx, "ag_attn_kernel");
  };
  // Overlapped with a copy kernel of its own on the same CUs: two attention
  // workgroups (one of 2 NT threads, for the register count) and one copy
  // workgroup must fit on a CU together.
  static_assert(2 * LDS_BYTES + 1024 <= 160 * 1024, "two attention workgroups and a copy workgroup share a CU");
  const bool side_copy = mode == TSG_MODE_OVERLAP && o.pull_units <= 0 &&
                         co_resident(ctx, (const void*)ag_attn_kernel, 2 * NT, (const void*)ag_attn_copy_kernel, 256);
  switch (mode) {
    case TSG_MODE_OVERLAP: {
      if (!side_copy) return launch(caller, (int)n_units, n_tiles, 1, 0);
      Pair pr;
      tsg_status st = streams(ctx, o, &pr, caller);
      if (st == TSG_OK) st = fork(ctx, caller, pr);
      if (st != TSG_OK) return st;
      // On shared CUs the caller's stream waits for the attention kernel
      // alone (a join would put a barrier packet between consecutive calls'
      // kernels on its queue): its tiles wait for their head's own-chunk
      // slabs after their stores, so its end implies every arrival, and the
      // copy kernel's workgroups may then still be leaving their queue,
      // whose words only later such copies on the same side stream use.
      // With a timeline (copy rows are written after the arrivals) or a
      // debug skip mask the call joins.
      const bool detached = o.aux_cus < 0 && pr.main == caller && !o.timeline && o.skip_mask == 0;
      ka.wait_own_end = detached ? 1 : 0;
      // the copy first, so that its workgroups are dispatched while the
      // attention workgroups start on their own chunks
      const int copy_grid = o.aux_wgs > 0 ? std::min(o.aux_wgs, 4 * ctx->n_cus) : ctx->n_cus;
      ck.queue = ctx->d_queue + kCopyQueueSlot + (detached ? 0 : 2);
      ck.n_workers = (uint32_t)copy_grid;
      time_begin(ctx, 1, pr.aux);
      hipLaunchKernelGGL(ag_attn_copy_kernel, dim3(copy_grid), dim3(256), 0, pr.aux, ck, cv);
      time_end(ctx, 1, pr.aux);
      st = check_launch(ctx, "ag_attn_copy_kernel");
      if (st == TSG_OK) st = launch(pr.main, 0, n_tiles, 1, 0);
      if (st != TSG_OK || detached) return st;
      return join(ctx, caller, pr);
    }
    case TSG_MODE_SERIAL: {
      tsg_status st = launch(caller, (int)n_units, 0, 0, 1);
      return st != TSG_OK ? st : launch(caller, 0, n_tiles, 1, 0);
    }
    case TSG_MODE_COMPUTE_ONLY: return launch(caller, 0, n_tiles, 0, 0);
    default: return launch(caller, (int)n_units, 0, 0, 1);
  }
}
