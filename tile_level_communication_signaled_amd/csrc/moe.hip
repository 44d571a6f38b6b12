// MoE expert compute with the gate-weighted combine overlapped through
// tile-level signals.
//
// Digest page "Resource-aware Computation-Communication Overlap for
// multi-GPU ML Workloads", abstract on MoE expert compute overlapped with the
// return all-to-all: a persistent per-rank producer covers all local experts
// and emits output tiles with ready signals; a persistent consumer on a small
// CU partition moves them back towards token order as they become ready.
// "TileLink: Generating Efficient Compute-Communication Overlapping Kernels
// using Tile-Centric Primitives", section 4.1 (dynamic mapping: lookup tables
// filled at run time by the routing) and section 7.2 (GroupGEMM + Scatter +
// Topk-Reduce).
//
// Kernels (one call):
//   1. moe_count_kernel and moe_place_kernel (one workgroup per 256 pairs):
//      expert_counts, a stable counting sort of the pairs
//      p = t*k + s by expert (sorted_ids, order (expert, t, s)), and the
//      lookup tables of the padded layout: every expert's rows are padded
//      to a multiple of BM = 256, row block rb belongs to one expert,
//      row_pair[row] = pair id or -1, row_token[row] = token or -1,
//      pair_row[p] = padded row of pair p.
//   2. moe_producer_kernel (persistent, atomic work queue): first every "up"
//      tile (row block rb, 224 columns of I): gather x rows through row_token,
//      multiply by w_up[e], h = bf16(SiLU(u)); each arrives on the signal of
//      its row block.  Then every "down" tile (rb, 224 columns of H): acquire
//      the row block's signal (all up tiles of rb done), y = h w_down[e] in
//      fp32 (bf16 with stage_dtype = TSG_BF16) into the staging buffer,
//      release the tile's ready signal.
//   3. The combine (combine_unit), per down tile in queue order: acquire
//      its ready signal, and for every token whose other routed row lies in
//      this or an earlier tile (acquiring that tile's signal too) write
//      out[t] = fl(fl(g0 y0) + fl(g1 y1)) in slot order.  Every token is
//      written exactly once, by the later of its two tiles: no atomics and no
//      zero-fill of out.  In overlap mode on shared CUs the combine units are
//      queue items of the producer itself, after the down tiles, so they run
//      on any CU as soon as their tiles are ready; with a CU split they run
//      in moe_combine_kernel, a persistent consumer on its own partition.
#include <mutex>

#include "tsg_gemm.hpp"
#include "tsg_internal.hpp"
#include "tsg_moe_route.hpp"

using namespace tsg;

namespace {

constexpr int BM = 256;                 // row padding unit and tile rows
constexpr int BN_UP = 224;
constexpr int BN_DN = 224;
constexpr int kCombMaxRb = 4096;         // row blocks the combine's partner list can name
constexpr size_t kSigH = size_t(1) << 19;          // h row-block signals
constexpr size_t kSigReady = kSigH + 65536;         // ready signals of down tiles
constexpr size_t kSigEnd = kSigReady + 262144;

// Eight waves, two per SIMD, 112 accumulator registers each: with
// direct-to-LDS loads (K a multiple of 128) 4 x 2 waves of 64 x 112 on
// 16x16x32 fragments, else 8 x 1 waves of 32 x 224 on 32x32x16 (the register
// path).  The persistent kernel holds both tile paths and the combine.
template <bool DIRECT>
using CfgOf = std::conditional_t<DIRECT, TileCfg<BM, BN_UP, 4, 2, 16>, TileCfg<BM, BN_UP, 8, 1>>;
static_assert(BN_UP == BN_DN, "up and down tiles share one shape");
constexpr int kProdThreads = CfgOf<true>::NT;
static_assert(CfgOf<false>::NT == kProdThreads, "both layouts use eight waves");

// Workspace layout (byte offsets, 256-aligned).
struct Layout {
  size_t meta, offs, poffs, rb_expert, row_pair, row_token, pair_row, rb_mask, rb_order, h, y, total;
  int64_t n_rb_max, rows_max;
};

inline size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

Layout layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  Layout L;
  const int64_t pairs = T * k;
  L.n_rb_max = (pairs + E * (BM - 1) + BM - 1) / BM;
  L.rows_max = L.n_rb_max * BM;
  size_t o = 0;
  L.meta = o;      o += up256(64 * 4);
  L.offs = o;      o += up256((E + 1) * 4);
  L.poffs = o;     o += up256((E + 1) * 4);
  L.rb_expert = o; o += up256(L.n_rb_max * 4);
  L.row_pair = o;  o += up256(L.rows_max * 4);
  L.row_token = o; o += up256(L.rows_max * 4);
  L.pair_row = o;  o += up256(pairs * 4);
  L.rb_mask = o;   o += up256(L.n_rb_max * 4);
  L.rb_order = o;  o += up256(L.n_rb_max * 4);
  L.h = o;         o += up256(L.rows_max * I * 2);
  L.y = o;         o += up256(L.rows_max * H * 4);
  L.total = o;
  return L;
}

struct Ws : MoeTables {
  uint32_t* rb_mask;  // source ranks of each row block's tokens (remote-critical order only)
  int* rb_order;      // row blocks in producer order (remote-critical order only)
  uint16_t* h;
  float* y;
};

Ws bind(char* base, const Layout& L) {
  Ws w;
  w.meta = (int*)(base + L.meta);
  w.offs = (int*)(base + L.offs);
  w.poffs = (int*)(base + L.poffs);
  w.rb_expert = (int*)(base + L.rb_expert);
  w.row_pair = (int*)(base + L.row_pair);
  w.row_token = (int*)(base + L.row_token);
  w.pair_row = (int*)(base + L.pair_row);
  w.rb_mask = (uint32_t*)(base + L.rb_mask);
  w.rb_order = (int*)(base + L.rb_order);
  w.h = (uint16_t*)(base + L.h);
  w.y = (float*)(base + L.y);
  return w;
}

// --------------------------------------------------------------- producer
struct CombArgs {
  const float* topk_w;
  float* out;
  Ws ws;
  const uint64_t* sig_ready;
  SyncArgs sa;
  Timeline tl;
  int H, k;
  int n_dn_nt, n_rb_max;
  int wait;
  int y_bf16;             // y staging holds bf16 (else fp32)
  const int* rb_order;    // row block at each position of the producer order (null: identity)
};

struct ProdArgs {
  const uint16_t* x;
  const uint16_t* w_up;
  const uint16_t* w_down;
  Ws ws;
  uint64_t* sig_h;
  uint32_t* cnt_h;
  uint64_t* sig_ready;
  uint32_t* queue;        // ticket counter, then the exit counter (both zero between calls)
  SyncArgs sa;
  Timeline tl;
  int T, H, I;
  int n_up_nt, n_dn_nt;
  int n_rb_max;
  int n_items;            // up + down tiles, then (fused mode) combine units
  int n_prod_items;       // up + down tiles
  CombArgs comb;          // combine units run as queue items after the down tiles
  uint32_t skip_mask;     // row blocks (mod 32) whose up tiles never arrive (test hook)
  int y_bf16;             // y staging holds bf16 (else fp32)
  int h_l1_only;          // h rows are whole 128-byte lines: acquire invalidates L1 only
  const int* rb_order;    // row block at each position of the tile order (null: identity)
};


// ---------------------------------------------------------------- combine

// Combine consumer.  Unit = one down tile (BM rows x BN_DN columns of y),
// in the producer's order (row block major).  A token is combined by the
// higher-numbered of the two row blocks holding its slots (when both slots
// sit in one block, both rows write the same value): out[t] = g0 * y(slot
// 0) + g1 * y(slot 1), products and sum rounded in that order (an absent
// slot contributes 0).  The units come after every down tile in the
// producer's queue, so the partner tiles a unit waits for were taken
// before it, whatever the order of the row blocks.
//   1. Threads 0..BM-1 read the routing of the unit's rows (pair, partner
//      row, token, gates) into LDS, and list the partner row blocks that
//      precede this one (their tiles must be ready too), once each.
//   2. Wave 0 reads every listed partner tile's signal in one load per 64,
//      polls only those not yet published, and the workgroup acquires.
//   3. Each wave takes an equal share of the rows: eight rows at a time it
//      issues all sixteen 16-byte loads of y (both slots, this lane's 4
//      columns), then combines and stores them; with bf16 staging, sixteen
//      rows and thirty-two 8-byte loads at a time.
// Called by every thread of the workgroup with uniform (rb, nt); `scratch`
// is kCombScratch bytes of LDS owned by the caller for the call.
constexpr int kCombScratch = 8 * BM * 4 + 16;

// Four bf16 values (one 8-byte word of the y staging) as floats.
__device__ __forceinline__ float4 bf16x4_to_float4(uint64_t v) {
  return make_float4(__uint_as_float((uint32_t)(v & 0xffffu) << 16),
                     __uint_as_float((uint32_t)((v >> 16) & 0xffffu) << 16),
                     __uint_as_float((uint32_t)((v >> 32) & 0xffffu) << 16),
                     __uint_as_float((uint32_t)(v >> 48) << 16));
}

__device__ __forceinline__ void combine_unit(const CombArgs& a, int rb, int nt, char* scratch) {
  int* s_tok = (int*)scratch;
  int* s_own = s_tok + BM;
  int* s_oth = s_own + BM;
  float* s_g0 = (float*)(s_oth + BM);
  float* s_g1 = s_g0 + BM;
  uint32_t* s_seen = (uint32_t*)(s_g1 + BM);   // kCombMaxRb bits
  int* s_list = (int*)(s_seen + BM);
  int* s_nlist = s_list + BM;
  static_assert(kCombMaxRb / 32 <= BM, "partner bitmap must fit its LDS slot");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
  const uint64_t target = sig_target(a.sa.epoch, 1);
  if (a.wait && threadIdx.x < 64) wave_poll_ge(a.sig_ready + (int64_t)rb * a.n_dn_nt + nt, target, a.sa);
  for (int i = threadIdx.x; i < kCombMaxRb / 32; i += blockDim.x) s_seen[i] = 0u;
  if (threadIdx.x == 0) *s_nlist = 0;
  __syncthreads();
  if (threadIdx.x < BM) {
    const int row = rb * BM + threadIdx.x;
    const int p = a.ws.row_pair[row];
    int tok = -1, own = -1, oth = -1;
    float g0 = 0.f, g1 = 0.f;
    if (p >= 0) {
      const int pr = a.ws.pair_row[p ^ 1];   // the token's other slot (k == 2)
      const int prb = pr >= 0 ? pr / BM : -1;
      if (prb <= rb) {                       // else the later tile combines this token
        tok = p / a.k;
        own = (p & 1) ? pr : row;            // row of slot 0 (-1: slot dropped)
        oth = (p & 1) ? row : pr;            // row of slot 1
        g0 = a.topk_w[(int64_t)tok * a.k];
        g1 = a.topk_w[(int64_t)tok * a.k + 1];
        if (prb >= 0 && prb < rb) {
          const uint32_t bit = 1u << (prb & 31);
          if (!(atomicOr(&s_seen[prb >> 5], bit) & bit)) s_list[atomicAdd(s_nlist, 1)] = prb;
        }
      }
    }
    s_tok[threadIdx.x] = tok;
    s_own[threadIdx.x] = own;
    s_oth[threadIdx.x] = oth;
    s_g0[threadIdx.x] = g0;
    s_g1[threadIdx.x] = g1;
  }
  __syncthreads();
  if (a.wait && threadIdx.x < 64) {
    const int nl = __builtin_amdgcn_readfirstlane(*s_nlist);
    for (int i0 = 0; i0 < nl; i0 += 64) {
      const int i = i0 + lane;
      uint64_t v = ~0ull;
      int prb = 0;
      if (i < nl) {
        prb = s_list[i];
        v = __hip_atomic_load(a.sig_ready + (int64_t)prb * a.n_dn_nt + nt, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
      }
      uint64_t pending = __builtin_amdgcn_ballot_w64(v < target);
      while (pending) {
        const int l = (int)__builtin_ctzll(pending);
        pending &= pending - 1;
        const int q = __builtin_amdgcn_readlane(prb, l);
        wave_poll_ge(a.sig_ready + (int64_t)q * a.n_dn_nt + nt, target, a.sa);
      }
    }
  }
  __syncthreads();  // y is read with coherent loads: no cache invalidation
  const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
  const int col = nt * BN_DN + lane * 4;
  const bool col_ok = lane * 4 < BN_DN && col < a.H;
  const int rpw = BM / (int)(blockDim.x >> 6);   // rows per wave (a multiple of 16)
  // out[t] = fl(fl(g0 y0) + fl(g1 y1)) for the row's token, four columns
  auto emit = [&](int j, float4 y0, float4 y1) {
    const int tok = s_tok[j];
    if (tok >= 0 && col_ok) {
      const float g0 = s_g0[j], g1 = s_g1[j];
      float4 o;
      o.x = __fadd_rn(__fmul_rn(g0, y0.x), __fmul_rn(g1, y1.x));
      o.y = __fadd_rn(__fmul_rn(g0, y0.y), __fmul_rn(g1, y1.y));
      o.z = __fadd_rn(__fmul_rn(g0, y0.z), __fmul_rn(g1, y1.z));
      o.w = __fadd_rn(__fmul_rn(g0, y0.w), __fmul_rn(g1, y1.w));
      *(float4*)(a.out + (int64_t)tok * a.H + col) = o;
    }
  };
  if (a.y_bf16) {
    // bf16 staging: sixteen rows at a time, both slots' 8-byte loads issued
    // before any is used (32 in flight, as many bytes as the fp32 form)
    const uint16_t* yb = (const uint16_t*)a.ws.y;
#pragma unroll 1
    for (int g = 0; g < rpw / 16; ++g) {
      const int j0 = wave * rpw + g * 16;
      uint64_t w0[16], w1[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int own = s_own[j0 + j], oth = s_oth[j0 + j];
        w0[j] = 0;
        w1[j] = 0;
        if (s_tok[j0 + j] >= 0 && col_ok) {
          if (own >= 0) w0[j] = __hip_atomic_load((const uint64_t*)(yb + (int64_t)own * a.H + col),
                                                  __ATOMIC_RELAXED, TSG_SIG_SCOPE);
          if (oth >= 0) w1[j] = __hip_atomic_load((const uint64_t*)(yb + (int64_t)oth * a.H + col),
                                                  __ATOMIC_RELAXED, TSG_SIG_SCOPE);
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) emit(j0 + j, bf16x4_to_float4(w0[j]), bf16x4_to_float4(w1[j]));
    }
  } else {
#pragma unroll 1
    for (int g = 0; g < rpw / 8; ++g) {
      const int j0 = wave * rpw + g * 8;
      float4 v0[8], v1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int own = s_own[j0 + j], oth = s_oth[j0 + j];
        v0[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        v1[j] = v0[j];
        if (s_tok[j0 + j] >= 0 && col_ok) {
          if (own >= 0) v0[j] = load_coherent((const float4*)(a.ws.y + (int64_t)own * a.H + col));
          if (oth >= 0) v1[j] = load_coherent((const float4*)(a.ws.y + (int64_t)oth * a.H + col));
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) emit(j0 + j, v0[j], v1[j]);
    }
  }
  if (a.tl.buf && threadIdx.x == 0) timeline_put(a.tl, 9, (uint32_t)(rb << 16 | nt), t0, t1, wall_clock64());
  __syncthreads();  // LDS routing of this unit fully read before the caller reuses it
}

// Combine kernel (serial, combine-only and CU-split modes).  The unit loop is
// uniform: its trip values come from kernel arguments or are read first-lane.
__global__ void __launch_bounds__(256) moe_combine_kernel(const CombArgs a) {
  __shared__ __attribute__((aligned(16))) char scratch[kCombScratch];
  const int n_rb = __builtin_amdgcn_readfirstlane(a.ws.meta[0]);
  const int n_units = a.n_rb_max * a.n_dn_nt;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int ord = u / a.n_dn_nt, nt = u % a.n_dn_nt;
    if (ord >= n_rb) break;                  // units are rb-major: the rest are empty too
    const int rb = a.rb_order ? __builtin_amdgcn_readfirstlane(a.rb_order[ord]) : ord;
    combine_unit(a, rb, nt, scratch);
  }
}

// Persistent producer: up tiles, then down tiles, then (fused mode) the
// combine units, all from one ticket queue, row blocks in the tile order
// (plain, or remote-critical blocks first).  Every item waits only for earlier items (down tiles for their row
// block's up tiles, combine units for down tiles), which running workgroups
// took before it and complete without waiting on later ones.
template <bool DIRECT_UP, bool DIRECT_DN>
__global__ void __launch_bounds__(kProdThreads) moe_producer_kernel(const ProdArgs a) {
  using CfgUp = CfgOf<DIRECT_UP>;
  using CfgDn = CfgOf<DIRECT_DN>;
  constexpr int LUP = DIRECT_UP ? CfgUp::LDS_DIRECT : CfgUp::LDS_REGS;
  constexpr int LDN = DIRECT_DN ? CfgDn::LDS_DIRECT : CfgDn::LDS_REGS;
  __shared__ __attribute__((aligned(16))) char lds[LUP > LDN ? LUP : LDN];
  // Every value that steers a loop or branch around a barrier is made
  // wave-uniform (readfirstlane): values read from memory are otherwise
  // treated as divergent, and a divergent loop around barriers is
  // restructured by the compiler into a form whose `continue` edge skipped
  // the fetch of the next item (an endless loop).
  const int n_rb = __builtin_amdgcn_readfirstlane(a.ws.meta[0]);
  const int n_up = a.n_rb_max * a.n_up_nt;
  // Next queue item, identical in every thread.  The loop below has a single
  // back edge that always passes through this fetch (no `continue`).
  // The ticket goes through the first word of the tile buffer, which is free
  // between items: a tile's last LDS access precedes a barrier (the K loop's
  // last one, or the staged epilogue's own wave-local reads, which wave 0
  // finishes before thread 0 writes), and a combine unit ends with one.
  auto fetch = [&]() -> int {
    volatile int* s_item = (volatile int*)lds;
    if (threadIdx.x == 0) *s_item = (int)atomicAdd(a.queue, 1u);
    __syncthreads();
    const int v = __builtin_amdgcn_readfirstlane(*s_item);
    __syncthreads();
    return v;
  };
  for (int item = fetch(); item < a.n_items; item = fetch()) {
    const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
    // item -> (kind, position ord in the tile order, column tile); then
    // ord -> row block (positions past the blocks in use stay past them)
    const bool comb = item >= a.n_prod_items;
    const bool up = item < n_up;
    const int j = comb ? item - a.n_prod_items : up ? item : item - n_up;
    const int ntc = up ? a.n_up_nt : a.n_dn_nt;
    const int ord = j / ntc, nt = j - ord * ntc;
    const int rb = a.rb_order && ord < n_rb ? __builtin_amdgcn_readfirstlane(a.rb_order[ord]) : ord;
    // no `continue`: the loop keeps a single back edge through the fetch
    if (comb) {                              // combine unit (fused mode)
      if (rb < n_rb) combine_unit(a.comb, rb, nt, lds);
    } else {
      if (rb < n_rb && up) {
        const int e = __builtin_amdgcn_readfirstlane(a.ws.rb_expert[rb]);
        const int col0 = nt * BN_UP;
        // rows past the expert's last pair are padding
        const int valid = __builtin_amdgcn_readfirstlane(
            min(BM, a.ws.offs[e + 1] - a.ws.offs[e] - (rb * BM - a.ws.poffs[e])));
        typename GemmTile<CfgUp>::Acc acc;
        const ARowsGather ar{a.x, a.H, a.ws.row_token + (int64_t)rb * BM};
        const uint16_t* B = a.w_up + (int64_t)e * a.H * a.I;
        if (DIRECT_UP)
          GemmTile<CfgUp>::run_direct(ar, B, a.I, col0, a.I, a.H, lds, acc, NoHook(), valid);
        else
          GemmTile<CfgUp>::run_regs(ar, B, a.I, col0, a.I, a.H, lds, acc);
        // h = bf16(SiLU(u)), SiLU(u) = u / (1 + e^-u)
        GemmTile<CfgUp>::template store_bf16_staged<sizeof(lds), true>(
            acc, lds, a.ws.h + (int64_t)rb * BM * a.I + col0, a.I, BM, a.I - col0,
            [](float u) { return u / (1.0f + expf(-u)); });
        block_coherent_complete();
        if (threadIdx.x == 0) {
          if (!((a.skip_mask >> (rb & 31)) & 1u))
            sig_arrive_counted_coherent(a.cnt_h + rb, a.sig_h + rb, (uint32_t)a.n_up_nt, a.sa.epoch);
          if (a.tl.buf) timeline_put(a.tl, 7, (uint32_t)(rb << 16 | nt), t0, t0, wall_clock64());
        }
      } else if (rb < n_rb) {
        const int e = __builtin_amdgcn_readfirstlane(a.ws.rb_expert[rb]);
        const int col0 = nt * BN_DN;
        block_wait_lines(a.sig_h + rb, sig_target(a.sa.epoch, (uint32_t)a.n_up_nt), a.sa, a.h_l1_only != 0);
        const uint64_t t1 = a.tl.buf ? wall_clock64() : 0;
        // rows past the expert's last pair are padding: not computed (whole
        // waves of them) and not stored
        const int valid = __builtin_amdgcn_readfirstlane(
            min(BM, a.ws.offs[e + 1] - a.ws.offs[e] - (rb * BM - a.ws.poffs[e])));
        typename GemmTile<CfgDn>::Acc acc;
        const ARowsLinear ar{a.ws.h, a.I, rb * BM, a.n_rb_max * BM};
        const uint16_t* B = a.w_down + (int64_t)e * a.I * a.H;
        if (DIRECT_DN)
          GemmTile<CfgDn>::run_direct(ar, B, a.H, col0, a.H, a.I, lds, acc, NoHook(), valid);
        else
          GemmTile<CfgDn>::run_regs(ar, B, a.H, col0, a.H, a.I, lds, acc);
        const int H = a.H;
        if (a.y_bf16) {
          uint16_t* yb = (uint16_t*)a.ws.y + (int64_t)rb * BM * H + col0;
          GemmTile<CfgDn>::template store_bf16_staged<sizeof(lds), true>(
              acc, lds, yb, H, valid, H - col0, [](float v) { return v; });
        } else {
          GemmTile<CfgDn>::template store_f32<true>(acc, a.ws.y + (int64_t)rb * BM * H + col0, H, valid, H - col0);
        }
        block_coherent_complete();
        if (threadIdx.x == 0) {
          sig_publish_coherent(a.sig_ready + (int64_t)rb * a.n_dn_nt + nt, a.sa.epoch, 1);
          if (a.tl.buf) timeline_put(a.tl, 8, (uint32_t)(rb << 16 | nt), t0, t1, wall_clock64());
        }
      }
    }
  }
  // Every workgroup leaves after its failing ticket, so once the last one has
  // left no claim of this call is outstanding: it resets both counters for
  // the next call.  A launch that never ran leaves them at zero.
  if (threadIdx.x == 0 && atomicAdd(a.queue + 1, 1u) == gridDim.x - 1) {
    __hip_atomic_store(a.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.queue + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool U, bool D>
void launch_prod(const ProdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((moe_producer_kernel<U, D>), dim3(grid), dim3(kProdThreads), 0, s, a);
}

}  // namespace

// Workspace of moe_expert_combine_noalloc: a static device array, one copy
// per GPU, held until the process ends.  Host code never uses the array's
// name as an address (on the host it is a stand-in, not device memory): its
// device address is looked up once per device, below, and kept.
namespace {
static __device__ __align__(256) char scratch[TSG_MOE_NOALLOC_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

tsg_status tsg_moe_scratch_init(tsg_ctx* ctx) {
  if (ctx->device < 0 || ctx->device >= 64) return tsgh::fail(ctx, TSG_E_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[ctx->device]) {
    // called with ctx->device current (tsg_ctx_create)
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return tsgh::hip_fail(ctx, e, "hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr & 255u))
      return tsgh::fail(ctx, TSG_E_HIP, "scratch buffer at an unexpected address %p", ptr);
    g_scratch_ptr[ctx->device] = ptr;
  }
  ctx->d_noalloc_ws = g_scratch_ptr[ctx->device];
  return TSG_OK;
}

size_t tsg_moe_workspace(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  if (T < 1 || H < 8 || I < 8 || E < 1 || E > kMaxExperts || k != 2) return 0;
  return layout(T, H, I, E, k).total;
}

bool tsg_moe_layout_fields(const int64_t* d, int64_t* out, int n) {
  if (!d || !out || n < 0 || tsg_moe_workspace(d[0], d[1], d[2], d[3], d[4]) == 0) return false;
  const Layout L = layout(d[0], d[1], d[2], d[3], d[4]);
  const int64_t f[TSG_MOE_LAYOUT_N] = {(int64_t)L.meta,     (int64_t)L.offs,     (int64_t)L.poffs,
                                       (int64_t)L.rb_expert, (int64_t)L.row_pair, (int64_t)L.row_token,
                                       (int64_t)L.pair_row,  (int64_t)L.h,        (int64_t)L.y,
                                       (int64_t)L.total,     L.rows_max,          L.n_rb_max,
                                       (int64_t)BM,          (int64_t)L.rb_order, (int64_t)L.rb_mask};
  for (int i = 0; i < n && i < TSG_MOE_LAYOUT_N; ++i) out[i] = f[i];
  return true;
}

tsg_status tsg_op_moe(tsg_ctx* ctx, const void* x, const int32_t* topk_ids, const float* topk_w,
                      const void* w_up, const void* w_down, float* out, int32_t* expert_counts,
                      int32_t* sorted_ids, void* workspace, size_t workspace_bytes, int T, int H,
                      int I, int E, int k, const tsg_opts* opts, int mode, void* stream, bool noalloc) {
  using namespace tsgh;
  if (noalloc) {
    // the library's static buffer stands in for the workspace argument
    workspace = ctx->d_noalloc_ws;
    workspace_bytes = TSG_MOE_NOALLOC_BYTES;
    if (!workspace) return fail(ctx, TSG_E_HIP, "moe_expert_combine_noalloc: no scratch buffer on this device");
  }
  if (!x || !topk_ids || !topk_w || !w_up || !w_down || !out || !expert_counts || !sorted_ids)
    return fail(ctx, TSG_E_INVALID, "moe_expert_combine: null pointer");
  if (mode < TSG_MODE_OVERLAP || mode > TSG_MODE_COMM_ONLY) return fail(ctx, TSG_E_INVALID, "bad mode");
  if (k != 2) return fail(ctx, TSG_E_UNSUPPORTED, "moe_expert_combine supports k == 2 only");
  if (T < 1 || E < 1 || E > kMaxExperts || H < 8 || I < 8 || H % 8 || I % 8)
    return fail(ctx, TSG_E_SHAPE, "moe_expert_combine: bad shape T=%d H=%d I=%d E=%d", T, H, I, E);
  if ((int64_t)T * k > kRouteMaxPairs)
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_expert_combine: T * k above %d routed pairs", kRouteMaxPairs);
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(out) ||
      !aligned16(workspace))
    return fail(ctx, TSG_E_ALIGN, "moe_expert_combine: pointers must be 16-byte aligned");
  const Layout L = layout(T, H, I, E, k);
  if (noalloc && L.total > workspace_bytes)
    return fail(ctx, TSG_E_WORKSPACE,
                "moe_expert_combine_noalloc: these dims need %zu bytes of workspace, above the %zu-byte static buffer",
                L.total, workspace_bytes);
  if (!workspace || workspace_bytes < L.total)
    return fail(ctx, TSG_E_WORKSPACE, "workspace of %zu bytes needed", L.total);
  if ((int64_t)T * H * 2 >= (int64_t(1) << 32) || (int64_t)H * I * 2 >= (int64_t(1) << 32) ||
      L.rows_max * I * 2 >= (int64_t(1) << 32))
    return fail(ctx, TSG_E_UNSUPPORTED, "operands of 4 GiB or more are not supported");
  const int n_up_nt = (I + BN_UP - 1) / BN_UP, n_dn_nt = (H + BN_DN - 1) / BN_DN;
  if (L.n_rb_max > kCombMaxRb)
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_expert_combine: more than %d row blocks", kCombMaxRb);
  if ((size_t)L.n_rb_max > kSigReady - kSigH || (size_t)L.n_rb_max * n_dn_nt > kSigEnd - kSigReady ||
      kSigEnd > ctx->n_sig)
    return fail(ctx, TSG_E_UNSUPPORTED, "too many tiles for the signal pool");

  const Opts o = resolve(opts, -1);
  if (o.stage_dtype != TSG_F32 && o.stage_dtype != TSG_BF16)
    return fail(ctx, TSG_E_INVALID, "moe_expert_combine: stage_dtype must be TSG_F32 or TSG_BF16");
  if (o.ep_ranks < 0 || o.ep_ranks > kRouteMaxRanks ||
      (o.ep_ranks > 0 && (T % o.ep_ranks || o.ep_rank < 0 || o.ep_rank >= o.ep_ranks)))
    return fail(ctx, TSG_E_INVALID,
                "moe_expert_combine: need 0 <= ep_ranks <= %d, T a multiple of ep_ranks and 0 <= ep_rank < ep_ranks "
                "(T=%d ep_ranks=%d ep_rank=%d)", kRouteMaxRanks, T, o.ep_ranks, o.ep_rank);
  if (o.ep_ranks > 0 && L.n_rb_max > kRouteMaskBlocks)
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_expert_combine: remote-critical order supports %d row blocks",
                kRouteMaskBlocks);
  // Everything on the caller's stream: no stream is created and no memset
  // is recorded (the timeline counter would need one).
  if (noalloc && (o.aux_cus > 0 || o.timeline))
    return fail(ctx, TSG_E_UNSUPPORTED, "moe_expert_combine_noalloc runs on shared CUs without a timeline");
  TSG_HIP(ctx, hipSetDevice(ctx->device));
  hipStream_t caller = (hipStream_t)stream;
  ++ctx->epoch;
  time_reset(ctx);
  const Ws ws = bind((char*)workspace, L);
  const SyncArgs sa = sync_args(ctx, o);
  const Timeline tl = timeline(ctx, o);
  if (o.timeline) TSG_HIP(ctx, hipMemsetAsync(ctx->d_timeline_n, 0, sizeof(uint32_t), caller));

  RouteArgs ra;
  ra.ids = topk_ids;
  ra.counts = expert_counts;
  ra.sorted_ids = sorted_ids;
  ra.ws = ws;
  ra.status = ctx->d_status;
  ra.P = T * k;
  ra.E = E;
  ra.k = k;
  ra.G = (ra.P + kRouteThreads - 1) / kRouteThreads;
  ra.rows_max = L.rows_max;
  ra.n_rb_max = L.n_rb_max;
  // remote-critical order: each row block's source ranks, then the order
  // (blocks with a token of another rank first)
  const bool prio = o.ep_ranks > 0;
  ra.rb_mask = prio ? ws.rb_mask : nullptr;
  ra.tokens_per_rank = prio ? T / o.ep_ranks : 1;
  RbOrderArgs oa;
  oa.meta = ws.meta;
  oa.rb_mask = ws.rb_mask;
  oa.rb_order = ws.rb_order;
  for (int c = 0; c < kRouteMaxRanks; ++c) oa.key_of[c] = c == o.ep_rank ? 1 : 0;
  oa.R = prio ? o.ep_ranks : 1;
  oa.min_key = 1;
  // the per-block counts use the start of the y staging area, which only
  // the down tiles write, after the routing (G E ints, far below its size)
  ra.blk = (int*)ws.y;

  ProdArgs pa;
  pa.x = (const uint16_t*)x;
  pa.w_up = (const uint16_t*)w_up;
  pa.w_down = (const uint16_t*)w_down;
  pa.ws = ws;
  pa.sig_h = ctx->d_sig + kSigH;
  pa.cnt_h = ctx->d_cnt + kSigH;
  pa.sig_ready = ctx->d_sig + kSigReady;
  pa.queue = ctx->d_queue;
  pa.sa = sa;
  pa.tl = tl;
  pa.T = T;
  pa.H = H;
  pa.I = I;
  pa.n_up_nt = n_up_nt;
  pa.n_dn_nt = n_dn_nt;
  pa.n_rb_max = (int)L.n_rb_max;
  pa.n_prod_items = (int)(L.n_rb_max * (n_up_nt + n_dn_nt));
  pa.n_items = pa.n_prod_items;
  pa.skip_mask = o.skip_mask;
  pa.y_bf16 = o.stage_dtype == TSG_BF16 ? 1 : 0;
  pa.h_l1_only = ((uintptr_t)ws.h % 128 == 0 && ((int64_t)I * 2) % 128 == 0) ? 1 : 0;
  pa.rb_order = prio ? ws.rb_order : nullptr;

  CombArgs ca;
  ca.topk_w = topk_w;
  ca.out = out;
  ca.ws = ws;
  ca.sig_ready = pa.sig_ready;
  ca.sa = sa;
  ca.tl = tl;
  ca.H = H;
  ca.k = k;
  ca.n_dn_nt = n_dn_nt;
  ca.n_rb_max = (int)L.n_rb_max;
  ca.y_bf16 = pa.y_bf16;
  // comm-only runs on the previous call's tables, whose order may not exist:
  // the combine's results do not depend on its order
  ca.rb_order = mode == TSG_MODE_COMM_ONLY ? nullptr : pa.rb_order;

  auto route = [&]() -> tsg_status {
    hipLaunchKernelGGL(moe_count_kernel<BM>, dim3(ra.G), dim3(kRouteThreads), 0, caller, ra);
    tsg_status rs = check_launch(ctx, "moe_count_kernel");
    if (rs != TSG_OK) return rs;
    hipLaunchKernelGGL(moe_place_kernel<BM>, dim3(ra.G), dim3(kRouteThreads), 0, caller, ra);
    rs = check_launch(ctx, "moe_place_kernel");
    if (rs != TSG_OK || !prio) return rs;
    hipLaunchKernelGGL(moe_rb_order_kernel<>, dim3(1), dim3(256), 0, caller, oa);
    return check_launch(ctx, "moe_rb_order_kernel");
  };
  auto produce = [&](hipStream_t s, int nwg) -> tsg_status {
    const bool du = H % 128 == 0, dd = I % 128 == 0;
    time_begin(ctx, 0, s);
    if (du && dd) launch_prod<true, true>(pa, nwg, s);
    else if (du) launch_prod<true, false>(pa, nwg, s);
    else if (dd) launch_prod<false, true>(pa, nwg, s);
    else launch_prod<false, false>(pa, nwg, s);
    time_end(ctx, 0, s);
    return check_launch(ctx, "moe_producer_kernel");
  };
  auto combine = [&](hipStream_t s, int nwg, int wait) -> tsg_status {
    ca.wait = wait;
    time_begin(ctx, 1, s);
    hipLaunchKernelGGL(moe_combine_kernel, dim3(nwg), dim3(256), 0, s, ca);
    time_end(ctx, 1, s);
    return check_launch(ctx, "moe_combine_kernel");
  };

  tsg_status st = TSG_OK;
  if (mode != TSG_MODE_COMM_ONLY) st = route();
  if (st != TSG_OK) return st;
  if (mode == TSG_MODE_OVERLAP && o.aux_cus < 0) {
    // Shared CUs: the combine units are queue items of the producer itself.
    ca.wait = 1;
    pa.comb = ca;
    pa.n_items = pa.n_prod_items + (int)(L.n_rb_max * n_dn_nt);
    return produce(caller, o.aux_wgs > 0 ? o.aux_wgs : ctx->n_cus);
  }
  if (mode == TSG_MODE_SERIAL || mode == TSG_MODE_COMPUTE_ONLY) {
    st = produce(caller, ctx->n_cus);
    if (st == TSG_OK && mode == TSG_MODE_SERIAL) st = combine(caller, ctx->n_cus * 2, 1);
    return st;
  }
  // Here the mode is COMM_ONLY, or OVERLAP on a CU split.  The combine alone
  // on shared CUs (always so in the no-alloc form) has nothing to overlap
  // with, so it runs on the caller's stream.
  if (o.aux_cus < 0) return combine(caller, o.aux_wgs > 0 ? o.aux_wgs : ctx->n_cus * 2, 0);
  Pair pr;
  st = streams(ctx, o, &pr);
  if (st != TSG_OK) return st;
  // Combine workgroups: overlap on shared CUs keeps the consumer small (64);
  // the combine alone uses the whole GPU, as in serial mode.
  const int nwg_c = o.aux_wgs > 0 ? o.aux_wgs
                    : mode == TSG_MODE_COMM_ONLY ? (o.aux_cus < 0 ? ctx->n_cus * 2 : pr.aux_cus * 4)
                    : (o.aux_cus < 0 ? 64 : pr.aux_cus * 4);
  st = fork(ctx, caller, pr);
  if (st != TSG_OK) return st;
  // Producer first, consumer second: the producer's only waits are on its own
  // earlier queue items, which are already running.
  if (mode == TSG_MODE_OVERLAP) st = produce(pr.main, pr.main_cus);
  if (st == TSG_OK) st = combine(pr.aux, nwg_c, mode == TSG_MODE_OVERLAP ? 1 : 0);
  tsg_status sj = join(ctx, caller, pr);
  return st != TSG_OK ? st : sj;
}
