// MFMA GEMM tile engine for gfx950 (CDNA4).
//
// One workgroup computes a BM x BN tile of C = A * B with A [M x K] and
// B [K x N] both row-major bf16, accumulating in fp32 with
// v_mfma_f32_32x32x16_bf16 (or, for tiles whose fragment size MF is 16 and
// only on the main path, v_mfma_f32_16x16x32_bf16).  The K loop moves BK = 64
// columns of A and rows of B per step through LDS:
//
//   * A is staged as BM rows x 8 chunks of 16 bytes (8 bf16 along k).  On the
//     main path A goes straight from global memory to LDS (16-byte
//     global_load_lds), through a three-stage ring, so it costs no registers.
//   * On the main path B also goes straight to LDS, row-major (64 rows of k x
//     BN columns), through a two-stage ring, and the MFMA B fragments are read
//     with the LDS transpose read (ds_read_b64_tr_b16), two per fragment.
//   * On the fallback path B is staged transposed, as BN rows (one per output
//     column n) x 8 chunks of 8 consecutive k: each thread loads an 8 (k) x
//     8 (n) block with eight coalesced 16-byte row loads and repacks it with
//     byte permutes.
//   * Chunk c of LDS row r is stored at chunk position c ^ ((r / 2) mod 8), so
//     the 16-byte reads of 16 consecutive rows (and the transposed B writes,
//     issued in an order that alternates row parity across lanes) hit
//     distinct bank groups.
//
// Waves are arranged WM x WN; a wave owns a (BM/WM) x (BN/WN) sub-tile made of
// 32x32 MFMA fragments.  Operand layout of the 32x32x16 bf16 MFMA: lane l
// supplies row (l mod 32) of A and column (l mod 32) of B, with the 8 k values
// 8*(l / 32) .. 8*(l / 32) + 7 of the current 16-wide k step.  The fp32 result
// fragment gives lane l column (l mod 32) and, in register v, row
// 8*(v / 4) + 4*(l / 32) + (v mod 4).
//
// Rows beyond M read a stand-in row of the operand instead, and columns beyond
// N read the operand's last 8 columns (main path) or zeros (fallback path);
// their results are never stored (N must be a multiple of 8).  The main path
// needs K to be a multiple of 128; the fallback path (A staged through
// registers too, one step of prefetch) zero-fills k beyond K (K a multiple of
// 8).  The pages ask tile-level single-device kernels to coalesce global
// accesses, keep LDS free of bank conflicts, pipeline loads against compute
// and use the matrix units ([TL] section 4.3).
#pragma once

#include <type_traits>

#include "tsg_device.hpp"

namespace tsg {

// MF: edge of the MFMA fragments, 32 (v_mfma_f32_32x32x16_bf16, four k steps
// of 16 per BK step) or 16 (v_mfma_f32_16x16x32_bf16, two k steps of 32).
template <int BM_, int BN_, int WM_, int WN_, int MF_ = 32>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_;
  static constexpr int BK = 64;
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / MF, FN = WTN / MF;
  static constexpr int KS = BK / (MF == 32 ? 16 : 32);  // MFMA k steps per BK step
  static_assert(MF == 32 || MF == 16, "fragments of 32 or 16");
  static constexpr int A_STAGE = BM * BK * 2;
  static constexpr int B_STAGE = BN * BK * 2;
  static constexpr int LDS_DIRECT = 3 * A_STAGE + 2 * B_STAGE;
  static constexpr int LDS_REGS = 2 * (A_STAGE + B_STAGE);
  static constexpr int A_CH = BM * 8;               // 16-byte chunks per A stage
  static constexpr int A_PT = (A_CH + NT - 1) / NT; // chunks per thread (register path)
  static constexpr int A_BLK = BM / 8;              // 1 KB blocks of 8 rows per A stage
  static constexpr int A_BPW = (A_BLK + NW - 1) / NW;  // blocks per wave (direct path)
  static constexpr int B_BL = BN;                   // 8x8 blocks per B stage
  static constexpr int B_PT = (B_BL + NT - 1) / NT; // blocks per thread
  static constexpr int VM_PER_STEP = A_BPW + 8 * B_PT;  // VMEM ops per thread per step
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the fragment");
  static_assert(BN % 8 == 0 && BM % 8 == 0, "BM and BN must be multiples of 8");
  static_assert(LDS_REGS <= 160 * 1024, "LDS budget of one CU exceeded");
  static_assert(VM_PER_STEP < 64, "too many loads per step for one wait count");
};

// threadIdx.x through an empty asm: values derived from it are recomputed
// where they are used instead of being hoisted out of enclosing loops.
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Physical 16-byte position of logical chunk `chunk` of LDS row `row`.  A
// row is 128 bytes; with 64 banks of 4 bytes, the 16 lanes served together by
// a 16-byte access hit distinct banks iff their (row parity, position) pairs
// are distinct.  The MFMA fragment reads touch 16 consecutive rows at one
// logical chunk, so the position is XORed with (row / 2) mod 8.
__device__ __forceinline__ int lds_pos(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ uint32_t lds_swz(int row, int chunk) {
  return (uint32_t)(((row << 3) | lds_pos(row, chunk)) << 4);
}

// lo = a.lo16, hi = b.lo16
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// lo = a.hi16, hi = b.hi16
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier of the K pipeline.  It waits for this wave's LDS
// accesses only, so global loads still in flight (the prefetch of later
// steps) are not drained, as __syncthreads() (whose fence also covers the
// direct-to-LDS loads, counted with global loads) would do.  Direct-to-LDS
// loads a step depends on are waited for explicitly (wait_vmcnt) before it.
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Source rows of the A operand of one tile.  row(r) gives the element offset
// of tile row r in `base`, or -1 for a row outside the operand.
struct ARowsLinear {
  const uint16_t* base;
  int64_t ld;
  int row0;
  int M;
  __device__ __forceinline__ int64_t row(int r) const {
    const int g = row0 + r;
    return g < M ? (int64_t)g * ld : (int64_t)-1;
  }
  // Row read in place of rows outside the operand: the operand's last row,
  // which belongs to the tile, so it is covered by whatever the tile waited
  // for before loading.
  __device__ __forceinline__ int64_t stand_in() const { return (int64_t)(M - 1) * ld; }
};

// Gathered rows: idx[r] is the source row index (or < 0 for no row).  Rows
// with no source read row `stand` of the operand instead (their results are
// never stored); when the operand is written while the tile runs, `stand`
// must be a row the tile waited for.
struct ARowsGather {
  const uint16_t* base;
  int64_t ld;
  const int* idx;
  int stand = 0;
  __device__ __forceinline__ int64_t row(int r) const {
    const int g = idx[r];
    return g >= 0 ? (int64_t)g * ld : (int64_t)-1;
  }
  __device__ __forceinline__ int64_t stand_in() const { return (int64_t)stand * ld; }
};

// Called with the first K column k0 of every step, in increasing order, just
// before that step's A loads are issued: a consumer whose A arrives in column
// slabs waits there for the slab's signal.  The K loops take the hook by
// reference, so state it keeps (the time spent waiting) is the caller's
// after the loop.
struct NoHook {
  __device__ __forceinline__ void before_a(int) {}
};

template <class Cfg>
struct GemmTile {
  using AccV = std::conditional_t<Cfg::MF == 32, f32x16_t, f32x4_t>;
  static constexpr int ACC_N = Cfg::MF == 32 ? 16 : 4;  // accumulator registers per fragment
  using Acc = AccV[Cfg::FM][Cfg::FN];

  struct BRegs {
    u32x4_t b[Cfg::B_PT][8];
  };

  __device__ __forceinline__ static void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
        for (int v = 0; v < ACC_N; ++v) acc[i][j][v] = 0.f;
  }

  // Thread q of a B stage moves the 8 x 8 block at k block (q mod 8) and n
  // block (q / 8): each of its 8 row loads is one 16-byte piece of a 128-byte
  // run that 8 consecutive lanes cover.  boff = byte offset of the block's
  // first element relative to row k0 of B (fixed for the whole K loop).
  struct BAddr {
    uint32_t boff[Cfg::B_PT];
    bool ok[Cfg::B_PT];
    int kb[Cfg::B_PT];
  };

  __device__ __forceinline__ static void b_addr(BAddr& ba, int64_t ldb, int col0, int N) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Cfg::B_PT; ++i) {
      const int q = tid + i * Cfg::NT;
      const int kb = q & 7;
      const int n = (q >> 3) * 8;
      ba.kb[i] = kb;
      ba.ok[i] = (q < Cfg::B_BL) && (col0 + n < N);
      ba.boff[i] = (uint32_t)(((int64_t)kb * 8 * ldb + col0 + n) * 2);
    }
  }

  // Global loads of one 64 x BN step of B into registers.  CHECK_K: zero the
  // rows at or beyond K.
  template <bool CHECK_K>
  __device__ __forceinline__ static void load_b(BRegs& rg, const BAddr& ba,
                                                const uint16_t* __restrict__ B, int64_t ldb, int K,
                                                int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const char* row = (const char*)B + (int64_t)(k0 + j) * ldb * 2;  // uniform
#pragma unroll
      for (int i = 0; i < Cfg::B_PT; ++i) {
        const bool ok = ba.ok[i] && (!CHECK_K || k0 + ba.kb[i] * 8 + j < K);
        if (ok)
          rg.b[i][j] = *(const u32x4_t*)(row + ba.boff[i]);
        else
          rg.b[i][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  // Transpose the 8x8 blocks in registers and write them to a B stage.  LDS
  // row n + s holds output column n + s.  Lanes whose n block is odd write
  // their rows in the order 1,0,3,2,... instead of 0,1,2,3,..., so that each
  // write instruction covers both row parities (see lds_swz).
  __device__ __forceinline__ static void store_b(const BRegs& rg, char* lb) {
    const int tid = threadIdx.x;
    constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;
#pragma unroll
    for (int i = 0; i < Cfg::B_PT; ++i) {
      const int q = tid + i * Cfg::NT;
      if (q < Cfg::B_BL) {
        const int kb = q & 7;
        const int n = (q >> 3) * 8;
        const int par = (q >> 3) & 1;
        const uint32_t s0 = par ? HI : LO, s1 = par ? LO : HI;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          u32x4_t v0, v1;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            v0[p] = __builtin_amdgcn_perm(rg.b[i][2 * p + 1][m], rg.b[i][2 * p][m], s0);
            v1[p] = __builtin_amdgcn_perm(rg.b[i][2 * p + 1][m], rg.b[i][2 * p][m], s1);
          }
          *(u32x4_t*)(lb + lds_swz(n + 2 * m + par, kb)) = v0;
          *(u32x4_t*)(lb + lds_swz(n + 2 * m + (par ^ 1), kb)) = v1;
        }
      }
    }
  }

  // One BK step from LDS: 4 k sub-steps of 16.  The fragments of sub-step
  // ks + 1 are read before the MFMAs of sub-step ks are issued.
  __device__ __forceinline__ static void compute(const char* la, const char* lb, Acc& acc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    bf16x8_t af[2][Cfg::FM], bfr[2][Cfg::FN];
    auto rd = [&](int buf, int ks) {
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
        af[buf][i] = *(const bf16x8_t*)(la + lds_swz(wm0 + i * 32 + l32, 2 * ks + hi));
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        bfr[buf][j] = *(const bf16x8_t*)(lb + lds_swz(wn0 + j * 32 + l32, 2 * ks + hi));
    };
    rd(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) rd((ks + 1) & 1, ks + 1);
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j],
                                                               acc[i][j], 0, 0, 0);
    }
    // Instruction order: the fragment reads of sub-step ks + 1 are spread
    // between the MFMAs of sub-step ks, so that the LDS latency is covered by
    // matrix work instead of being waited out before it (one wave per SIMD
    // leaves no other wave to cover it).
    constexpr int NR = Cfg::FM + Cfg::FN, NM = Cfg::FM * Cfg::FN;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // reads of sub-step 0
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM > NR ? NM - NR : 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }

  // Fragment reads of a B stage laid out row-major, [BK rows (k)] x [BN
  // columns (n)], with the LDS transpose read: one ds_read_b64_tr_b16 gives a
  // lane four consecutive k of one column.  In each group of 16 lanes, lane
  // 4i + q points at row i, columns 4q..4q+3 of a 4 x 16 block, and lane
  // 4q + e receives column 4q + e of rows 0..3.  With the block's rows at
  // k = 16 ks + 8 (l / 32) + 4 t and its columns at n = 16 ((l / 16) mod 2)
  // of the fragment, lane l ends up with column (l mod 32) and k values
  // 8 (l / 32) .. + 7 of sub-step ks (t = 0, 1): the MFMA B operand layout.
  // B stages are row-major with BN columns.  When a row is a multiple of 128
  // bytes every row starts at the same bank, and the four rows that one
  // transpose read touches collide: half a wave reads 64 bytes of each of
  // four rows, which fill the 64 banks only if the rows' pieces land on
  // different banks.  The 16-byte chunk c of row r is then stored at
  // position c ^ (4 (r mod 4)) (rows of a multiple of 256 bytes) or
  // c ^ (2 (r mod 4)) (rows of an odd multiple of 128 bytes, which leaves a
  // two-way overlap); chunks are permuted within aligned groups of 16 or 8,
  // so a row keeps its place.
  // With 16-column fragments one half wave reads rows 8 g .. 8 g + 3 for
  // g = 0, 1 (32 bytes of each); rows eight apart start at the same bank
  // whenever BN is a multiple of 16, and (r mod 4) does not tell them
  // apart, so chunk c of a row with bit 3 set is moved by a further XOR
  // with 2 (32 bytes over, within its aligned group of four chunks): with
  // rows of a multiple of 256 bytes the half wave's eight rows then take
  // the sixteen 16-byte slots of one 256-byte bank cycle once each.
  static constexpr int B_SWZ = Cfg::BN % 128 == 0 ? 4 : Cfg::BN % 64 == 0 ? 2 : 0;
  static constexpr int B_SWZ8 = (Cfg::MF == 16 && B_SWZ != 2 && Cfg::BN % 32 == 0) ? 2 : 0;
  __device__ __forceinline__ static int b_swz(int row) {
    return B_SWZ * (row & 3) ^ B_SWZ8 * ((row >> 3) & 1);
  }

  // LDS byte offset of this lane's transpose reads of B fragment j (32
  // columns at wn0 + 32 j), step 0: lane 4i + q of each 16-lane group points
  // at row i, columns 4q .. 4q + 3; lanes 16-31 take the next 16 columns and
  // lanes 32-63 rows 8-11.  The second read of a fragment is 4 rows further,
  // step ks 16 rows further (neither changes row mod 4).
  // With 16-column fragments (MF = 16) the four 16-lane groups take k rows
  // 8 g .. 8 g + 7 of the 32-wide k step (two reads of four rows) and the
  // same 16 columns: lane l ends with column (l mod 16) and k values
  // 8 (l / 16) .. + 7, the B operand layout of the 16x16x32 MFMA.
  __device__ __forceinline__ static void tr_lane_offsets(int wn0, int lane, uint32_t (&off)[Cfg::FN]) {
    const int hi = lane >> 5, g = lane >> 4, sl = lane & 15;
    const int row = Cfg::MF == 32 ? 8 * hi + (sl >> 2) : 8 * g + (sl >> 2);
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int col = Cfg::MF == 32 ? wn0 + 32 * j + 16 * (g & 1) + 4 * (sl & 3) : wn0 + 16 * j + 4 * (sl & 3);
      const int chunk = (col >> 3) ^ b_swz(row);
      off[j] = (uint32_t)((row * Cfg::BN + chunk * 8 + (col & 7)) * 2);
    }
  }

  __device__ __forceinline__ static bf16x8_t read_b_tr(const char* lb, uint32_t lane_off, int ks) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const char* p = lb + lane_off + ks * (Cfg::MF == 32 ? 16 : 32) * Cfg::BN * 2;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p + 4 * Cfg::BN * 2));
    const v8i16 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, w);
  }

  // MFMA fragments of one 16-wide k step ks of a BK step: A from a swizzled
  // stage, B from a row-major stage through transpose reads.
  struct Frags {
    bf16x8_t a[Cfg::FM], b[Cfg::FN];
  };
  __device__ __forceinline__ static void read_frags(Frags& f, const char* la, const char* lb,
                                                    const uint32_t (&tr_off)[Cfg::FN], int ks, int lane,
                                                    int wm0) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      if constexpr (Cfg::MF == 32)
        f.a[i] = *(const bf16x8_t*)(la + lds_swz(wm0 + i * 32 + (lane & 31), 2 * ks + (lane >> 5)));
      else  // lane l: row (l mod 16), k chunk 4 ks + l / 16 of the BK step
        f.a[i] = *(const bf16x8_t*)(la + lds_swz(wm0 + i * 16 + (lane & 15), 4 * ks + (lane >> 4)));
    }
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) f.b[j] = read_b_tr(lb, tr_off[j], ks);
  }
  __device__ __forceinline__ static void mma(const Frags& f, Acc& acc) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        if constexpr (Cfg::MF == 32)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      }
  }

  // Main path (K % 128 == 0): both operands go from global memory straight
  // to LDS (16-byte global_load_lds, no registers).  A uses three stages in
  // the swizzled layout; B two stages, row-major, read with transpose reads.
  // Step kt: the loads of B for step kt + 1 and of A for step kt + 2 are
  // issued first (into the stages step kt - 1 vacated), then step kt is
  // computed; before its last k step, the wait leaves only the A loads just
  // issued in flight, so everything step kt + 1 reads has landed before the
  // barrier.
  // LDS layout: [A0 A1 A2 B0 B1], Cfg::LDS_DIRECT bytes.
  template <class ARows, class Hook = NoHook>
  __device__ __forceinline__ static void run_direct(const ARows& ar,
                                                    const uint16_t* __restrict__ B, int64_t ldb,
                                                    int col0, int N, int K, char* lds, Acc& acc,
                                                    Hook&& hook = Hook(), int rows_active = Cfg::BM) {
    static_assert(Cfg::B_STAGE % 1024 == 0, "a B stage must be whole 1 KB load blocks");
    constexpr int B_BLK = Cfg::B_STAGE / 1024;
    constexpr int B_BPW = (B_BLK + Cfg::NW - 1) / Cfg::NW;
    // The lane's offsets are derived from a thread index the compiler cannot
    // see through, so they are computed per call: in a persistent kernel they
    // would otherwise be hoisted out of the tile loop and stay live across
    // every other kind of tile the kernel runs.
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    char* const lds_a = lds;
    char* const lds_b = lds + 3 * Cfg::A_STAGE;
    zero(acc);

    // Byte offsets of the A rows this lane moves: block b = wave + t*NW covers
    // tile rows 8b .. 8b + 7; lane l fills LDS slot l of the block, i.e. row
    // r = 8b + l/8 at position l mod 8, which holds logical chunk
    // (l mod 8) ^ ((r / 2) mod 8) (lds_pos is its own inverse in the chunk).
    uint32_t a_off[Cfg::A_BPW];
#pragma unroll
    for (int t = 0; t < Cfg::A_BPW; ++t) {
      const int b = wave + t * Cfg::NW;
      const int r = b * 8 + (lane >> 3);
      int64_t off = (b < Cfg::A_BLK) ? ar.row(r) : (int64_t)0;
      if (off < 0) off = ar.stand_in();  // outside the operand: result never stored
      a_off[t] = (uint32_t)((off + lds_pos(r, lane & 7) * 8) * 2);
    }
    // B: 16-byte chunk c = 64 blk + lane of a stage is row c / (BN/8) at
    // position c mod (BN/8), which holds column chunk position ^ b_swz(row);
    // columns at or beyond N read the operand's last 8 columns instead (their
    // results are never stored).
    uint32_t b_off[B_BPW];
#pragma unroll
    for (int t = 0; t < B_BPW; ++t) {
      const int c = (wave + t * Cfg::NW) * 64 + lane;
      const int row = c / (Cfg::BN / 8);
      int col = col0 + ((c % (Cfg::BN / 8)) ^ b_swz(row)) * 8;
      if (col >= N) col = N - 8;
      b_off[t] = (uint32_t)(((int64_t)row * ldb + col) * 2);
    }
    auto issue_a = [&](int stage, int k0) {
      char* la = lds_a + stage * Cfg::A_STAGE;
      const char* base = (const char*)ar.base + (int64_t)k0 * 2;  // uniform
#pragma unroll
      for (int t = 0; t < Cfg::A_BPW; ++t) {
        const int b = wave + t * Cfg::NW;
        if (b < Cfg::A_BLK)
          __builtin_amdgcn_global_load_lds((const void*)(base + a_off[t]),
                                           (__attribute__((address_space(3))) void*)(la + b * 1024),
                                           16, 0, 0);
      }
    };
    auto issue_b = [&](int stage, int k0) {
      char* lb = lds_b + stage * Cfg::B_STAGE;
      const char* base = (const char*)B + (int64_t)k0 * ldb * 2;  // uniform
#pragma unroll
      for (int t = 0; t < B_BPW; ++t) {
        const int blk = wave + t * Cfg::NW;
        if (blk < B_BLK)
          __builtin_amdgcn_global_load_lds((const void*)(base + b_off[t]),
                                           (__attribute__((address_space(3))) void*)(lb + blk * 1024),
                                           16, 0, 0);
      }
    };
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;
    uint32_t tr_off[Cfg::FN];
    tr_lane_offsets(wn0, lane, tr_off);

    const int nk = K / Cfg::BK;
    issue_b(0, 0);  // B never waits for a signal: its first stage loads during the A wait
    hook.before_a(0);
    issue_a(0, 0);
    if (nk > 1) {
      hook.before_a(Cfg::BK);
      issue_a(1, Cfg::BK);
      wait_vmcnt<Cfg::A_BPW>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    // Fragments are double-buffered across the four k steps of a BK step and
    // across BK steps: the wait and barrier that make the next stage readable
    // come after the last fragment read of the current stage, and the first
    // fragments of the next stage are read while the current stage's last
    // MFMAs run, so neither the barrier nor the LDS latency of a stage's first
    // reads leaves the matrix units idle.
    // A wave whose rows all lie at or past rows_active (padding rows of the
    // tile, wave-uniform) keeps its loads, waits and barriers but skips its
    // fragment reads and MFMAs; its accumulators stay zero.  With two waves
    // per SIMD from different row halves (4 x 2 waves), a tile with at most
    // half its rows in use then takes about half the matrix time.
    const bool on = rows_active >= Cfg::BM || wm0 < rows_active;  // folds to true for the default
    auto rd = [&](Frags& f, const char* la, const char* lb, int ks) {
      if (on) read_frags(f, la, lb, tr_off, ks, lane, wm0);
    };
    auto mm = [&](const Frags& f) {
      if (on) mma(f, acc);
    };
    Frags f0, f1;
    rd(f0, lds_a, lds_b, 0);
    int sa = 0;  // kt % 3
    for (int kt = 0; kt < nk; ++kt) {
      const int sa2 = sa >= 1 ? sa - 1 : 2;   // (kt + 2) % 3
      if (kt + 1 < nk) issue_b((kt + 1) & 1, (kt + 1) * Cfg::BK);
      if (kt + 2 < nk) {
        hook.before_a((kt + 2) * Cfg::BK);
        issue_a(sa2, (kt + 2) * Cfg::BK);
      }
      const char* la = lds_a + sa * Cfg::A_STAGE;
      const char* lb = lds_b + (kt & 1) * Cfg::B_STAGE;
      if constexpr (Cfg::KS == 4) {
        rd(f1, la, lb, 1);
        mm(f0);
        rd(f0, la, lb, 2);
        mm(f1);
        rd(f1, la, lb, 3);
        mm(f0);
      } else {
        rd(f1, la, lb, 1);
        mm(f0);
      }
      sa = sa == 2 ? 0 : sa + 1;
      if (kt + 1 < nk) {
        if (kt + 2 < nk) wait_vmcnt<Cfg::A_BPW>(); else wait_vmcnt<0>();
        lds_barrier();
        rd(f0, lds_a + sa * Cfg::A_STAGE, lds_b + ((kt + 1) & 1) * Cfg::B_STAGE, 0);
      }
      mm(f1);
    }
    lds_barrier();  // every wave is done with the stages before the LDS is reused
  }

  // Fallback path (any K multiple of 8): A and B staged through registers,
  // one step of prefetch, two LDS stages.  LDS layout: [A0 B0 A1 B1].
  template <class ARows, class Hook = NoHook>
  __device__ __forceinline__ static void run_regs(const ARows& ar, const uint16_t* __restrict__ B,
                                                  int64_t ldb, int col0, int N, int K, char* lds,
                                                  Acc& acc, Hook&& hook = Hook()) {
    zero(acc);
    if constexpr (Cfg::MF != 32) {
      return;  // 16-column fragments have the main path only (the host requires K % 128 == 0)
    } else {
    const int tid = threadIdx.x;
    constexpr int STAGE = Cfg::A_STAGE + Cfg::B_STAGE;
    u32x4_t ra[Cfg::A_PT];
    BRegs rb;
    BAddr ba;
    b_addr(ba, ldb, col0, N);
    const int a_c = tid & 7;
    auto load = [&](int k0) {
      const int kc = k0 + a_c * 8;
#pragma unroll
      for (int i = 0; i < Cfg::A_PT; ++i) {
        const int q = tid + i * Cfg::NT;
        const int64_t off = (q < Cfg::A_CH) ? ar.row(q >> 3) : (int64_t)-1;
        if (off >= 0 && kc < K)
          ra[i] = *(const u32x4_t*)(ar.base + off + kc);
        else
          ra[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
      load_b<true>(rb, ba, B, ldb, K, k0);
    };
    auto store = [&](int stage) {
      char* la = lds + stage * STAGE;
#pragma unroll
      for (int i = 0; i < Cfg::A_PT; ++i) {
        const int q = tid + i * Cfg::NT;
        if (q < Cfg::A_CH) *(u32x4_t*)(la + lds_swz(q >> 3, q & 7)) = ra[i];
      }
      store_b(rb, la + Cfg::A_STAGE);
    };
    const int nk = (K + Cfg::BK - 1) / Cfg::BK;
    hook.before_a(0);
    load(0);
    store(0);
    lds_barrier();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) {
        hook.before_a((kt + 1) * Cfg::BK);
        load((kt + 1) * Cfg::BK);
      }
      compute(lds + cur * STAGE, lds + cur * STAGE + Cfg::A_STAGE, acc);
      if (kt + 1 < nk) store(cur ^ 1);
      lds_barrier();
    }
    }
  }

  // Visit every accumulator element: f(row_in_tile, col_in_tile, value).
  template <class F>
  __device__ __forceinline__ static void for_each(const Acc& acc, F&& f) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
        for (int v = 0; v < ACC_N; ++v) {
          // 32x32 result: lane l has column l mod 32, register v row
          // 8 (v / 4) + 4 (l / 32) + v mod 4; 16x16: column l mod 16, row
          // 4 (l / 16) + v
          const int r = Cfg::MF == 32 ? wm0 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)
                                      : wm0 + i * 16 + (lane >> 4) * 4 + v;
          const int c = Cfg::MF == 32 ? wn0 + j * 32 + (lane & 31) : wn0 + j * 16 + (lane & 15);
          f(r, c, acc[i][j][v]);
        }
  }

  // fp32 epilogue: element (r, c) of the tile goes to C[r * ldc + c] for
  // r < rows and c < cols, one 4-byte store each (COHERENT: stores that
  // write through to memory, for data a concurrent kernel reads).  A
  // store's address is the tile's wave-uniform base plus a 32-bit per-lane
  // offset, built fragment by fragment from an offset the compiler cannot
  // see through (the empty asm), so that it computes at most one fragment's
  // offsets ahead: all of a lane's 64-bit addresses computed in advance made
  // persistent kernels spill.
  template <bool COHERENT = true>
  __device__ __forceinline__ static void store_f32(const Acc& acc, float* C, int64_t ldc, int rows, int cols) {
    const int tid = opaque_tid();
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM, wn0 = (wave % Cfg::WN) * Cfg::WTN;
    // 32x32 result: lane l has column l mod 32 and rows 4 (l / 32) + 8 (v /
    // 4) + v mod 4; 16x16: column l mod 16, rows 4 (l / 16) + v
    const int r_l = Cfg::MF == 32 ? (lane >> 5) * 4 : (lane >> 4) * 4;
    const int c_l = Cfg::MF == 32 ? (lane & 31) : (lane & 15);
    const char* base = (const char*)C;
    const uint32_t row_b = (uint32_t)ldc * 4u;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const int r0 = wm0 + i * Cfg::MF + r_l, c = wn0 + j * Cfg::MF + c_l;
        uint32_t off = (uint32_t)r0 * row_b + (uint32_t)c * 4u;
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int v = 0; v < ACC_N; ++v) {
          const int dr = Cfg::MF == 32 ? (v >> 2) * 8 + (v & 3) : v;
          if (r0 + dr < rows && c < cols) {
            float* p = (float*)(base + off + (uint32_t)dr * row_b);
            if (COHERENT)
              store_coherent(p, acc[i][j][v]);
            else
              *p = acc[i][j][v];
          }
        }
        // one fragment at a time (plain stores could otherwise be batched
        // with every address live at once)
        if (!COHERENT) __builtin_amdgcn_sched_barrier(0);
      }
  }

  // bf16 epilogue through LDS.  C points at the tile's first element, with
  // ldc elements per row; ldc and the address are multiples of 8 elements,
  // and only the first `rows` rows and `cols` columns of the tile are stored
  // (cols a multiple of 8).  Each wave rounds f(value) of its results to
  // bf16 (nearest even) into its own region of LDS, row-major, then reads
  // the region back in 16-byte row pieces and stores those: a wave writes
  // whole 16-byte vectors instead of one 2-byte element per lane and value.
  // Rows are padded by 32 bytes when the LDS allows it, so that the two row
  // groups of a fragment (rows r and r + 4) write different banks.  Called by
  // every thread after the K loop, whose last barrier freed the LDS;
  // LDS_BYTES is the size of the caller's LDS array.  COHERENT: the stores go
  // through to the coherence point (store_coherent), for data a consumer in
  // the same kernel reads after a signal.
  // Row stride of a wave's staging region: padded by 32 bytes when the LDS
  // allows, so that the two row groups of a fragment write different banks.
  template <int LDS_BYTES>
  static constexpr int stage_stride() {
    return Cfg::WTN * 2 + (Cfg::NW * Cfg::WTM * (Cfg::WTN * 2 + 32) <= LDS_BYTES ? 32 : 0);
  }

  // Rounds f(value) of this wave's results to bf16 into its own LDS region
  // (row-major, stage_stride bytes per row) and returns the region, after
  // the wave's writes have completed.
  template <int LDS_BYTES, class F>
  __device__ __forceinline__ static char* stage_bf16(const Acc& acc, char* lds, F&& f) {
    constexpr int STRIDE = stage_stride<LDS_BYTES>();
    static_assert(Cfg::NW * Cfg::WTM * STRIDE <= LDS_BYTES, "staged tile does not fit the LDS");
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    char* reg = lds + wave * (Cfg::WTM * STRIDE);
    char* wr = Cfg::MF == 32 ? reg + ((lane >> 5) * 4) * STRIDE + (lane & 31) * 2
                             : reg + ((lane >> 4) * 4) * STRIDE + (lane & 15) * 2;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
      {
#pragma unroll
        for (int v = 0; v < ACC_N; ++v) {
          const int r = Cfg::MF == 32 ? i * 32 + (v >> 2) * 8 + (v & 3) : i * 16 + v;
          *(uint16_t*)(wr + r * STRIDE + j * 2 * Cfg::MF) = (uint16_t)f32_to_bf16(f(acc[i][j][v]));
        }
        // one fragment at a time: keeps the compiler from moving every
        // accumulator into vector registers at once
        __builtin_amdgcn_sched_barrier(0);
      }
    // The region is this wave's alone: its LDS writes complete before its
    // reads, and the clobber keeps the compiler from reordering them.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    return reg;
  }

  // bf16 epilogue with scattered rows: tile row r is stored to row
  // dst_row[r] of C (ldc elements per row; the row is skipped when
  // dst_row[r] < 0), its first `cols` columns (a multiple of 8) as 16-byte
  // pieces.  Called by every thread after the K loop, whose last barrier
  // freed the LDS.
  template <int LDS_BYTES, class F>
  __device__ __forceinline__ static void store_bf16_rows(const Acc& acc, char* lds, uint16_t* C, int64_t ldc,
                                                        const int* __restrict__ dst_row, int cols, F&& f) {
    constexpr int STRIDE = stage_stride<LDS_BYTES>();
    constexpr int VPR = Cfg::WTN / 8;
    constexpr int TOT = Cfg::WTM * VPR;
    static_assert(TOT % 64 == 0, "pieces must fill whole wave passes");
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;
    const char* reg = stage_bf16<LDS_BYTES>(acc, lds, f);
#pragma unroll 4
    for (int it = 0; it < TOT / 64; ++it) {
      const int idx = it * 64 + lane;
      const int r = idx / VPR, q = idx - r * VPR;
      const u32x4_t v = *(const u32x4_t*)(reg + r * STRIDE + q * 16);
      const int dr = dst_row[wm0 + r];
      if (dr >= 0 && wn0 + q * 8 < cols) *(u32x4_t*)(C + (int64_t)dr * ldc + wn0 + q * 8) = v;
    }
  }

  template <int LDS_BYTES, bool COHERENT, class F>
  __device__ __forceinline__ static void store_bf16_staged(const Acc& acc, char* lds, uint16_t* C,
                                                          int64_t ldc, int rows, int cols, F&& f) {
    constexpr int STRIDE = stage_stride<LDS_BYTES>();
    constexpr int VPR = Cfg::WTN / 8;          // 16-byte pieces per row
    constexpr int TOT = Cfg::WTM * VPR;
    static_assert(TOT % 64 == 0, "pieces must fill whole wave passes");
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wn0 = (wave % Cfg::WN) * Cfg::WTN;
    const char* reg = stage_bf16<LDS_BYTES>(acc, lds, f);
    uint16_t* dst0 = C + (int64_t)wm0 * ldc + wn0;
    if (COHERENT) {
      // 8-byte pieces: each store instruction of the wave then writes
      // consecutive bytes of a row, whole lines at a time (16-byte coherent
      // stores go out as two 8-byte halves, each instruction writing every
      // other 8 bytes)
      constexpr int WPR = Cfg::WTN / 4;
      constexpr int TOT8 = Cfg::WTM * WPR;
      static_assert(TOT8 % 64 == 0, "pieces must fill whole wave passes");
#pragma unroll 4
      for (int it = 0; it < TOT8 / 64; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx / WPR, q = idx - r * WPR;
        const uint64_t v = *(const uint64_t*)(reg + r * STRIDE + q * 8);
        if (wm0 + r < rows && wn0 + q * 4 < cols) store_coherent((uint64_t*)(dst0 + (int64_t)r * ldc + q * 4), v);
      }
    } else {
#pragma unroll 4
      for (int it = 0; it < TOT / 64; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx / VPR, q = idx - r * VPR;
        const u32x4_t v = *(const u32x4_t*)(reg + r * STRIDE + q * 16);
        if (wm0 + r < rows && wn0 + q * 8 < cols) *(u32x4_t*)(dst0 + (int64_t)r * ldc + q * 8) = v;
      }
    }
  }
};

}  // namespace tsg
