// MFMA GEMM tile engine for gfx950 (CDNA4).
//
// One workgroup computes a BM x BN tile of C = A * B with A [M x K] and
// B [K x N] both row-major bf16, accumulating in fp32 with
// v_mfma_f32_32x32x16_bf16.  The K loop moves BK = 64 columns of A and rows of
// B per step through a two-stage LDS ring:
//
//   * A is staged as BM rows x 8 chunks of 16 bytes (8 bf16 along k).
//   * B is staged transposed, as BN rows (one per output column n) x 8 chunks
//     of 8 consecutive k, so that both MFMA operands are read as one 16-byte
//     LDS load per lane.  The transpose happens in registers while staging:
//     each thread loads an 8 (k) x 8 (n) block with eight coalesced 16-byte
//     row loads and repacks it with byte permutes.
//   * Chunk c of LDS row r is stored at chunk position c ^ (r & 7), so the
//     16-byte reads of 8 consecutive rows hit 8 distinct bank groups.
//
// Waves are arranged WM x WN; a wave owns a (BM/WM) x (BN/WN) sub-tile made of
// 32x32 MFMA fragments.  Operand layout of the 32x32x16 bf16 MFMA: lane l
// supplies row (l mod 32) of A and column (l mod 32) of B, with the 8 k values
// 8*(l / 32) .. 8*(l / 32) + 7 of the current 16-wide k step.  The fp32 result
// fragment gives lane l column (l mod 32) and, in register v, row
// 8*(v / 4) + 4*(l / 32) + (v mod 4).
//
// Loads of rows beyond M, columns beyond N and k beyond K read zeros (N and K
// must be multiples of 8), so ragged tiles need no special path.  The pages
// ask tile-level single-device kernels to coalesce global accesses, keep LDS
// free of bank conflicts, pipeline loads against compute and use the matrix
// units ([TL] section 4.3).
#pragma once

#include "tsg_device.hpp"

namespace tsg {

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = 64;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_STAGE = BM * BK * 2;
  static constexpr int B_STAGE = BN * BK * 2;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int A_CH = BM * 8;               // 16-byte chunks per A stage
  static constexpr int A_PT = (A_CH + NT - 1) / NT; // chunks per thread
  static constexpr int B_BL = BN;                   // 8x8 blocks per B stage
  static constexpr int B_PT = (B_BL + NT - 1) / NT; // blocks per thread
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BN % 8 == 0, "BN must be a multiple of 8");
  static_assert(LDS <= 160 * 1024, "LDS budget of one CU exceeded");
};

__device__ __forceinline__ uint32_t lds_swz(int row, int chunk) {
  return (uint32_t)(((row << 3) | (chunk ^ (row & 7))) << 4);
}

// lo = a.lo16, hi = b.lo16
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// lo = a.hi16, hi = b.hi16
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Source rows of the A operand of one tile.  row(r) gives the element offset
// of tile row r in `base`, or -1 for a row that reads as zeros.
struct ARowsLinear {
  const uint16_t* base;
  int64_t ld;
  int row0;
  int M;
  __device__ __forceinline__ int64_t row(int r) const {
    const int g = row0 + r;
    return g < M ? (int64_t)g * ld : (int64_t)-1;
  }
};

// Gathered rows: idx[r] is the source row index (or < 0 for a zero row).
struct ARowsGather {
  const uint16_t* base;
  int64_t ld;
  const int* idx;
  __device__ __forceinline__ int64_t row(int r) const {
    const int g = idx[r];
    return g >= 0 ? (int64_t)g * ld : (int64_t)-1;
  }
};

template <class Cfg>
struct GemmTile {
  using Acc = f32x16_t[Cfg::FM][Cfg::FN];

  // A source of this tile, B source, sizes.
  template <class ARows>
  __device__ __forceinline__ static void run(const ARows& ar, const uint16_t* __restrict__ B,
                                             int64_t ldb, int col0, int N, int K, char* lds,
                                             Acc& acc) {
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
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Per-thread A chunks: fixed row and chunk column for the whole K loop.
    int64_t a_off[Cfg::A_PT];
    int a_c[Cfg::A_PT];
#pragma unroll
    for (int i = 0; i < Cfg::A_PT; ++i) {
      const int q = tid + i * Cfg::NT;
      const int r = q >> 3;
      a_c[i] = q & 7;
      a_off[i] = (q < Cfg::A_CH) ? ar.row(r) : (int64_t)-1;
    }
    // Per-thread B blocks: k block kb (8 rows) and n block nb (8 columns).
    int b_kb[Cfg::B_PT], b_n[Cfg::B_PT];
    bool b_ok[Cfg::B_PT];
#pragma unroll
    for (int i = 0; i < Cfg::B_PT; ++i) {
      const int q = tid + i * Cfg::NT;
      b_kb[i] = q / (Cfg::BN / 8);
      b_n[i] = (q % (Cfg::BN / 8)) * 8;
      b_ok[i] = (q < Cfg::B_BL) && (col0 + b_n[i] < N);
    }

    u32x4_t ra[Cfg::A_PT];
    u32x4_t rb[Cfg::B_PT][8];

    auto load = [&](int k0) {
#pragma unroll
      for (int i = 0; i < Cfg::A_PT; ++i) {
        const int kc = k0 + a_c[i] * 8;
        if (a_off[i] >= 0 && kc < K)
          ra[i] = *(const u32x4_t*)(ar.base + a_off[i] + kc);
        else
          ra[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < Cfg::B_PT; ++i) {
        const int kr = k0 + b_kb[i] * 8;
        const uint16_t* p = B + (int64_t)kr * ldb + col0 + b_n[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (b_ok[i] && kr + j < K)
            rb[i][j] = *(const u32x4_t*)(p + (int64_t)j * ldb);
          else
            rb[i][j] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };

    auto store = [&](int stage) {
      char* la = lds + stage * Cfg::STAGE;
      char* lb = la + Cfg::A_STAGE;
#pragma unroll
      for (int i = 0; i < Cfg::A_PT; ++i) {
        const int q = tid + i * Cfg::NT;
        if (q < Cfg::A_CH) *(u32x4_t*)(la + lds_swz(q >> 3, q & 7)) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < Cfg::B_PT; ++i) {
        const int q = tid + i * Cfg::NT;
        if (q < Cfg::B_BL) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            // columns n = 2m (low halves) and 2m + 1 (high halves)
            u32x4_t lo, hi;
            lo[0] = pack_lo16(rb[i][0][m], rb[i][1][m]);
            lo[1] = pack_lo16(rb[i][2][m], rb[i][3][m]);
            lo[2] = pack_lo16(rb[i][4][m], rb[i][5][m]);
            lo[3] = pack_lo16(rb[i][6][m], rb[i][7][m]);
            hi[0] = pack_hi16(rb[i][0][m], rb[i][1][m]);
            hi[1] = pack_hi16(rb[i][2][m], rb[i][3][m]);
            hi[2] = pack_hi16(rb[i][4][m], rb[i][5][m]);
            hi[3] = pack_hi16(rb[i][6][m], rb[i][7][m]);
            *(u32x4_t*)(lb + lds_swz(b_n[i] + 2 * m, b_kb[i])) = lo;
            *(u32x4_t*)(lb + lds_swz(b_n[i] + 2 * m + 1, b_kb[i])) = hi;
          }
        }
      }
    };

    auto compute = [&](int stage) {
      const char* la = lds + stage * Cfg::STAGE;
      const char* lb = la + Cfg::A_STAGE;
      const int l32 = lane & 31;
      const int hi = lane >> 5;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t af[Cfg::FM], bfr[Cfg::FN];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
          af[i] = *(const bf16x8_t*)(la + lds_swz(wm0 + i * 32 + l32, 2 * ks + hi));
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
          bfr[j] = *(const bf16x8_t*)(lb + lds_swz(wn0 + j * 32 + l32, 2 * ks + hi));
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
          for (int j = 0; j < Cfg::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    };

    const int nk = (K + Cfg::BK - 1) / Cfg::BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load((kt + 1) * Cfg::BK);
      compute(cur);
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
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
        for (int v = 0; v < 16; ++v) {
          const int r = wm0 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const int c = wn0 + j * 32 + (lane & 31);
          f(r, c, acc[i][j][v]);
        }
  }
};

}  // namespace tsg
