// The copy that stands in for peers' arrival in the AllGather paths: a work
// queue of copy units, each a piece of one (channel, column slab) of one
// row chunk, moved with coherent stores and counted on its signal.  Shared
// by the AllGather + GEMM path and the AllGather + MoE gather path.
//
// "Triton-distributed: Programming Overlapping Kernels on Distributed AI
// Systems with the Triton Compiler", section 3.2, Algorithm 2 (pull-mode
// AllGather: one copy and one signal per peer chunk), section 3.7 (arrival
// order, sub-chunks from every peer at each step); "TileLink: Generating
// Efficient Compute-Communication Overlapping Kernels using Tile-Centric
// Primitives", section 3.1 (communication tiles sized independently of
// compute tiles) and section 4.1 (static mapping: rank and channel of a row).
#pragma once

#include "tsg_device.hpp"

namespace tsg {

constexpr int kMaxRanks = 32;

struct ChunkOrder {
  int8_t chunk[kMaxRanks];  // chunk copied at arrival position p (p = 0: local)
};

// ---------------------------------------------------------------- copy
constexpr int kHead = 4;  // leading slabs with their own piece counts

struct CopyArgs {
  const u32x4_t* a_local;  // [chunk_rows x K] bf16, as 16-byte vectors
  const u32x4_t* a_peers;  // [(R - 1) x chunk_rows x K], ascending rank without `rank`
  u32x4_t* a_full;         // [M x K]
  uint64_t* sig;           // signal of (chunk c, slab s) at c * n_slab + s
  uint32_t* cnt;           // arrival counters, same indexing
  SyncArgs sa;
  Timeline tl;
  ChunkOrder ord;
  int64_t k8;              // vectors per row (K / 8)
  int chunk_rows, R, rank;
  int C, ch_rows;          // channels per chunk, rows per channel
  int n_slab;              // slabs per chunk
  int vpr_log2;            // log2(vectors per slab row), <= 8: slab width W = 8 << vpr_log2
  // Pieces per channel of slab s: np[s] for s < kHead, np[kHead] for the
  // rest; the units of slab s < kHead start at ustart[s], those of the rest
  // at ustart[kHead].
  int np[kHead + 1];
  int ustart[kHead + 1];
  int n_units;
  uint32_t skip_mask;
  // Work queue shared by the copy kernel's workgroups and the GEMM
  // workgroups that pull units: a ticket counter and an exit counter; the
  // last of the n_workers claimers to leave resets both for the next call.
  uint32_t* queue;
  uint32_t n_workers;
  int unit_base;           // ticket t of the queue is unit unit_base + t (units below are taken statically)
  // Arrival pacing (pace_ticks > 0): unit u is published no earlier than
  // (u + 1) * pace_ticks wall-clock ticks after the first unit was taken;
  // the taker of ticket 0 stores that time, tagged with the call's epoch,
  // in pace_word.
  uint64_t* pace_word;
  float pace_ticks;
};

constexpr uint64_t kPaceClockMask = (uint64_t(1) << 48) - 1;

// Time the first unit of this call was taken (one lane; bounded wait for the
// taker of unit 0 to publish it).
__device__ __forceinline__ uint64_t pace_base(const CopyArgs& a) {
  const uint64_t tag = (uint64_t)(a.sa.epoch & 0xffffu) << 48;
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const uint64_t v = __hip_atomic_load(a.pace_word, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
    if ((v & ~kPaceClockMask) == tag) return v & kPaceClockMask;
    if (wall_clock64() - t0 > a.sa.spin_ticks) {
      __hip_atomic_fetch_or(a.sa.status, ERR_TIMEOUT, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
      return t0 & kPaceClockMask;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Work unit u -> (slab s, channel ch, arrival position p, piece j), in that
// order of significance: slab-major, then channel 0 of every chunk in
// arrival order, then channel 1, and so on.  One unit copies piece j (np[s]
// pieces of about equal rows) of channel ch of slab s of chunk ord[p], then
// arrives on that (channel, slab) signal.  The first slabs are cut into
// more pieces so that many workgroups share them: every GEMM tile needs
// slab 0 before it can start, slab 1 soon after, and so on, while later
// slabs have time to arrive in larger pieces, which need fewer store drains
// and arrivals.  Called by every thread of a workgroup of NT threads with
// the same u.
template <int NT>
__device__ __forceinline__ void copy_unit(const CopyArgs& a, int u) {
  constexpr int U = 8;  // 8-byte words in flight per thread
  const int vpr = 1 << a.vpr_log2;
  const uint64_t t0 = a.tl.buf ? wall_clock64() : 0;
  int s, rem, npc;
  if (u >= a.ustart[kHead]) {
    npc = a.np[kHead];
    const int v = u - a.ustart[kHead];
    const int per = a.R * a.C * npc;
    s = kHead + v / per;
    rem = v - (s - kHead) * per;
  } else {
    s = 0;
    while (u >= a.ustart[s + 1]) ++s;
    npc = a.np[s];
    rem = u - a.ustart[s];
  }
  const int cp = rem / npc;          // ch * R + p
  const int j = rem - cp * npc;
  const int ch = cp / a.R;
  const int p = cp - ch * a.R;
  const int c = a.ord.chunk[p];
  const int rp = (a.ch_rows + npc - 1) / npc;
  const int r0 = ch * a.ch_rows + j * rp;
  const int nr = min(rp, (ch + 1) * a.ch_rows - r0);
  const int64_t col0 = (int64_t)s * vpr;
  const int width = (int)min((int64_t)vpr, a.k8 - col0);
  const int64_t chunk_vec = (int64_t)a.chunk_rows * a.k8;
  const u32x4_t* __restrict__ src =
      (c == a.rank ? a.a_local : a.a_peers + (int64_t)(c < a.rank ? c : c - 1) * chunk_vec) +
      (int64_t)r0 * a.k8 + col0;
  u32x4_t* __restrict__ dst = a.a_full + ((int64_t)c * a.chunk_rows + r0) * a.k8 + col0;
  // The piece moves in 8-byte words, so that each coherent store instruction
  // of a wave covers 64 consecutive words of a row (512 contiguous bytes, or
  // whole rows of a narrow slab) and writes whole lines: stores of 16 bytes
  // per lane would go out as two 8-byte halves, each instruction writing
  // every other 8 bytes.  A slab row is wpr <= 512 words; thread t moves word
  // t mod tpr (+ NT when the row is wider than the workgroup) of rows
  // t / tpr, t / tpr + rows_p, ...  Addresses are a uniform base plus a
  // 32-bit byte offset (one register per access).
  static_assert(NT == 64 || NT == 128 || NT == 256 || NT == 512, "copy workgroups of 64 to 512 threads");
  constexpr int NT_LOG2 = NT == 64 ? 6 : NT == 128 ? 7 : NT == 256 ? 8 : 9;
  const int wpr = 2 * vpr;
  const int tpr_log2 = min(a.vpr_log2 + 1, NT_LOG2);
  const int tpr = 1 << tpr_log2;
  const int rows_p = NT >> tpr_log2;
  const int rr = threadIdx.x >> tpr_log2;
  const int wwidth = 2 * width;
  const char* sb = (const char*)src;
  char* db = (char*)dst;
  const uint32_t row_bytes = (uint32_t)(a.k8 * 16);
  const uint32_t step = (uint32_t)rows_p * row_bytes;
  const int cw = threadIdx.x & (tpr - 1);
  for (int k = 0; k < wpr; k += NT) {  // a second pass only for rows wider than the workgroup
    if (cw + k < wwidth) {
      const char* sk = sb + k * 8;
      char* dk = db + k * 8;
      uint32_t off = (uint32_t)rr * row_bytes + (uint32_t)cw * 8u;
      int r = rr;
      for (; r + (U - 1) * rows_p < nr; r += U * rows_p, off += U * step) {
        // addresses as base + q * step + off: eight words in flight fit in
        // the kernel's 32 registers (the form base + (off + q * step) kept
        // one offset register per word and did not)
        uint64_t v[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
          v[q] = __builtin_nontemporal_load((const uint64_t*)(sk + (size_t)q * step + off));
        }
#pragma unroll
        for (int q = 0; q < U; ++q) store_coherent((uint64_t*)(dk + (size_t)q * step + off), v[q]);
      }
      for (; r < nr; r += rows_p, off += step)
        store_coherent((uint64_t*)(dk + off), __builtin_nontemporal_load((const uint64_t*)(sk + off)));
    }
  }
  // The piece is published without an L2 write-back: its stores went
  // through to the coherence point (store_coherent).
  block_coherent_complete();
  if (a.pace_ticks > 0.f && threadIdx.x == 0) {
    // paced arrival: not before this unit's due time (the wait is bounded by
    // the paced duration of the whole copy)
    const uint64_t due = (pace_base(a) + (uint64_t)((float)(u + 1) * a.pace_ticks)) & kPaceClockMask;
    while ((int64_t)(((wall_clock64() & kPaceClockMask) - due) << 16) < 0) __builtin_amdgcn_s_sleep(8);
  }
  const int g = c * a.C + ch;         // global channel id
  const size_t si = (size_t)g * a.n_slab + s;
  if (threadIdx.x == 0 && !(g < 32 && ((a.skip_mask >> g) & 1u)))
    sig_arrive_counted_coherent(a.cnt + si, a.sig + si, (uint32_t)npc, a.sa.epoch);
  if (threadIdx.x == 0 && a.tl.buf)
    timeline_put(a.tl, 1, (uint32_t)(c << 24 | s << 12 | ((ch * npc + j) & 0xfff)), t0, t0, wall_clock64());
}

// Paced arrival: the taker of unit 0 records when the copy started (one lane).
__device__ __forceinline__ void pace_start(const CopyArgs& a) {
  if (a.pace_ticks > 0.f)
    __hip_atomic_store(a.pace_word,
                       ((uint64_t)(a.sa.epoch & 0xffffu) << 48) | (wall_clock64() & kPaceClockMask),
                       __ATOMIC_RELAXED, TSG_SIG_SCOPE);
}

// Next unit from the queue, identical in every thread (`slot` is one int of
// LDS owned by the caller).
__device__ __forceinline__ int claim_unit(const CopyArgs& a, volatile int* slot) {
  if (threadIdx.x == 0) {
    const int t = (int)atomicAdd(a.queue, 1u);
    if (t + a.unit_base == 0) pace_start(a);
    *slot = t + a.unit_base;
  }
  __syncthreads();
  const int u = __builtin_amdgcn_readfirstlane(*slot);
  __syncthreads();
  return u;
}

// A claimer is done with the queue; the last one resets it.  One lane.
__device__ __forceinline__ void leave_queue(const CopyArgs& a) {
  if (atomicAdd(a.queue + 1, 1u) == a.n_workers - 1) {
    __hip_atomic_store(a.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.queue + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


}  // namespace tsg
