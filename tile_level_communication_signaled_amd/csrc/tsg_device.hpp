// Device-side helpers shared by the tile-signaled kernels: vector types,
// bf16 rounding, and the signal protocol that links producer and consumer
// tiles.
//
// Signal protocol ([TL] = "TileLink: Generating Efficient Compute-Communication
// Overlapping Kernels using Tile-Centric Primitives", Table 3 and section 3.2.1:
// notify carries release semantics, wait carries acquire semantics; a consumer
// tile is ready once every producer tile it depends on is done).
//
// A signal is one 64-bit word {epoch:32 | n:32}.  Each call of the host API
// draws a fresh epoch e.  A signal with one producer is published by storing
// {e | 1} with release ordering.  A signal shared by n producers has a 32-bit
// arrival counter beside it: every producer adds one (acquire-release), and
// the one that completes the count resets the counter and stores {e | n}.  A
// consumer spins until the word is >= {e | n}, then acquires.  Because epochs
// only grow, signal words need no reset pass between calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Scope of every signal operation.  One GPU only needs agent scope for
// coherence across its XCDs; system scope is kept so that the same protocol
// stays valid when the signal words are written by peer GPUs over xGMI.
#define TSG_SIG_SCOPE __HIP_MEMORY_SCOPE_SYSTEM

enum : uint32_t { ERR_TIMEOUT = 1u, ERR_BAD_EXPERT = 2u };

// Per-launch synchronisation context.
struct SyncArgs {
  uint32_t epoch;        // epoch of this call
  uint32_t pad;
  uint32_t* status;      // error word (ERR_* bits), sticky until read by the host
  uint64_t spin_ticks;   // bound of one wait, in wall-clock ticks
};

__device__ __forceinline__ uint64_t sig_target(uint32_t epoch, uint32_t n) {
  return ((uint64_t)epoch << 32) | (uint64_t)n;
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Single producer: publish {epoch | n} with release ordering (one lane).
__device__ __forceinline__ void sig_publish_lane(uint64_t* s, uint32_t epoch, uint32_t n) {
  __hip_atomic_store(s, sig_target(epoch, n), __ATOMIC_RELEASE, TSG_SIG_SCOPE);
}

// n producers share one signal: each arrives once on the 32-bit arrival
// counter `cnt` with a release fetch-add; the last one to arrive acquires
// (a fence after reading the count of n - 1, which synchronises with every
// earlier arriver's release), resets the counter for the next call and
// publishes {epoch | n} with release ordering.  Only the last arriver pays
// for the acquire, which invalidates its XCD's caches.  One lane.
__device__ __forceinline__ void sig_arrive_counted_lane(uint32_t* cnt, uint64_t* s, uint32_t n,
                                                        uint32_t epoch) {
  const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, TSG_SIG_SCOPE);
  if (old == n - 1) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
    __hip_atomic_store(s, sig_target(epoch, n), __ATOMIC_RELEASE, TSG_SIG_SCOPE);
  }
}

// Coherent-store publication.  A store issued at signal scope writes through
// the XCD's L2 to the device's coherence point, and the wave's store counter
// drops only once the write is acknowledged there.  A producer whose data
// stores are all of this kind needs no L2 write-back before its signal: once
// every wave has waited for its stores, the data is visible to every XCD, and
// the signal (also a signal-scope store) is ordered after it.  This avoids the
// release's write-back of the whole L2, which serialises on the XCD and stalls
// its other traffic, at the price of 8-byte store instructions.
__device__ __forceinline__ void store_coherent(u32x4_t* p, u32x4_t v) {
  uint64_t* q = (uint64_t*)p;
  __hip_atomic_store(q, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  __hip_atomic_store(q + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED, TSG_SIG_SCOPE);
}

__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, TSG_SIG_SCOPE);
}

__device__ __forceinline__ void store_coherent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
}

// Coherent load of 16 bytes (two 64-bit relaxed atomic loads at signal
// scope): it bypasses the caches that may hold an older copy of the line, so
// a consumer that reads data once after a signal needs no cache invalidation.
__device__ __forceinline__ float4 load_coherent(const float4* p) {
  const uint64_t* q = (const uint64_t*)p;
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                     __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}

// Whole workgroup, after its coherent stores: every wave waits until they are
// acknowledged, then the barrier orders all waves before the lane that
// arrives.
__device__ __forceinline__ void block_coherent_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Counted arrival after block_coherent_complete(): no fence is needed, as the
// data each arriver made visible is complete before its fetch-add, and the
// last arriver's signal store follows its fetch-add.  One lane.
__device__ __forceinline__ void sig_arrive_counted_coherent(uint32_t* cnt, uint64_t* s, uint32_t n,
                                                            uint32_t epoch) {
  const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  if (old == n - 1) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
    // the reset is acknowledged before the signal: whoever has seen the
    // signal (and a launch ordered after it) finds the counter at zero
    __builtin_amdgcn_s_waitcnt(0);
    __hip_atomic_store(s, sig_target(epoch, n), __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  }
}

// Single producer after block_coherent_complete(): publish {epoch | n}.
__device__ __forceinline__ void sig_publish_coherent(uint64_t* s, uint32_t epoch, uint32_t n) {
  __hip_atomic_store(s, sig_target(epoch, n), __ATOMIC_RELAXED, TSG_SIG_SCOPE);
}

// Whole workgroup, before one lane publishes or arrives: every wave waits
// until its global stores have been acknowledged by its XCD's L2, then the
// barrier orders all waves before the publishing lane, whose release at
// system scope writes that L2 back.  One write-back per workgroup instead of
// one per wave.
__device__ __forceinline__ void block_release_fence() {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
}

// Wave-level poll: every lane of the calling wave executes this with the same
// arguments.  Lane 0 polls the signal (system-scope atomic load) and the value
// is broadcast to the wave with readfirstlane, so the loop stays uniform.
// Bounded: after sa.spin_ticks the error word gets ERR_TIMEOUT and the poll
// returns; once that bit is set, later polls return immediately, so a missing
// producer turns into an error instead of a hang.  No acquire: the caller
// follows it with the fence its data needs (wave_wait_ge below).
__device__ __forceinline__ void wave_poll_ge(const uint64_t* s, uint64_t target,
                                             const SyncArgs& sa) {
  const int lane = __lane_id();
  uint64_t v = 0;
  if (lane == 0) v = __hip_atomic_load(s, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  v = ((uint64_t)hi << 32) | lo;
  if (v < target) {
    uint32_t st = 0;
    if (lane == 0) st = __hip_atomic_load(sa.status, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
    st = __builtin_amdgcn_readfirstlane(st);
    if (st & ERR_TIMEOUT) return;
    const uint64_t t0 = wall_clock64();
    for (;;) {
      __builtin_amdgcn_s_sleep(1);
      if (lane == 0) v = __hip_atomic_load(s, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
      lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      v = ((uint64_t)hi << 32) | lo;
      if (v >= target) break;
      if ((uint64_t)(wall_clock64() - t0) > sa.spin_ticks) {
        if (lane == 0) __hip_atomic_fetch_or(sa.status, ERR_TIMEOUT, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
        return;
      }
    }
  }
}

// Wave-level wait: poll, then acquire at agent scope.
__device__ __forceinline__ void wave_wait_ge(const uint64_t* s, uint64_t target,
                                             const SyncArgs& sa) {
  wave_poll_ge(s, target, sa);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Workgroup-level wait: wave 0 polls, the barrier releases the other waves,
// and every wave performs its own acquire fence (invalidating the caches it
// reads through) before touching the guarded data.
__device__ __forceinline__ void block_wait_ge(const uint64_t* s, uint64_t target,
                                              const SyncArgs& sa) {
  if (threadIdx.x < 64) wave_wait_ge(s, target, sa);
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Workgroup-level wait without an acquire: for consumers that read the
// guarded data only with coherent loads (load_coherent), issued after the
// barrier and therefore after the signal was seen.
__device__ __forceinline__ void block_poll_ge(const uint64_t* s, uint64_t target,
                                              const SyncArgs& sa) {
  if (threadIdx.x < 64) wave_poll_ge(s, target, sa);
  __syncthreads();
}

// Acquire for a consumer that reads guarded data with ordinary loads, per
// wave, after the signal was seen.  Every kernel starts with caches that hold
// no stale device data (the dispatch's acquire invalidates them), so an
// XCD's L2 can hold an old copy of a guarded line only if something on that
// XCD read the line earlier in the same kernel.  When the guarded regions
// are whole 128-byte lines that nothing reads before their signal
// (`line_exclusive`), only this CU's L1 can be stale and invalidating it is
// enough; the L2, and with it the operands of every other workgroup on the
// XCD, is kept.  Otherwise the acquire invalidates both.
__device__ __forceinline__ void acquire_lines(bool line_exclusive) {
  if (line_exclusive)
    asm volatile("buffer_inv sc0" ::: "memory");
  else
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Workgroup-level wait followed by acquire_lines in every wave.
__device__ __forceinline__ void block_wait_lines(const uint64_t* s, uint64_t target,
                                                 const SyncArgs& sa, bool line_exclusive) {
  block_poll_ge(s, target, sa);
  acquire_lines(line_exclusive);
}

// Per-XCD phased work queues of a persistent kernel.  Phase p has n[p]
// items, cut into 8 contiguous shares (share x = [n x / 8, n (x + 1) / 8)),
// one ticket counter per (phase, XCD) at q[8 p + x].  The items an XCD runs
// then form a compact block whose operands its L2 can reuse.  Called by all
// lanes of one wave with uniform arguments; returns the phase and the index
// in the phase (uniform), or phase -1 once every phase is used up.  Within a
// phase the wave tries its own XCD's share first; if that is used up, one
// load per counter shows which shares still have tickets, and only those are
// tried.  A failed claim proves its share used up, so a wave leaves phase p
// only once every item of phase p has been taken.
struct QueueItem {
  int phase, index;
};
// `from` is the phase of the caller's previous item (0 at first): the
// phases before it are used up, so they are not probed again.
template <int NP>
__device__ __forceinline__ QueueItem xcd_queue_claim(uint32_t* q, const int (&n)[NP], int my_xcd, int from = 0) {
  const int lane = __lane_id();
  for (int ph = from; ph < NP; ++ph) {
    const int np = n[ph];
    int got = -1;
    auto claim = [&](int x) {
      const int lo = (int)((int64_t)np * x / 8), hi = (int)((int64_t)np * (x + 1) / 8);
      if (hi == lo) return;
      uint32_t t = 0;
      if (lane == 0) t = atomicAdd(q + ph * 8 + x, 1u);
      t = __builtin_amdgcn_readfirstlane(t);
      if (t < (uint32_t)(hi - lo)) got = lo + (int)t;
    };
    claim(my_xcd);
    if (got < 0) {
      bool open = false;
      if (lane < 8 && lane != my_xcd) {
        const int lo = (int)((int64_t)np * lane / 8), hi = (int)((int64_t)np * (lane + 1) / 8);
        const uint32_t c = __hip_atomic_load(q + ph * 8 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        open = c < (uint32_t)(hi - lo);
      }
      uint64_t cand = __builtin_amdgcn_ballot_w64(open);
      while (cand != 0 && got < 0) {
        const int x = (int)__builtin_ctzll(cand);
        cand &= cand - 1;
        claim(x);
      }
    }
    if (got >= 0) return QueueItem{ph, got};
  }
  return QueueItem{-1, 0};
}

// The XCD the calling wave runs on (XCC_ID hardware register).
__device__ __forceinline__ int xcd_id() { return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7); }

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Map launch index w to a logical tile index so that every XCD runs a
// contiguous block of `per_xcd` logical tiles out of each wave of
// 8 * per_xcd (neighbouring tiles share operand rows or columns, which then
// stay in one L2).  A final partial wave keeps the identity mapping, so the
// map is a bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int w, int G, int per_xcd) {
  const int wave = 8 * per_xcd;
  const int v = w / wave;
  if (per_xcd <= 0 || (v + 1) * wave > G) return w;
  const int r = w - v * wave;
  return v * wave + (r & 7) * per_xcd + (r >> 3);
}

// Where the calling wave runs: XCD (bits 8..11), shader engine (4..6) and
// CU within it (0..3), from the HW_ID and XCC_ID hardware registers.
__device__ __forceinline__ uint32_t hw_where() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID, all 32 bits
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // XCC_ID, bits 0..3
  return (xcc & 0xFu) << 8 | ((hw >> 13) & 0x7u) << 4 | ((hw >> 8) & 0xFu);
}

// Grouped tile order: logical tile t -> tile (m, n), walking groups of G
// tile rows column by column.  A run of consecutive logical tiles (one XCD's
// share after xcd_remap) then forms a near-square block of the tile grid, so
// the operand rows and columns it reads are reused by more of the XCD's
// tiles in its L2.  A bijection on [0, n_m * n_n) for any G >= 1.
__device__ __forceinline__ void grouped_tile(int t, int n_m, int n_n, int G, int& m, int& n) {
  const int per_group = G * n_n;
  const int g = t / per_group;
  const int first = g * G;
  const int rows = min(G, n_m - first);
  const int r = t - g * per_group;
  m = first + r % rows;
  n = r / rows;
}

// Timeline record: {kind<<56 | where<<32 | id, t_start, t_start + ticks spent
// in signal waits, t_end}.
struct Timeline {
  uint64_t* buf;     // 4 x cap words, or null
  uint32_t* count;   // number of records written
  uint32_t cap;
};

__device__ __forceinline__ void timeline_put(const Timeline& tl, uint32_t kind, uint32_t id,
                                             uint64_t t0, uint64_t t1, uint64_t t2) {
  if (tl.buf == nullptr) return;
  const uint32_t i = atomicAdd(tl.count, 1u);
  if (i < tl.cap) {
    uint64_t* r = tl.buf + 4ull * i;
    r[0] = ((uint64_t)kind << 56) | ((uint64_t)hw_where() << 32) | id;
    r[1] = t0;
    r[2] = t1;
    r[3] = t2;
  }
}

}  // namespace tsg
