// Device-side helpers shared by the tile-signaled kernels: vector types,
// bf16 rounding, and the signal protocol that links producer and consumer
// tiles.
//
// Signal protocol ([TL] = "TileLink: Generating Efficient Compute-Communication
// Overlapping Kernels using Tile-Centric Primitives", Table 3 and section 3.2.1:
// notify carries release semantics, wait carries acquire semantics; a consumer
// tile is ready once every producer tile it depends on is done).
//
// A signal is one 64-bit word {epoch:32 | count:32}.  Each call of the host API
// draws a fresh epoch e; a producer "arrives" by moving the word to
// {e | count+1} (or to {e | 1} if the word still carries an older epoch), with
// release ordering.  A consumer waiting for n arrivals spins until the word is
// >= {e | n}, then acquires.  Because epochs only grow, no reset pass is needed
// between calls, and any number of producers may share one signal.
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

// One producer arrives on signal `s` (release).  Must be called by a single
// lane after the data it publishes is complete and visible (see
// block_release_arrive).
__device__ __forceinline__ void sig_arrive_lane(uint64_t* s, uint32_t epoch) {
  uint64_t old = __hip_atomic_load(s, __ATOMIC_RELAXED, TSG_SIG_SCOPE);
  for (;;) {
    const uint64_t nv = ((uint32_t)(old >> 32) == epoch) ? old + 1 : sig_target(epoch, 1);
    if (__hip_atomic_compare_exchange_strong(s, &old, nv, __ATOMIC_RELEASE, __ATOMIC_RELAXED,
                                             TSG_SIG_SCOPE))
      return;
  }
}

// Whole workgroup: make this block's prior global stores visible device-wide
// (each wave waits for its stores and writes back its XCD's L2 through the
// release fence), then one lane arrives on each of `n` signals.
__device__ __forceinline__ void block_release_arrive(uint64_t* sigs, const int* idx, int n,
                                                     uint32_t epoch) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < n; ++i) sig_arrive_lane(sigs + idx[i], epoch);
  }
}

__device__ __forceinline__ void block_release_arrive1(uint64_t* s, uint32_t epoch) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) sig_arrive_lane(s, epoch);
}

// Wave-level wait: every lane of the calling wave executes this with the same
// arguments.  Lane 0 polls the signal (system-scope atomic load) and the value
// is broadcast to the wave with readfirstlane, so the loop stays uniform.
// Bounded: after sa.spin_ticks the error word gets ERR_TIMEOUT and the wait
// returns; once that bit is set, later waits return immediately, so a missing
// producer turns into an error instead of a hang.
__device__ __forceinline__ void wave_wait_ge(const uint64_t* s, uint64_t target,
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

// Timeline record: {kind<<56 | id, t_start, t_ready, t_end}.
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
    r[0] = ((uint64_t)kind << 56) | id;
    r[1] = t0;
    r[2] = t1;
    r[3] = t2;
  }
}

}  // namespace tsg
