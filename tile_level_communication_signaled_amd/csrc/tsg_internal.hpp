// Host-side internals shared by the op translation units: the context, error
// reporting, CU-partitioned side streams and the fork/join launch helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <map>
#include <string>
#include <vector>

#include "tsg.h"
#include "tsg_device.hpp"

struct tsg_ctx {
  int device = 0;
  int n_cus = 0;
  int64_t wall_khz = 100000;
  uint32_t epoch = 0;

  uint64_t* d_sig = nullptr;   // signal words
  uint32_t* d_cnt = nullptr;   // arrival counters, one per signal word (zero between calls)
  size_t n_sig = 0;
  uint32_t* d_status = nullptr;  // sticky device error bits
  uint32_t* d_queue = nullptr;   // work-queue tickets of persistent kernels (zero between calls)

  uint64_t* d_timeline = nullptr;
  uint32_t* d_timeline_n = nullptr;
  uint32_t timeline_cap = 0;

  // side streams keyed by CU mask (empty key: unmasked streams 0 / 1)
  std::map<std::vector<uint32_t>, hipStream_t> masked;
  hipStream_t side[2] = {nullptr, nullptr};
  // Copy-engine streams of the AllGather (one per chunk, then a join
  // stream), their events, and the ring of signal values the engines copy.
  // The runtime runs device copies below 64 KB as blit kernels, so a signal
  // travels as a 64 KB copy: the window of the ring that ends at the call's
  // value (the ring has kDmaRingPad words ahead of its entries), into a
  // 64 KB signal block whose last word is the signal the GEMM polls.
  static constexpr int kDmaStreams = 33;
  static constexpr int kDmaRing = 1 << 16;
  static constexpr size_t kDmaSigBytes = size_t(64) << 10;
  static constexpr int kDmaRingPad = (int)(kDmaSigBytes / 8);
  hipStream_t dma[kDmaStreams] = {};
  hipEvent_t ev_dma[kDmaStreams] = {};
  uint64_t* d_dma_ring = nullptr;  // kDmaRingPad + kDmaRing words; entries from kDmaRingPad on
  void* d_dma_sig = nullptr;       // signal blocks of kDmaSigBytes (zeroed when allocated)
  int dma_sig_blocks = 0;
  void* d_noalloc_ws = nullptr;  // device address of the MoE no-alloc workspace (static)
  uint32_t dma_ring_base = 0;
  bool dma_ring_valid = false;
  hipEvent_t ev_fork = nullptr;
  hipEvent_t ev_join[2] = {nullptr, nullptr};
  hipEvent_t ev_k[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
  bool timing = false;
  bool ran[2] = {false, false};

  bool probed = false;
  int n_xcd = 0;
  std::map<std::pair<const void*, const void*>, bool> co_res;  // co_resident() cache

  std::string err;
};

namespace tsgh {

tsg_status fail(tsg_ctx* ctx, tsg_status st, const char* fmt, ...);
tsg_status hip_fail(tsg_ctx* ctx, hipError_t e, const char* what);

#define TSG_HIP(ctx, expr)                                   \
  do {                                                       \
    hipError_t e_ = (expr);                                  \
    if (e_ != hipSuccess) return tsgh::hip_fail(ctx, e_, #expr); \
  } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Resolved options with defaults applied.
struct Opts {
  int aux_cus;   // -1 = shared (no split)
  int main_cus;
  int tile;
  int order;
  uint32_t timeout_ms;
  uint32_t skip_mask;
  int timeline;
  int aux_wgs;   // 0 = the op's default
  int comm_tile; // 0 = the op's default
  int pull_units; // 0 = the op's default, -1 = none
  int stage_dtype; // MoE y staging: TSG_F32 or TSG_BF16
  int arrival_gbps; // AG arrival pacing, 0 = none
  int copy_engine;  // AG: 1 = DMA copy engines move the data
  int channels;     // AG: signals per rank (0 = 1)
  int ep_ranks;     // MoE: source ranks of the tokens (0 = plain tile order)
  int ep_rank;      // MoE: this rank among them
};
Opts resolve(const tsg_opts* o, int default_aux_cus);

// Producer / consumer streams for one call.  In split mode they are CU-masked
// to disjoint CU sets (consumer CUs spread evenly over the XCDs); in shared
// mode both are unmasked, and when `caller` is given the main kernel runs on
// the caller's stream itself (no fork or join for it).
struct Pair {
  hipStream_t main;
  hipStream_t aux;
  int main_cus;
  int aux_cus;
};
tsg_status streams(tsg_ctx* ctx, const Opts& o, Pair* out, hipStream_t caller = nullptr);

// Copy-engine stream i (0 <= i < tsg_ctx::kDmaStreams) and its event,
// created on first use.
tsg_status dma_stream(tsg_ctx* ctx, int i, hipStream_t* s);
// At least n zeroed signal blocks in ctx->d_dma_sig (reallocated, after a
// device synchronisation, when fewer exist).
tsg_status dma_sig_blocks(tsg_ctx* ctx, int n);

// True when one workgroup of kernel `a` (nt_a threads) and one of kernel `b`
// fit on one CU together: registers of their waves on each SIMD and LDS.
// Kernels whose workgroups cannot share a CU must not be relied on to run
// concurrently.
bool co_resident(tsg_ctx* ctx, const void* a, int nt_a, const void* b, int nt_b);

tsg::SyncArgs sync_args(tsg_ctx* ctx, const Opts& o);
tsg::Timeline timeline(tsg_ctx* ctx, const Opts& o);

// Fork: side streams wait for everything already queued on `caller`.
tsg_status fork(tsg_ctx* ctx, hipStream_t caller, const Pair& p);
// Join: `caller` waits for both side streams.
tsg_status join(tsg_ctx* ctx, hipStream_t caller, const Pair& p);
// Kernel timing brackets (no-ops unless timing is enabled).
void time_begin(tsg_ctx* ctx, int which, hipStream_t s);
void time_end(tsg_ctx* ctx, int which, hipStream_t s);
void time_reset(tsg_ctx* ctx);

tsg_status check_launch(tsg_ctx* ctx, const char* what);

}  // namespace tsgh

// Op entry points implemented in the op translation units.
tsg_status tsg_op_ag(tsg_ctx*, const void*, const void*, void*, const void*, void*, int, int, int,
                     int, int, int, const int*, const tsg_opts*, int, void*);
tsg_status tsg_op_rs(tsg_ctx*, const void*, const void*, float*, const float*, float*, int, int,
                     int, int, int, const tsg_opts*, int, void*);
tsg_status tsg_op_mlp2(tsg_ctx*, const void*, const void*, void*, const void*, float*, int, int,
                       int, int, const tsg_opts*, int, void*);
tsg_status tsg_op_moe_ag(tsg_ctx*, const void*, const void*, void*, const int32_t*, const void*, void*, int32_t*,
                         int32_t*, void*, size_t, int, int, int, int, int, int, int, const int*,
                         const tsg_opts*, int, void*);
size_t tsg_moe_ag_workspace(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k);
tsg_status tsg_op_attn(tsg_ctx*, const void*, const void*, const void*, const void*, const void*, void*, void*,
                       void*, int, int, int, int, int, const int*, const tsg_opts*, int, void*);
tsg_status tsg_op_moe(tsg_ctx*, const void*, const int32_t*, const float*, const void*,
                      const void*, float*, int32_t*, int32_t*, void*, size_t, int, int, int, int,
                      int, const tsg_opts*, int, void*, bool noalloc);
// Looks up (once per device) the device address of the MoE no-alloc
// workspace and stores it in ctx->d_noalloc_ws; ctx->device must be current.
tsg_status tsg_moe_scratch_init(tsg_ctx* ctx);
size_t tsg_moe_workspace(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k);
// Piece plan of the AllGather copy (tsg_copy.hpp): pieces per channel of the
// head slabs and the body (np[5]), first unit of each (ustart[5]) and the
// unit count; false if the copy's offsets or unit count would overflow.
bool copy_plan(int R, int C, int chunk_rows, int K, int n_slab, int vpr_log2, int nwg, int* np, int* ustart,
               int64_t* n_units);
bool tsg_moe_layout_fields(const int64_t* dims, int64_t* out, int n);
tsg_status tsg_probe_xcd(tsg_ctx* ctx);
