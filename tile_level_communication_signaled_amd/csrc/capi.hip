// C-ABI of the tile-signaled GEMM library and the host runtime around it:
// context (signal words, epoch, error word, timeline), CU-partitioned side
// streams, fork/join events and per-kernel timing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "tsg_internal.hpp"

namespace {

constexpr size_t kSignals = size_t(1) << 20;  // 8 MiB of 64-bit signal words
constexpr uint32_t kTimelineCap = 1u << 16;

// Reports the XCD (hardware register XCC_ID) the calling workgroup runs on.
__global__ void probe_xcd_kernel(int* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xF);
}

}  // namespace

namespace tsgh {

tsg_status fail(tsg_ctx* ctx, tsg_status st, const char* fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->err = buf;
  }
  return st;
}

tsg_status hip_fail(tsg_ctx* ctx, hipError_t e, const char* what) {
  return fail(ctx, TSG_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

Opts resolve(const tsg_opts* o, int default_aux_cus) {
  Opts r;
  r.aux_cus = o && o->aux_cus ? o->aux_cus : default_aux_cus;
  r.main_cus = o ? o->main_cus : 0;
  r.tile = o ? o->tile : 0;
  r.order = o ? o->order : 0;
  r.timeout_ms = o && o->timeout_ms ? o->timeout_ms : 2000u;
  r.skip_mask = o ? o->debug_skip_mask : 0u;
  r.timeline = o ? o->timeline : 0;
  r.aux_wgs = o ? o->aux_wgs : 0;
  r.comm_tile = o ? o->comm_tile : 0;
  r.pull_units = o ? o->pull_units : 0;
  r.stage_dtype = o ? o->stage_dtype : TSG_F32;
  r.arrival_gbps = o ? o->arrival_gbps : 0;
  r.copy_engine = o ? o->copy_engine : 0;
  r.channels = o ? o->channels : 0;
  r.ep_ranks = o ? o->ep_ranks : 0;
  r.ep_rank = o ? o->ep_rank : 0;
  return r;
}

tsg_status dma_stream(tsg_ctx* ctx, int i, hipStream_t* s) {
  if (i < 0 || i >= tsg_ctx::kDmaStreams) return fail(ctx, TSG_E_INVALID, "copy-engine stream %d", i);
  if (!ctx->dma[i]) {
    if (!ctx->d_dma_ring) {
      TSG_HIP(ctx, hipMalloc(&ctx->d_dma_ring,
                             (size_t)(tsg_ctx::kDmaRingPad + tsg_ctx::kDmaRing) * sizeof(uint64_t)));
      TSG_HIP(ctx, hipMemset(ctx->d_dma_ring, 0,
                             (size_t)(tsg_ctx::kDmaRingPad + tsg_ctx::kDmaRing) * sizeof(uint64_t)));
      ctx->dma_ring_valid = false;
    }
    tsg_status st = dma_sig_blocks(ctx, 1);
    if (st != TSG_OK) return st;
    TSG_HIP(ctx, hipStreamCreateWithFlags(&ctx->dma[i], hipStreamNonBlocking));
    TSG_HIP(ctx, hipEventCreateWithFlags(&ctx->ev_dma[i], hipEventDisableTiming));
    // The first engine copy on a new stream takes milliseconds (the runtime
    // sets up its engine queue).  Pay it here, with one signal-sized copy of
    // the ring's zero padding into the first signal block (zero there
    // already), rather than inside the first call's signal waits.
    TSG_HIP(ctx, hipMemcpyAsync(ctx->d_dma_sig, ctx->d_dma_ring, tsg_ctx::kDmaSigBytes,
                                hipMemcpyDeviceToDeviceNoCU, ctx->dma[i]));
    TSG_HIP(ctx, hipStreamSynchronize(ctx->dma[i]));
  }
  *s = ctx->dma[i];
  return TSG_OK;
}

tsg_status dma_sig_blocks(tsg_ctx* ctx, int n) {
  if (n <= ctx->dma_sig_blocks) return TSG_OK;
  const int cap = (n + 63) / 64 * 64;
  if (ctx->d_dma_sig) {
    TSG_HIP(ctx, hipDeviceSynchronize());
    TSG_HIP(ctx, hipFree(ctx->d_dma_sig));
    ctx->d_dma_sig = nullptr;
    ctx->dma_sig_blocks = 0;
  }
  TSG_HIP(ctx, hipMalloc(&ctx->d_dma_sig, (size_t)cap * tsg_ctx::kDmaSigBytes));
  TSG_HIP(ctx, hipMemset(ctx->d_dma_sig, 0, (size_t)cap * tsg_ctx::kDmaSigBytes));
  ctx->dma_sig_blocks = cap;
  return TSG_OK;
}

static tsg_status unmasked(tsg_ctx* ctx, int i, hipStream_t* s) {
  if (!ctx->side[i]) TSG_HIP(ctx, hipStreamCreateWithFlags(&ctx->side[i], hipStreamNonBlocking));
  *s = ctx->side[i];
  return TSG_OK;
}

static tsg_status masked(tsg_ctx* ctx, const std::vector<uint32_t>& mask, hipStream_t* s) {
  auto it = ctx->masked.find(mask);
  if (it != ctx->masked.end()) {
    *s = it->second;
    return TSG_OK;
  }
  hipStream_t st = nullptr;
  TSG_HIP(ctx, hipExtStreamCreateWithCUMask(&st, (uint32_t)mask.size(), mask.data()));
  ctx->masked[mask] = st;
  *s = st;
  return TSG_OK;
}

tsg_status streams(tsg_ctx* ctx, const Opts& o, Pair* out, hipStream_t caller) {
  const int n = ctx->n_cus;
  if (o.aux_cus < 0) {
    tsg_status st = TSG_OK;
    if (caller)
      out->main = caller;
    else
      st = unmasked(ctx, 0, &out->main);
    if (st != TSG_OK) return st;
    st = unmasked(ctx, 1, &out->aux);
    out->main_cus = n;
    out->aux_cus = n;
    return st;
  }
  const int q = o.aux_cus;
  const int p = o.main_cus > 0 ? o.main_cus : n - q;
  // CU-mask bit i selects a CU of XCD (i mod 8): a mask must give every XCD
  // at least one CU, and an unbalanced mask starves some XCD's L2.  Both
  // partitions are therefore built from whole groups of 8 consecutive bits,
  // one CU per XCD each.
  if (q < 8 || p < 8 || q % 8 || p % 8 || p + q > n)
    return fail(ctx, TSG_E_INVALID,
                "CU split %d/%d must use multiples of 8 CUs, at least 8 per side, within %d CUs", p, q, n);
  std::vector<uint32_t> mc((n + 31) / 32, 0u), mp((n + 31) / 32, 0u);
  for (int i = 0; i < q; ++i) mc[i / 32] |= 1u << (i % 32);
  for (int i = q; i < q + p; ++i) mp[i / 32] |= 1u << (i % 32);
  tsg_status st = masked(ctx, mp, &out->main);
  if (st != TSG_OK) return st;
  st = masked(ctx, mc, &out->aux);
  out->main_cus = p;
  out->aux_cus = q;
  return st;
}

tsg::SyncArgs sync_args(tsg_ctx* ctx, const Opts& o) {
  tsg::SyncArgs s;
  s.epoch = ctx->epoch;
  s.pad = 0;
  s.status = ctx->d_status;
  s.spin_ticks = (uint64_t)o.timeout_ms * (uint64_t)ctx->wall_khz;
  return s;
}

tsg::Timeline timeline(tsg_ctx* ctx, const Opts& o) {
  tsg::Timeline t;
  t.buf = o.timeline ? ctx->d_timeline : nullptr;
  t.count = ctx->d_timeline_n;
  t.cap = ctx->timeline_cap;
  return t;
}

tsg_status fork(tsg_ctx* ctx, hipStream_t caller, const Pair& p) {
  TSG_HIP(ctx, hipEventRecord(ctx->ev_fork, caller));
  if (p.main != caller) TSG_HIP(ctx, hipStreamWaitEvent(p.main, ctx->ev_fork, 0));
  if (p.aux != p.main && p.aux != caller) TSG_HIP(ctx, hipStreamWaitEvent(p.aux, ctx->ev_fork, 0));
  return TSG_OK;
}

tsg_status join(tsg_ctx* ctx, hipStream_t caller, const Pair& p) {
  if (p.main != caller) {
    TSG_HIP(ctx, hipEventRecord(ctx->ev_join[0], p.main));
    TSG_HIP(ctx, hipStreamWaitEvent(caller, ctx->ev_join[0], 0));
  }
  if (p.aux != p.main && p.aux != caller) {
    TSG_HIP(ctx, hipEventRecord(ctx->ev_join[1], p.aux));
    TSG_HIP(ctx, hipStreamWaitEvent(caller, ctx->ev_join[1], 0));
  }
  return TSG_OK;
}

bool co_resident(tsg_ctx* ctx, const void* a, int nt_a, const void* b, int nt_b) {
  const auto key = std::make_pair(a, b);
  auto it = ctx->co_res.find(key);
  if (it != ctx->co_res.end()) return it->second;
  hipFuncAttributes fa, fb;
  bool ok = hipFuncGetAttributes(&fa, a) == hipSuccess && hipFuncGetAttributes(&fb, b) == hipSuccess;
  if (ok) {
    // Registers: a workgroup's waves are spread over the CU's 4 SIMDs; each
    // SIMD holds 512 registers per lane, allocated in granules of 8.
    auto regs = [](const hipFuncAttributes& f, int nt) {
      const int waves_per_simd = ((nt + 63) / 64 + 3) / 4;
      return ((f.numRegs + 7) / 8) * 8 * waves_per_simd;
    };
    ok = regs(fa, nt_a) + regs(fb, nt_b) <= 512 &&
         fa.sharedSizeBytes + fb.sharedSizeBytes <= (size_t)160 * 1024;
  }
  (void)hipGetLastError();
  ctx->co_res[key] = ok;
  return ok;
}

void time_reset(tsg_ctx* ctx) { ctx->ran[0] = ctx->ran[1] = false; }

void time_begin(tsg_ctx* ctx, int which, hipStream_t s) {
  if (ctx->timing) (void)hipEventRecord(ctx->ev_k[which][0], s);
}

void time_end(tsg_ctx* ctx, int which, hipStream_t s) {
  if (ctx->timing) {
    (void)hipEventRecord(ctx->ev_k[which][1], s);
    ctx->ran[which] = true;
  }
}

tsg_status check_launch(tsg_ctx* ctx, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(ctx, e, what);
  return TSG_OK;
}

}  // namespace tsgh

tsg_status tsg_probe_xcd(tsg_ctx* ctx) {
  // One workgroup per CU slot on the null stream; the highest XCC_ID seen
  // gives the number of XCDs.
  int* d = nullptr;
  TSG_HIP(ctx, hipMalloc(&d, sizeof(int) * 1024));
  hipLaunchKernelGGL(probe_xcd_kernel, dim3(1024), dim3(64), 0, nullptr, d);
  int h[1024];
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost);
  (void)hipFree(d);
  if (e != hipSuccess) return tsgh::hip_fail(ctx, e, "XCD probe");
  int mx = 0;
  for (int i = 0; i < 1024; ++i) mx = std::max(mx, h[i]);
  ctx->n_xcd = mx + 1;
  ctx->probed = true;
  return TSG_OK;
}

extern "C" {

tsg_status tsg_ctx_create(int device, tsg_ctx** out) {
  if (!out) return TSG_E_INVALID;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) return TSG_E_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return TSG_E_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return TSG_E_UNSUPPORTED;
  tsg_ctx* c = new tsg_ctx();
  c->device = device;
  c->n_cus = prop.multiProcessorCount;
  hipError_t e = hipSetDevice(device);
  int khz = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device);
  if (khz > 0) c->wall_khz = khz;
  if (e == hipSuccess) e = hipMalloc(&c->d_sig, kSignals * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMemset(c->d_sig, 0, kSignals * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMalloc(&c->d_cnt, kSignals * sizeof(uint32_t));
  if (e == hipSuccess) e = hipMemset(c->d_cnt, 0, kSignals * sizeof(uint32_t));
  if (e == hipSuccess) e = hipMalloc(&c->d_status, 64);
  if (e == hipSuccess) e = hipMemset(c->d_status, 0, 64);
  if (e == hipSuccess) e = hipMalloc(&c->d_queue, 128 * sizeof(uint32_t));
  if (e == hipSuccess) e = hipMemset(c->d_queue, 0, 128 * sizeof(uint32_t));
  if (e == hipSuccess) e = hipMalloc(&c->d_timeline, (size_t)kTimelineCap * 4 * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMalloc(&c->d_timeline_n, 64);
  if (e == hipSuccess) e = hipMemset(c->d_timeline_n, 0, 64);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join[0], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join[1], hipEventDisableTiming);
  for (int i = 0; i < 2 && e == hipSuccess; ++i)
    for (int j = 0; j < 2 && e == hipSuccess; ++j) e = hipEventCreate(&c->ev_k[i][j]);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  c->n_sig = kSignals;
  c->timeline_cap = kTimelineCap;
  if (e != hipSuccess || tsg_moe_scratch_init(c) != TSG_OK) {
    tsg_ctx_destroy(c);
    return TSG_E_HIP;
  }
  *out = c;
  return TSG_OK;
}

void tsg_ctx_destroy(tsg_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  for (auto& kv : c->masked) (void)hipStreamDestroy(kv.second);
  for (int i = 0; i < 2; ++i)
    if (c->side[i]) (void)hipStreamDestroy(c->side[i]);
  for (int i = 0; i < tsg_ctx::kDmaStreams; ++i) {
    if (c->dma[i]) (void)hipStreamDestroy(c->dma[i]);
    if (c->ev_dma[i]) (void)hipEventDestroy(c->ev_dma[i]);
  }
  if (c->d_dma_ring) (void)hipFree(c->d_dma_ring);
  if (c->d_dma_sig) (void)hipFree(c->d_dma_sig);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  for (int i = 0; i < 2; ++i) {
    if (c->ev_join[i]) (void)hipEventDestroy(c->ev_join[i]);
    for (int j = 0; j < 2; ++j)
      if (c->ev_k[i][j]) (void)hipEventDestroy(c->ev_k[i][j]);
  }
  if (c->d_sig) (void)hipFree(c->d_sig);
  if (c->d_cnt) (void)hipFree(c->d_cnt);
  if (c->d_status) (void)hipFree(c->d_status);
  if (c->d_queue) (void)hipFree(c->d_queue);
  if (c->d_timeline) (void)hipFree(c->d_timeline);
  if (c->d_timeline_n) (void)hipFree(c->d_timeline_n);
  delete c;
}

const char* tsg_last_error(const tsg_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

tsg_status tsg_check(tsg_ctx* ctx, void* stream) {
  if (!ctx) return TSG_E_INVALID;
  TSG_HIP(ctx, hipSetDevice(ctx->device));
  TSG_HIP(ctx, hipStreamSynchronize((hipStream_t)stream));
  for (auto& kv : ctx->masked) TSG_HIP(ctx, hipStreamSynchronize(kv.second));
  for (int i = 0; i < 2; ++i)
    if (ctx->side[i]) TSG_HIP(ctx, hipStreamSynchronize(ctx->side[i]));
  for (int i = 0; i < tsg_ctx::kDmaStreams; ++i)
    if (ctx->dma[i]) TSG_HIP(ctx, hipStreamSynchronize(ctx->dma[i]));
  uint32_t st = 0;
  TSG_HIP(ctx, hipMemcpy(&st, ctx->d_status, sizeof st, hipMemcpyDeviceToHost));
  if (st) {
    // A timed-out call may have left arrival counters part-way: clear them.
    TSG_HIP(ctx, hipDeviceSynchronize());
    TSG_HIP(ctx, hipMemset(ctx->d_cnt, 0, ctx->n_sig * sizeof(uint32_t)));
    TSG_HIP(ctx, hipMemset(ctx->d_status, 0, sizeof(uint32_t)));
    if (st & tsg::ERR_TIMEOUT)
      return tsgh::fail(ctx, TSG_E_TIMEOUT, "a device-side signal wait timed out (status 0x%x)", st);
    return tsgh::fail(ctx, TSG_E_INVALID, "device reported invalid input (status 0x%x)", st);
  }
  return TSG_OK;
}

tsg_status tsg_device_info(tsg_ctx* ctx, int* n_cus, int* n_xcds) {
  if (!ctx) return TSG_E_INVALID;
  if (n_cus) *n_cus = ctx->n_cus;
  if (n_xcds) {
    if (!ctx->probed) {
      TSG_HIP(ctx, hipSetDevice(ctx->device));
      tsg_status st = tsg_probe_xcd(ctx);
      if (st != TSG_OK) return st;
    }
    *n_xcds = ctx->n_xcd;
  }
  return TSG_OK;
}

tsg_status tsg_enable_kernel_timing(tsg_ctx* ctx, int enable) {
  if (!ctx) return TSG_E_INVALID;
  ctx->timing = enable != 0;
  return TSG_OK;
}

tsg_status tsg_kernel_ms(tsg_ctx* ctx, int which, float* ms) {
  if (!ctx || !ms || which < 0 || which > 1) return TSG_E_INVALID;
  if (!ctx->ran[which]) return tsgh::fail(ctx, TSG_E_INVALID, "kernel %d not timed in the last call", which);
  TSG_HIP(ctx, hipEventSynchronize(ctx->ev_k[which][1]));
  TSG_HIP(ctx, hipEventElapsedTime(ms, ctx->ev_k[which][0], ctx->ev_k[which][1]));
  return TSG_OK;
}

tsg_status tsg_timeline(tsg_ctx* ctx, uint64_t* out, size_t cap, size_t* n) {
  if (!ctx || !n) return TSG_E_INVALID;
  TSG_HIP(ctx, hipSetDevice(ctx->device));
  TSG_HIP(ctx, hipDeviceSynchronize());
  uint32_t cnt = 0;
  TSG_HIP(ctx, hipMemcpy(&cnt, ctx->d_timeline_n, sizeof cnt, hipMemcpyDeviceToHost));
  size_t m = std::min<size_t>(std::min<size_t>(cnt, ctx->timeline_cap), cap);
  if (m && out) TSG_HIP(ctx, hipMemcpy(out, ctx->d_timeline, m * 4 * sizeof(uint64_t), hipMemcpyDeviceToHost));
  *n = m;
  return TSG_OK;
}

size_t tsg_workspace_bytes(int op, const int64_t* dims) {
  if (op == TSG_OP_MOE && dims) return tsg_moe_workspace(dims[0], dims[1], dims[2], dims[3], dims[4]);
  if (op == TSG_OP_MOE_AG && dims) return tsg_moe_ag_workspace(dims[0], dims[1], dims[2], dims[3], dims[4]);
  return 0;
}

tsg_status tsg_moe_workspace_layout(const int64_t* dims, int64_t* out, int n) {
  if (!out || n < 0 || n > TSG_MOE_LAYOUT_N) return TSG_E_INVALID;
  return tsg_moe_layout_fields(dims, out, n) ? TSG_OK : TSG_E_SHAPE;
}

tsg_status gemm_ag_overlap(tsg_ctx* ctx, const void* a_local, const void* a_peers, void* a_full,
                           const void* b, void* c, int c_dtype, int M, int N, int K, int R,
                           int rank, const int* arrival_order, const tsg_opts* opts, int mode,
                           void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_ag(ctx, a_local, a_peers, a_full, b, c, c_dtype, M, N, K, R, rank, arrival_order,
                   opts, mode, stream);
}

tsg_status gemm_rs_overlap(tsg_ctx* ctx, const void* x, const void* w, float* partial,
                           const float* peer_partials, float* out, int M, int N, int K, int R,
                           int rank, const tsg_opts* opts, int mode, void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_rs(ctx, x, w, partial, peer_partials, out, M, N, K, R, rank, opts, mode, stream);
}

tsg_status mlp2_pipelined(tsg_ctx* ctx, const void* x, const void* w1, void* h, const void* w2,
                          float* y, int M, int K1, int N1, int N2, const tsg_opts* opts, int mode,
                          void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_mlp2(ctx, x, w1, h, w2, y, M, K1, N1, N2, opts, mode, stream);
}

tsg_status moe_expert_combine(tsg_ctx* ctx, const void* x, const int32_t* topk_ids,
                              const float* topk_w, const void* w_up, const void* w_down,
                              float* out, int32_t* expert_counts, int32_t* sorted_ids,
                              void* workspace, size_t workspace_bytes, int T, int H, int I, int E,
                              int k, const tsg_opts* opts, int mode, void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_moe(ctx, x, topk_ids, topk_w, w_up, w_down, out, expert_counts, sorted_ids,
                    workspace, workspace_bytes, T, H, I, E, k, opts, mode, stream, false);
}

tsg_status moe_ag_group_gemm(tsg_ctx* ctx, const void* x_local, const void* x_peers, void* x_full,
                             const int32_t* topk_ids, const void* w_up, void* h, int32_t* expert_counts,
                             int32_t* sorted_ids, void* workspace, size_t workspace_bytes, int T, int H, int I,
                             int E, int k, int R, int rank, const int* arrival_order, const tsg_opts* opts,
                             int mode, void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_moe_ag(ctx, x_local, x_peers, x_full, topk_ids, w_up, h, expert_counts, sorted_ids, workspace,
                       workspace_bytes, T, H, I, E, k, R, rank, arrival_order, opts, mode, stream);
}

tsg_status ag_kv_attention(tsg_ctx* ctx, const void* q, const void* k_local, const void* k_peers,
                           const void* v_local, const void* v_peers, void* k_full, void* v_full, void* out, int S,
                           int heads, int head_dim, int R, int rank, const int* arrival_order,
                           const tsg_opts* opts, int mode, void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_attn(ctx, q, k_local, k_peers, v_local, v_peers, k_full, v_full, out, S, heads, head_dim, R, rank,
                     arrival_order, opts, mode, stream);
}

tsg_status moe_expert_combine_noalloc(tsg_ctx* ctx, const void* x, const int32_t* topk_ids,
                                      const float* topk_w, const void* w_up, const void* w_down,
                                      float* out, int32_t* expert_counts, int32_t* sorted_ids, int T,
                                      int H, int I, int E, int k, const tsg_opts* opts, int mode,
                                      void* stream) {
  if (!ctx) return TSG_E_INVALID;
  ctx->err.clear();
  return tsg_op_moe(ctx, x, topk_ids, topk_w, w_up, w_down, out, expert_counts, sorted_ids, nullptr, 0,
                    T, H, I, E, k, opts, mode, stream, true);
}

}  // extern "C"
