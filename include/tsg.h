/*
 * tsg.h -- tile-signaled GEMM paths for one MI355X (gfx950).
 *
 * A GEMM whose tiles are linked to a concurrent producer or consumer through
 * per-chunk or per-tile signals in device memory, run at one rank's share of
 * a tensor-parallel or expert-parallel layer.  Peers are stood in for by
 * buffers already resident in HBM.
 *
 * Pages cited:
 *   [TL] "TileLink: Generating Efficient Compute-Communication Overlapping
 *        Kernels using Tile-Centric Primitives" (arXiv 2503.20313).
 *   [TD] "Triton-distributed: Programming Overlapping Kernels on Distributed
 *        AI Systems with the Triton Compiler" (arXiv 2504.19442).
 *   [DG] Digest page "Resource-aware Computation-Communication Overlap for
 *        multi-GPU ML Workloads" (CTA-pipelining abstract; MoE tile-level
 *        signaling abstract).
 *
 * Conventions shared by every entry point
 *   - Matrices are dense and row-major.  "bf16" arguments hold bfloat16 bit
 *     patterns (uint16 per element); "f32" arguments hold IEEE binary32.
 *   - Every device pointer is caller-owned device memory of the current
 *     device of `ctx`, 16-byte aligned, and must stay valid until the work
 *     enqueued by the call has completed on `stream`.  Nothing is retained
 *     after that.  Output buffers must not alias inputs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are asynchronous and stream-ordered: work forks from `stream` to
 *     the context's side streams and joins back before the call returns, so
 *     later work on `stream` sees every output (gemm_ag_overlap,
 *     gemm_rs_overlap and ag_kv_attention in overlap mode on shared CUs join
 *     through their compute kernel instead: see there).
 *   - Return value: TSG_OK or a negative tsg_status.  Argument errors are
 *     detected before anything is enqueued; the message is available from
 *     tsg_last_error().  Device-side errors (a signal wait that exceeded its
 *     bounded spin) are latched in the context and reported by tsg_check().
 *     No C++ exception or abort crosses this interface.
 *   - Calls that share one context must not overlap in time on different
 *     host threads; distinct contexts are independent.
 */
#ifndef TSG_H_
#define TSG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tsg_ctx tsg_ctx;

typedef enum tsg_status {
  TSG_OK = 0,
  TSG_E_INVALID = -1,     /* null pointer, bad enum, bad option value        */
  TSG_E_SHAPE = -2,       /* dimensions violate the documented constraints   */
  TSG_E_ALIGN = -3,       /* pointer not 16-byte aligned                     */
  TSG_E_HIP = -4,         /* a HIP runtime call failed                       */
  TSG_E_TIMEOUT = -5,     /* a device-side signal wait exceeded its bound    */
  TSG_E_UNSUPPORTED = -6, /* valid request the library does not implement    */
  TSG_E_WORKSPACE = -7    /* workspace missing or smaller than required      */
} tsg_status;

/* Execution modes; all four run the same kernels.  The overlap ratio of
 * [TL] section 7.2 is (t_compute_only + t_comm_only - t_overlap) / t_comm_only. */
typedef enum tsg_mode {
  TSG_MODE_OVERLAP = 0,      /* producer and consumer run concurrently, linked
                                by tile/chunk signals                           */
  TSG_MODE_SERIAL = 1,       /* same kernels back to back on `stream`, each
                                with the whole GPU: communication first, then
                                compute (AG) or compute, then reduce/combine   */
  TSG_MODE_COMPUTE_ONLY = 2, /* the GEMM kernel(s) alone, whole GPU, every
                                wait pre-satisfied; outputs hold valid values
                                only if the data they read is already present  */
  TSG_MODE_COMM_ONLY = 3     /* the copy / reduce / combine kernel alone, with
                                the grid of overlap mode; on shared CUs it
                                runs on `stream` itself (no side stream), and
                                the GEMM+RS reduce then takes one pass per
                                unit, as when it follows the GEMM             */
} tsg_mode;

typedef enum tsg_dtype { TSG_F32 = 0, TSG_BF16 = 1 } tsg_dtype;

/* Options; a zeroed struct (or NULL) selects the defaults. */
typedef struct tsg_opts {
  /* CU partition ([TL] section 3.1, resource binding; [TD] section 3.8,
   * resource partition).  aux_cus = CUs reserved for the auxiliary kernel:
   * the copy kernel of AG+GEMM, the reduce kernel of GEMM+RS, GEMM2 of the
   * MLP, the combine kernel of MoE.  0 = the op's default; -1 = no split:
   * both kernels may use every CU and co-reside.  main_cus = CUs for the main
   * GEMM kernel (AG GEMM, RS producer GEMM, MLP GEMM1, MoE expert producer);
   * 0 = every CU not given to the auxiliary kernel.  Both sides of a split
   * must be multiples of 8 CUs (one CU per XCD per group of 8), at least 8
   * each. */
  int aux_cus;
  int main_cus;
  /* GEMM tile configuration id (BM x BN, waves), 0 = the op's default.
   * AG+GEMM: 1 = 256x256 (2x2), 2 = 256x224 (4x1), 3 = 128x128 (2x2),
   * 4 = 256x128 (2x2), 5 = 128x256 (2x2), 6 = 64x64 (1), 7 = 128x64 (2x1),
   * 8 = 256x224 (8x1, two waves per SIMD), 9 = 256x224 (4x2 on 16x16x32
   * MFMA fragments, two waves per SIMD; needs K % 128 == 0, else
   * TSG_E_UNSUPPORTED).  GEMM+RS: 1, 3, 4, 5, and 6 = 256x256 (4x2 on
   * 16x16x32 fragments, two waves per SIMD; needs K % 128 == 0, else
   * TSG_E_UNSUPPORTED; its GEMM is the fastest alone, but a reduce
   * workgroup cannot share its CU, so overlap on shared CUs runs the two
   * kernels back to back).  The MLP: 1, 3, 4, 5 (the same tile for both
   * GEMMs), 6 = the pair of 16x16x32 eight-wave tiles 128x256 (2x4) for
   * GEMM1 and 256x256 (4x2) for GEMM2, 7 = 128x256 (2x4 on 16x16x32) for
   * both; 6 and 7 need K1 and N1 multiples of 128, else TSG_E_UNSUPPORTED.
   * The MLP's default is 6 when M, N1 and N2 are all at least 1024 and K1
   * and N1 are multiples of 128, 128x256 then 256x256 on 2x2 waves of
   * 32x32x16 for other shapes of that size, and 3 below it.  An id the op
   * does not have is rejected with TSG_E_INVALID. */
  int tile;
  /* Tile order knob.  AG+GEMM: 0 = start at the local chunk and follow the
   * arrival order; 1 = plain row-major order.  GEMM+RS: 0 = local chunk
   * first, 1 = local chunk last ([TD] section 3.7).  MLP2 (both GEMMs):
   * 0 = row-block-major, so GEMM1 completes row blocks one after another
   * and GEMM2's first tiles read the first ones; 1 = groups of 8 tile rows
   * walked column by column (operand reuse in each XCD's L2 when every tile
   * runs at once).  Other values: TSG_E_INVALID (MLP2). */
  int order;
  /* Bound of every device-side signal wait, in milliseconds (0 = 2000). */
  uint32_t timeout_ms;
  /* Test hook: bit c set = the signals of AG channel c (the chunk when
   * channels = 1), RS chunk c, MLP or MoE row block c (mod 32) are never
   * published in this call, so its consumers
   * time out (the call then reports TSG_E_TIMEOUT from tsg_check).  0 in
   * normal use. */
  uint32_t debug_skip_mask;
  /* Nonzero: record per-tile device timestamps into the context's timeline
   * buffer (tsg_timeline). */
  int timeline;
  /* Workgroups of the auxiliary kernel (AG copy, RS reduce, MLP GEMM2, MoE
   * combine); 0 = the op's default. */
  int aux_wgs;
  /* AG+GEMM: width in K columns of one communication tile.  Each chunk of A
   * is moved and signalled as ceil(K / comm_tile) column slabs, and a GEMM
   * tile waits for slab s of its rows just before it loads them, so compute
   * starts on the first slab instead of the whole chunk ([TL] section 3.1:
   * communication and computation tiles are sized independently).  A power
   * of two, at least 64; 0 = 512.  Capped at 2048 and at K rounded up to a
   * power of two (one signal per chunk when K <= 2048). */
  int comm_tile;
  /* AG+GEMM, shared CUs: copy units (pieces of the first column slabs, in
   * the copy's order) that the GEMM's workgroups move themselves at their
   * start, before their first wait: workgroup b moves unit b, for b below
   * min(pull_units, GEMM grid, units).  The consumer pulls the head of the
   * data ([TL] Table 3, tile_pull_data), so compute need not wait for the
   * copy kernel to be scheduled; the copy kernel's queue hands out the units
   * after them.
   * 0 = the op's default (one unit per CU, at most the first slab's units;
   * when the whole copy is at most 1 MiB, every unit: each GEMM workgroup
   * takes units until none is left, and no copy kernel or second stream is
   * used), -1 = none.  AllGather KV + attention, overlapped: > 0 = the attention
   * workgroups take every copy unit from their own queue before the tiles;
   * 0 or -1 = a copy kernel runs beside them. */
  int pull_units;
  /* MoE: element type of the y staging between the down projection and the
   * combine.  TSG_F32 (0, default): y is kept in fp32.  TSG_BF16 (1): y is
   * rounded to bf16 (nearest even) when stored, halving the staging traffic;
   * out = g0 * y0 + g1 * y1 is then formed from the rounded values. */
  int stage_dtype;
  /* AG+GEMM: pace the arrival of the gathered data at this many GB/s (0 =
   * as fast as the copy runs).  Copy unit u (of n, in arrival order) is
   * published no earlier than total_bytes * (u + 1) / (n * rate) after the
   * first unit was taken, so that one GPU's timeline follows a link-bound
   * arrival such as seven peers over xGMI ([TD] section 3.6: AMD all-to-all
   * links; section 3.7: arrival order).  Negative: TSG_E_INVALID. */
  int arrival_gbps;
  /* AG+GEMM: 1 = move the gathered data with the DMA copy engines instead of
   * the CU copy kernel ([TD] section 3.6: intra-node AllGather on AMD with
   * copy engines, transfers issued on several streams at once, each signal
   * sent as a separate data transfer).  Each chunk gets a stream of its own;
   * on it every channel of the chunk is one hipMemcpyAsync with
   * hipMemcpyDeviceToDeviceNoCU, followed by a 64 KB NoCU copy that ends
   * with the call's signal value into the channel's 64 KB signal block,
   * whose last word the GEMM polls (the runtime runs device copies below
   * 64 KB as kernels on the CUs, larger ones on the DMA engines).  comm_tile does not apply (one slab: whole rows), the GEMM
   * pulls nothing, and no CU runs any part of the transfer, so overlap runs
   * on shared CUs.  0 = the CU copy kernel (default).  Other values, or
   * together with arrival_gbps: TSG_E_INVALID. */
  int copy_engine;
  /* AG+GEMM: channels per rank C ([TL] section 4.1, static mapping:
   * M_per_channel = M / (R C) rows, channel of row r = floor(r /
   * M_per_channel)).  Every (channel, column slab) has its own signal, and
   * a GEMM tile waits for the signals of every channel its rows span.  The
   * copy moves channel 0 of every chunk (in arrival order), then channel 1,
   * and so on, so that each step brings a sub-chunk from every peer ([TD]
   * section 3.7, Figure 8).  debug_skip_mask bit g then names global
   * channel g = chunk * C + channel.  0 = 1.  C must divide M / R, leave at
   * least 8 rows per channel (else TSG_E_SHAPE) and be at most 64
   * (else TSG_E_INVALID). */
  int channels;
  /* MoE expert compute + combine: remote-critical tiles first (the MoE
   * overlap page's producer, which covers all local experts and takes the
   * tiles whose outputs go back to other ranks first, so that their return
   * transfers start earliest).  The T tokens come from ep_ranks source
   * ranks in contiguous blocks of T / ep_ranks; this rank is ep_rank.  A row
   * block holding a pair of a token from another rank is remote-critical:
   * the producer takes the up tiles, then the down tiles, then the combine
   * units of those blocks before the others' (stable), and the table of the
   * order is readable in the workspace (TSG_MOE_RB_ORDER).  Results are
   * bit-identical to the plain row-block order.  0 = plain order (default);
   * otherwise 1 <= ep_ranks <= 32, T % ep_ranks == 0 and 0 <= ep_rank <
   * ep_ranks (else TSG_E_INVALID). */
  int ep_ranks;
  int ep_rank;
} tsg_opts;

/* ------------------------------------------------------------------ ctx */

/* Create a context on HIP device `device`: it owns the signal words (epoch
 * tagged, so no reset pass is needed between calls), the error word, the
 * side streams (CU-masked on request), events and the timeline buffer.
 * Returns TSG_E_HIP if the device cannot be used, TSG_E_UNSUPPORTED if it is
 * not a gfx950 device. */
tsg_status tsg_ctx_create(int device, tsg_ctx** out);

/* Destroy a context.  Waits for the context's side streams to drain. */
void tsg_ctx_destroy(tsg_ctx* ctx);

/* Message of the last error raised through `ctx` ("" if none).  The string
 * is owned by the context and valid until the next call on it. */
const char* tsg_last_error(const tsg_ctx* ctx);

/* Synchronise `stream`, then return TSG_E_TIMEOUT if any device-side wait
 * enqueued through `ctx` since the previous tsg_check timed out (and clear
 * that state), TSG_E_HIP on a runtime error, else TSG_OK. */
tsg_status tsg_check(tsg_ctx* ctx, void* stream);

/* Number of CUs and of XCDs (accelerator complex dies, each with its own L2)
 * of the context's device.  Either pointer may be NULL.  The XCD count is
 * read from the hardware on first use (one short kernel, synchronising). */
tsg_status tsg_device_info(tsg_ctx* ctx, int* n_cus, int* n_xcds);

/* Per-kernel timing.  When enabled, every launch is bracketed by HIP events
 * on the stream it runs on; tsg_kernel_ms returns the elapsed milliseconds of
 * the most recent call's main GEMM kernel (which = 0) and auxiliary kernel
 * (which = 1: copy, reduce, GEMM2 or combine), after the call has completed.  Returns TSG_E_INVALID if the last
 * call did not run that kernel. */
tsg_status tsg_enable_kernel_timing(tsg_ctx* ctx, int enable);
tsg_status tsg_kernel_ms(tsg_ctx* ctx, int which, float* ms);

/* Timeline of the most recent call made with opts.timeline != 0: up to
 * `cap` records of 4 uint64 each {kind<<56 | where<<32 | id, t_start,
 * t_start + ticks spent waiting for signals, t_end} in device wall-clock
 * ticks (100 MHz), copied to host memory `out`; *n receives the record
 * count.  Synchronises the device.  where = XCD<<8 | shader engine<<4 | CU
 * of the workgroup.  kind / id: 1 AG copy unit (chunk<<24 | slab<<12 |
 * piece), 2 AG GEMM tile, 3 RS GEMM tile, 4 RS reduce tile, 5 MLP GEMM1
 * tile, 6 MLP GEMM2 tile (m_tile<<16 | n_tile for tiles), 7 MoE up tile,
 * 8 MoE down tile, 9 MoE combine unit (row_block<<16 | n_tile), 10 MoE
 * gather-side up tile (row_block<<16 | n_tile), 11 attention tile
 * (head<<16 | query block). */
tsg_status tsg_timeline(tsg_ctx* ctx, uint64_t* out, size_t cap, size_t* n);

/* ------------------------------------------------------------- AG+GEMM */

/* AllGather + GEMM, one rank's share ([TL] section 2.1 and Figure 1: the
 * activation is gathered along M, then multiplied by the local weight
 * shard; [TD] section 3.2, Algorithm 2: pull-mode AllGather with one ready
 * signal per source rank; [TD] section 3.7: compute tiles start at the local
 * chunk and follow the arrival order).
 *
 * A copy kernel (the stand-in for peer arrival) writes chunk c of a_full
 * (rows [c*M/R, (c+1)*M/R)) from a_peers in arrival order, then the local
 * chunk from a_local, column slab by column slab (opts.comm_tile), releasing
 * each slab's signal; the MFMA GEMM consumer computes c = a_full * b.  A tile
 * inside the local chunk reads a_local in place and never waits; every other
 * tile waits (acquire) for slab s of the chunks its rows span just before it
 * loads slab s ([TL] section 3.1: communication tiles sized independently of
 * compute tiles).
 *
 *   a_local  bf16 [M/R x K]            this rank's shard (input)
 *   a_peers  bf16 [(R-1) x M/R x K]    the other ranks' shards in ascending
 *                                      rank order, skipping `rank` (input)
 *   a_full   bf16 [M x K]              gathered operand (output)
 *   b        bf16 [K x N]              local weight shard (input)
 *   c        [M x N], c_dtype          TSG_F32 or TSG_BF16 (round to nearest
 *                                      even of the fp32 accumulator) (output)
 *   arrival_order  host int[R-1] or NULL: order in which peer chunks arrive
 *                  (a permutation of the ranks != rank); NULL = ring order
 *                  rank+1, rank+2, ... (mod R)
 * Constraints: 1 <= R <= 32, 0 <= rank < R, M % R == 0, M >= R,
 * N % 8 == 0, K % 8 == 0, N, K >= 8 (else TSG_E_SHAPE).
 * COMPUTE_ONLY expects a_full to hold the gathered peer chunks already.
 *
 * Overlap on shared CUs (opts.aux_cus < 0, no timeline, no debug skip mask)
 * from a non-null `stream`, with a copy kernel beside the GEMM: `stream`
 * waits for the GEMM only, not for the copy kernel on the side stream.  The
 * GEMM ends only after it has observed every chunk's arrival (tiles inside
 * the local chunk wait for it after their stores), so a_full and c are
 * complete, and a_local and a_peers no longer read, when `stream` passes the
 * call; the copy kernel's workgroups may still be leaving its work queue
 * (context-internal words).
 * After a device-side error the copy may still run: tsg_check() waits for
 * the side streams before it reports. */
tsg_status gemm_ag_overlap(tsg_ctx* ctx, const void* a_local, const void* a_peers,
                           void* a_full, const void* b, void* c, int c_dtype,
                           int M, int N, int K, int R, int rank,
                           const int* arrival_order, const tsg_opts* opts,
                           int mode, void* stream);

/* ------------------------------------------------------------- GEMM+RS */

/* GEMM + ReduceScatter, one rank's share ([TL] section 2.1; [TL] Table 3
 * producer_tile_notify / consumer_tile_wait; [TD] section 3.3, Algorithm 3:
 * the reduction stream sums every rank's contribution to the local chunk as
 * its signal arrives; [TD] section 3.6: the scatter is fused into the
 * producer GEMM's epilogue).
 *
 * The producer GEMM computes partial = x * w (fp32, all M rows; row chunk c
 * is the contribution destined for rank c) and releases one done signal per
 * 128x128 tile of `partial` as soon as the tile is stored.  The reduce
 * consumer computes, for the local chunk,
 *     out = sum over ranks r of (r == rank ? partial[rank chunk] : peer r),
 * summing the peers while the GEMM runs and adding each local tile once its
 * signal is acquired.
 *
 *   x              bf16 [M x K]                 (input)
 *   w              bf16 [K x N]                 (input)
 *   partial        f32  [M x N]                 (output)
 *   peer_partials  f32  [(R-1) x M/R x N]       other ranks' partial sums for
 *                                               this rank's chunk, ascending
 *                                               rank order skipping `rank`
 *   out            f32  [M/R x N]               (output)
 * Constraints: 1 <= R <= 32, 0 <= rank < R, M % R == 0, N % 8 == 0,
 * K % 8 == 0, N, K >= 8.  COMM_ONLY expects `partial` to be computed already.
 *
 * Overlap on shared CUs (opts.aux_cus < 0, no timeline, no debug skip mask)
 * from a non-null `stream`, with the reduce beside the GEMM: `stream` waits
 * for the GEMM only.  The reduce stores out coherently and signals its end,
 * and the GEMM's last workgroup waits for that signal, so `partial` and `out`
 * are complete, and `peer_partials` no longer read, when `stream` passes the
 * call.  After a device-side error the reduce may still run: tsg_check()
 * waits for the side streams before it reports. */
tsg_status gemm_rs_overlap(tsg_ctx* ctx, const void* x, const void* w, float* partial,
                           const float* peer_partials, float* out,
                           int M, int N, int K, int R, int rank,
                           const tsg_opts* opts, int mode, void* stream);

/* ---------------------------------------------------------------- MLP2 */

/* CTA-pipelined two-GEMM MLP ([DG] CTA-pipelining abstract: dependent
 * kernels run concurrently on CTA-level dependencies, shown on a 2-layer
 * GEMM; [TL] Table 3: a consumer tile is ready when all the producer tiles
 * it depends on are done).
 *
 * GEMM1 (producer) computes h = bf16(GELU(x * w1)) (exact erf GELU on the
 * fp32 accumulator, rounded to nearest even) and, after each tile, counts
 * an arrival on the signal of each 128-row block the tile covers.  GEMM2
 * (consumer) computes y = h * w2 (fp32); each tile starts as soon as every
 * GEMM1 tile of its row blocks is done.
 *
 *   x   bf16 [M x K1], w1 bf16 [K1 x N1], h bf16 [M x N1] (output),
 *   w2  bf16 [N1 x N2], y f32 [M x N2] (output)
 * Constraints: N1 % 8 == 0, N2 % 8 == 0, K1 % 8 == 0, all >= 8, M >= 1.
 * CU partition in OVERLAP mode:
 *   aux_cus = 0 or -1 (default): shared CUs.  Both GEMMs run in one
 *     persistent kernel on every CU; its workgroups take GEMM1 tiles first
 *     and GEMM2 tiles after, from per-XCD ticket queues, and a GEMM2 tile
 *     waits for its row blocks' signals.
 *   aux_cus = q > 0: GEMM1 runs on main_cus CUs (default 256 - q) and GEMM2
 *     as a persistent consumer kernel on the other q CUs, concurrently (for
 *     example the 192/64 split: aux_cus = 64).
 * COMPUTE_ONLY runs GEMM1 then GEMM2 on the whole GPU without waits
 * (identical to SERIAL for this op); COMM_ONLY is unsupported
 * (TSG_E_UNSUPPORTED): both halves are compute. */
tsg_status mlp2_pipelined(tsg_ctx* ctx, const void* x, const void* w1, void* h,
                          const void* w2, float* y, int M, int K1, int N1, int N2,
                          const tsg_opts* opts, int mode, void* stream);

/* ----------------------------------------------------------------- MoE */

/* MoE expert compute with overlapped gate-weighted combine ([DG] MoE
 * tile-level signaling abstract: a persistent producer covering all local
 * experts emits output tiles with ready signals, and a persistent consumer
 * on a small CU partition returns them to token order as they become ready;
 * [TL] section 4.1: dynamic mapping through lookup tables filled at run
 * time; [TL] section 7.2: GroupGEMM + Scatter + Topk-Reduce).
 *
 * For every pair p = t*k + s (token t, slot s, expert e = topk_ids[t][s]):
 *     u = x[t] * w_up[e];  hh = bf16(SiLU(u));  y_p = hh * w_down[e]  (fp32)
 * and out[t] = fl(fl(topk_w[t][0] * y_(t,0)) + fl(topk_w[t][1] * y_(t,1)))
 * (k == 2; the two products are rounded to fp32 and added in slot order).
 * expert_counts[e] = number of pairs routed to e; sorted_ids = pair ids in
 * (expert, token, slot) order.
 *
 *   x         bf16 [T x H]        topk_ids  int32 [T x k]   topk_w f32 [T x k]
 *   w_up      bf16 [E x H x I]    w_down    bf16 [E x I x H]
 *   out       f32 [T x H] (output)
 *   expert_counts int32 [E] (output), sorted_ids int32 [T*k] (output)
 *   workspace device memory of at least tsg_workspace_bytes(TSG_OP_MOE, dims)
 *             bytes with dims = {T, H, I, E, k}; caller-owned, contents
 *             undefined on entry and exit.
 * Constraints: k == 2 and T * k <= 65535 (TSG_E_UNSUPPORTED otherwise),
 * 1 <= E <= 256, T >= 1, H % 8 == 0, I % 8 == 0, H, I >= 8; x, topk_ids,
 * w_up, w_down, out and workspace 16-byte aligned (TSG_E_ALIGN).  Expert ids outside [0, E) are
 * detected on the device: the affected pairs are dropped and the call's
 * tsg_check returns TSG_E_INVALID.
 * CU partition in OVERLAP mode:
 *   aux_cus = 0 or -1 (default): shared CUs.  One persistent kernel on every
 *     CU takes the up tiles, then the down tiles, then the combine units
 *     from one ticket queue; a combine unit waits for the ready signals of
 *     its down tile and of the tiles holding its tokens' other slots.
 *   aux_cus = q > 0: the producer (up and down tiles) runs on main_cus CUs
 *     (default 256 - q) and the combine as a persistent consumer kernel on
 *     the other q CUs, concurrently (the 16-CU consumer: aux_cus = 16). */
tsg_status moe_expert_combine(tsg_ctx* ctx, const void* x, const int32_t* topk_ids,
                              const float* topk_w, const void* w_up, const void* w_down,
                              float* out, int32_t* expert_counts, int32_t* sorted_ids,
                              void* workspace, size_t workspace_bytes,
                              int T, int H, int I, int E, int k,
                              const tsg_opts* opts, int mode, void* stream);

/* ------------------------------------------------- AllGather + MoE gather */

/* AllGather + Gather + grouped GEMM: the gather side of a tensor-parallel MoE
 * layer at one rank's share ([TL] section 5, Figure 5: AllGather + MoE,
 * whose dynamic routing makes the shape, rank and channel mapping of every
 * tile a lookup table filled at run time, through which the tile's loads
 * gather its tokens; [TL] section 7.2, MoE layer, first part: AG + Gather +
 * GroupGEMM; [TD] section 3.2, Algorithm 2: pull-mode AllGather, local chunk
 * first).
 *
 * The T tokens are sharded over R ranks along T: chunk c = tokens
 * [c T/R, (c+1) T/R) belongs to rank c.  A copy standing in for the peers'
 * arrival (the AllGather + GEMM path's copy units: column slabs of each
 * chunk, the local chunk first, then the peers in arrival order, each slab
 * signalled once complete) fills x_full.  For every routed pair
 * p = t*k + s with e = topk_ids[t][s]:
 *     h[p] = bf16(SiLU(x_full[t] * w_up[e]))
 * (fp32 accumulation, SiLU(u) = u / (1 + e^-u), rounded to nearest even).
 * Row tiles of the grouped GEMM are 256 rows of one expert's pairs (each
 * expert's rows padded to a multiple of 256).  Every row block's set of
 * source ranks is filled into a lookup table by the routing, and its tiles
 * wait for exactly those chunks' signals; the blocks are visited in order
 * of the arrival position of the last chunk they need (ties by block), the
 * runtime counterpart of the AllGather GEMM's swizzle.
 *
 *   x_local  bf16 [T/R x H]             this rank's tokens (input)
 *   x_peers  bf16 [(R-1) x T/R x H]     the other ranks' tokens, ascending
 *                                       rank order skipping `rank` (input)
 *   x_full   bf16 [T x H]               gathered tokens (output)
 *   topk_ids int32 [T x k]              routing of all T tokens (input)
 *   w_up     bf16 [E x H x I]           this rank's shard of every expert's
 *                                       up projection (input)
 *   h        bf16 [T*k x I]             output, in pair order
 *   expert_counts int32 [E], sorted_ids int32 [T*k]: outputs, as in
 *            moe_expert_combine
 *   workspace: at least tsg_workspace_bytes(TSG_OP_MOE_AG, {T, H, I, E, k})
 *            bytes, caller-owned, contents undefined on entry and exit.
 *   arrival_order: as in gemm_ag_overlap.
 * Modes: OVERLAP runs one persistent kernel whose workgroups take the copy
 * units first and then the tiles from one queue (a tile only waits for
 * copy units, all taken before it by workgroups that never wait); SERIAL
 * runs the copy, then the tiles; COMPUTE_ONLY the tiles without waits
 * (x_full must hold the tokens already); COMM_ONLY the copy alone.  Shared
 * CUs only (aux_cus > 0: TSG_E_UNSUPPORTED).  comm_tile sets the slab width
 * (default 2048 columns); debug_skip_mask bit c withholds chunk c's signals.
 * Constraints: k == 2, T * k <= 65535, 1 <= R <= 32, T % R == 0,
 * 1 <= E <= 256, H % 8 == 0, I % 8 == 0, H, I >= 8, 16-byte aligned
 * pointers.  Expert ids outside [0, E) are dropped and reported by
 * tsg_check as TSG_E_INVALID. */
tsg_status moe_ag_group_gemm(tsg_ctx* ctx, const void* x_local, const void* x_peers, void* x_full,
                             const int32_t* topk_ids, const void* w_up, void* h,
                             int32_t* expert_counts, int32_t* sorted_ids,
                             void* workspace, size_t workspace_bytes,
                             int T, int H, int I, int E, int k, int R, int rank,
                             const int* arrival_order, const tsg_opts* opts, int mode,
                             void* stream);

/* ------------------------------------------------ AllGather KV + attention */

/* AllGather of the key/value context + self-attention, sequence parallel,
 * one rank's share ([TL] section 2.1: the context is sharded across ranks
 * and gathered before the attention; [TL] section 5, Figure 6: AllGather
 * KV + self-attention, the communication tile being one rank's share of the
 * sequence and the computation tile a different one, with tile-centric
 * mapping keeping the barriers between them; [TL] section 7.2: two batched
 * GEMMs and a softmax fused as in Flash-Attention).
 *
 * The S tokens are sharded over R ranks along the sequence: chunk c = rows
 * [c S/R, (c+1) S/R) belongs to rank c.  A copy standing in for the peers'
 * arrival (the AllGather copy's units over K, then V, each viewed as an
 * [S x heads*head_dim] matrix: column slabs of comm_tile columns, default
 * one head, of each chunk; peers in arrival order, the own chunk last; each
 * (chunk, slab) signalled once complete) fills k_full and v_full.  For
 * every head h and local query q (no mask):
 *     out[q, h] = sum_j softmax_j(q[q, h] . K[j, h] / sqrt(head_dim)) V[j, h]
 * over all S keys j, with fp32 scores and accumulators, probabilities
 * rounded to bf16 for the second product, and out rounded to bf16.  A tile
 * (one head, 128 queries) takes the chunks in arrival order, its own chunk
 * first, read in place from k_local / v_local; before a peer chunk it waits
 * for the K and V signals of the slabs holding its head.
 *
 *   q        bf16 [S/R x heads x head_dim]   this rank's queries (input)
 *   k_local, v_local  bf16 [S/R x heads x head_dim]   (input)
 *   k_peers, v_peers  bf16 [(R-1) x S/R x heads x head_dim], ascending rank
 *            order skipping `rank` (input)
 *   k_full, v_full    bf16 [S x heads x head_dim]   gathered (output)
 *   out      bf16 [S/R x heads x head_dim]   (output)
 *   arrival_order: as in gemm_ag_overlap.
 * Modes: OVERLAP runs the copy as a small kernel beside the attention
 * kernel on the same CUs (a copy wave per SIMD next to two attention
 * waves), moving the units arrival position by position (K and V of every
 * slab of the first peer, then of the next), while the tiles start on their
 * own chunks; with opts.pull_units > 0 (or where the two kernels cannot share
 * a CU) it runs one persistent kernel whose workgroups take the copy units
 * first and then the tiles from one queue.  SERIAL runs the copy, then the
 * tiles; COMPUTE_ONLY the tiles without waits (k_full / v_full must hold
 * the context already); COMM_ONLY the copy alone.  Shared CUs only (aux_cus
 * > 0: TSG_E_UNSUPPORTED).  debug_skip_mask bit c withholds chunk c's
 * signals.  Constraints: head_dim == 128 (else TSG_E_UNSUPPORTED),
 * 1 <= R <= 32, S a positive multiple of 64 R, heads >= 1, comm_tile a power
 * of two in [64, 2048] or 0, 16-byte aligned pointers.
 *
 * With the copy kernel beside the tiles, from a non-null `stream` and with no
 * timeline or debug skip mask, `stream` waits for the attention kernel only:
 * its tiles wait for their head's own-chunk slabs after their stores, so
 * k_full, v_full and out are complete, and the local and peer chunks no
 * longer read, when `stream` passes the call; the copy kernel's workgroups
 * may still be leaving its work queue (context-internal words). */
tsg_status ag_kv_attention(tsg_ctx* ctx, const void* q, const void* k_local, const void* k_peers,
                           const void* v_local, const void* v_peers, void* k_full, void* v_full,
                           void* out, int S, int heads, int head_dim, int R, int rank,
                           const int* arrival_order, const tsg_opts* opts, int mode, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_expert_combine with the workspace taken from the library's own static
 * device buffer of TSG_MOE_NOALLOC_BYTES (64 MiB) instead of an argument.
 * Every other argument, the results and the errors are those of
 * moe_expert_combine.  The call allocates nothing (no hipMalloc, hipFree,
 * stream creation or memset) and queues its work on `stream` only, so it
 * supports shared CUs only: aux_cus > 0 or opts.timeline != 0 give
 * TSG_E_UNSUPPORTED.  Dims whose workspace (tsg_workspace_bytes) exceeds the
 * buffer give TSG_E_WORKSPACE, before anything is queued.  The buffer is
 * one per GPU, set up by tsg_ctx_create and held until the process ends;
 * every call on that GPU shares it (each call rebuilds all of its content),
 * so calls that overlap in time on one GPU (different streams or contexts)
 * race and must not be issued. */
#define TSG_MOE_NOALLOC_BYTES (64u << 20)
tsg_status moe_expert_combine_noalloc(tsg_ctx* ctx, const void* x, const int32_t* topk_ids,
                                      const float* topk_w, const void* w_up, const void* w_down,
                                      float* out, int32_t* expert_counts, int32_t* sorted_ids,
                                      int T, int H, int I, int E, int k,
                                      const tsg_opts* opts, int mode, void* stream);

enum { TSG_OP_AG = 0, TSG_OP_RS = 1, TSG_OP_MLP2 = 2, TSG_OP_MOE = 3, TSG_OP_MOE_AG = 4 };

/* Workspace bytes an op needs for `dims` (TSG_OP_MOE and TSG_OP_MOE_AG:
 * {T, H, I, E, k}); 0 for ops that need none or for invalid dims. */
size_t tsg_workspace_bytes(int op, const int64_t* dims);

/* Layout of the MoE workspace for dims = {T, H, I, E, k}, so that the
 * intermediate results of a completed call can be read back (tests compare
 * them with an independent reference).  out[i] receives field i, for
 * i < n <= TSG_MOE_LAYOUT_N; region fields are byte offsets from the start
 * of the workspace.  After moe_expert_combine has completed on its stream
 * the regions hold ([TL] section 4.1, dynamic mapping: these are the lookup
 * tables that map row tiles to experts and rows to pairs, filled at run
 * time from topk_ids):
 *   TSG_MOE_META       int32[2]: row blocks in use, routed pairs kept
 *   TSG_MOE_OFFS       int32[E+1]: exclusive prefix sum of expert_counts
 *   TSG_MOE_POFFS      int32[E+1]: first padded row of each expert (every
 *                      expert's rows are padded to a multiple of BM)
 *   TSG_MOE_RB_EXPERT  int32[RB_MAX]: expert of each BM-row block, -1 past
 *                      the last block in use
 *   TSG_MOE_ROW_PAIR   int32[ROWS_MAX]: pair p = t*k + s held by each padded
 *                      row, -1 for padding rows
 *   TSG_MOE_ROW_TOKEN  int32[ROWS_MAX]: token of each padded row, -1 for
 *                      padding rows
 *   TSG_MOE_PAIR_ROW   int32[T*k]: padded row of each pair
 *   TSG_MOE_H          bf16 [ROWS_MAX x I]: bf16(SiLU(x[t] w_up[e])) of the
 *                      pair in each row (padding rows: unspecified)
 *   TSG_MOE_Y          [ROWS_MAX x H]: y of the pair in each row, fp32 (bf16
 *                      with stage_dtype = TSG_BF16; padding rows:
 *                      unspecified)
 *   TSG_MOE_RB_ORDER   int32[RB_MAX]: with opts.ep_ranks > 0, the row blocks
 *                      in use in the order the producer takes them
 *                      (remote-critical first, each group by block index;
 *                      entries past the blocks in use unspecified); not
 *                      written otherwise
 *   TSG_MOE_RB_MASK    uint32[RB_MAX]: with opts.ep_ranks > 0, bit c of
 *                      entry rb set when a row of block rb holds a token of
 *                      source rank c; not written otherwise
 * TSG_MOE_TOTAL = tsg_workspace_bytes; TSG_MOE_ROWS_MAX, TSG_MOE_RB_MAX:
 * the padded rows and row blocks the layout provides for; TSG_MOE_BM: rows
 * per block.  Returns TSG_E_SHAPE for dims moe_expert_combine rejects,
 * TSG_E_INVALID for a null `out` or n outside [0, TSG_MOE_LAYOUT_N]. */
enum {
  TSG_MOE_META = 0, TSG_MOE_OFFS, TSG_MOE_POFFS, TSG_MOE_RB_EXPERT, TSG_MOE_ROW_PAIR, TSG_MOE_ROW_TOKEN,
  TSG_MOE_PAIR_ROW, TSG_MOE_H, TSG_MOE_Y, TSG_MOE_TOTAL, TSG_MOE_ROWS_MAX, TSG_MOE_RB_MAX, TSG_MOE_BM,
  TSG_MOE_RB_ORDER, TSG_MOE_RB_MASK, TSG_MOE_LAYOUT_N
};
tsg_status tsg_moe_workspace_layout(const int64_t* dims, int64_t* out, int n);

#ifdef __cplusplus
}
#endif
#endif /* TSG_H_ */
