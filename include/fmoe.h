/*
 * fmoe.h -- C ABI of libfmoe, a fused mixture-of-experts layer for AMD Instinct MI355X
 * (gfx950): router top-k (softmax or sigmoid), per-expert grouping of the routed rows,
 * grouped gate/up GEMM with SiLU-and-mul, grouped down GEMM (bf16 weights, or OCP e4m3
 * weights with one fp32 scale per [128,128] block and per-token per-128-column activation
 * scales), and the routing-weighted combine back to token order.
 *
 * Sources (web pages, cited by title and section):
 *   [H20]     "vLLM Community Traces H20 MoE Scheduling Inefficiency to Expert-Load Kernel
 *             Selection": paragraph 2 (a fused-experts entry point that takes expert-parallel
 *             size and rank and FP8 block scales), paragraph 3 (workspace sized for the worst
 *             case first; tile choice from rows per expert = ceil(tokens*top_k/experts) >= 1),
 *             paragraph 4 (uniform and concentrated routing differ).
 *   [PR39593] "PR #39593: [Bug]: Fix FlashInfer CUTLASS BF16 + CUDA graphs IMA": Root cause
 *             (NaN logits made top-k repeat one id; repeated ids crashed the expert kernels;
 *             the FP8 conversion clamps with fminf/fmaxf to +-448), Fix (NaN -> -FLT_MAX in the
 *             router; K distinct ids), Test Plan (128x128 top-8 router micro-benchmark).
 *   [LAB6]    "Lab notes #6: We tuned vLLM's MoE kernels on an H100 ...": intro (fp8_w8a8,
 *             block_shape [128,128], E=128, N=768).
 *
 * Conventions for every entry point:
 *   - All device pointers are plain device addresses; the caller allocates and owns every
 *     buffer (inputs, outputs, weights, workspace).  The library allocates nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; none synchronises except fmoe_read_stats.
 *   - All argument checks run on the host before anything is enqueued.  A failed check
 *     returns its status and enqueues nothing.  A launch error returns FMOE_ERR_HIP.
 *   - tokens == 0 returns FMOE_OK and launches nothing.
 *   - Identical inputs give bitwise identical outputs (no order-dependent atomics).
 *   - One workspace must not be used by two calls that run concurrently.
 *   - Row-major layouts everywhere; "[A,B]" lists dimensions outermost first.
 */
#ifndef FMOE_H
#define FMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMOE_ABI_VERSION 4

/* Limits of the library (checked, FMOE_ERR_UNSUPPORTED beyond them). */
#define FMOE_MAX_EXPERTS 1024     /* experts (total) for the router; local experts likewise   */
#define FMOE_MAX_TOP_K 64         /* top_k                                                     */
#define FMOE_MAX_DIM 65536        /* hidden and inter                                          */
#define FMOE_MAX_ASSIGNMENTS (1 << 23) /* tokens * top_k                                       */

typedef enum {
    FMOE_OK = 0,
    FMOE_ERR_ARG = 1,          /* null pointer, misaligned pointer, inconsistent sizes   */
    FMOE_ERR_UNSUPPORTED = 2,  /* a size or dtype outside the limits of the library      */
    FMOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than fmoe_workspace_bytes              */
    FMOE_ERR_HIP = 4           /* a HIP launch or runtime call failed                    */
} fmoe_status;

typedef enum { FMOE_BF16 = 0, FMOE_FP32 = 1, FMOE_FP8_E4M3 = 2 } fmoe_dtype; /* e4m3 = OCP E4M3FN, max 448 */
typedef enum { FMOE_SOFTMAX = 0, FMOE_SIGMOID = 1 } fmoe_scoring;

/* Shape of one layer call.
 *   tokens  T >= 0, T*top_k <= FMOE_MAX_ASSIGNMENTS
 *   hidden H, inter I: positive multiples of 128, at most 65536
 *   experts E (total physical expert slots, [H20] paragraph 3), 1 <= top_k <= min(E, 64)
 *   ep_size divides E; this rank owns experts [ep_rank*E/ep_size, (ep_rank+1)*E/ep_size)
 *   ([H20] paragraph 2); E_loc = E/ep_size <= 1024.
 *   weight_dtype: FMOE_BF16 or FMOE_FP8_E4M3. */
typedef struct {
    int32_t tokens, hidden, inter, experts, top_k, ep_size, ep_rank;
    int32_t weight_dtype;
} fmoe_shape;

/* Local expert weights, output features by rows, the reduction dimension contiguous:
 *   gate, up [E_loc, I, H];  down [E_loc, H, I]   (bf16, or e4m3 codes one byte each)
 *   FP8 only: gate_scale, up_scale [E_loc, I/128, H/128]; down_scale [E_loc, H/128, I/128]
 *   (fp32 per [128,128] block, [H20] paragraph 2, [LAB6] intro).  bf16: all three NULL.
 *   Weight pointers must be 16-byte aligned. */
typedef struct {
    const void *gate, *up, *down;
    const float *gate_scale, *up_scale, *down_scale;
} fmoe_weights;

/* Counters the kernels leave in the workspace header (read with fmoe_read_stats). */
typedef struct {
    int64_t dropped_ids;     /* ids outside [0, E) seen by the grouping step (skipped)       */
    int32_t local_rows;      /* R = rows of this rank's experts                              */
    int32_t max_rows;        /* largest per-expert row count                                */
    int32_t empty_experts;   /* local experts with no row                                   */
    int32_t m_tiles;         /* row tiles of the grouped GEMMs (light + heavy)              */
    int32_t rows_estimate;   /* host plan: max(1, ceil(T*top_k/E))                          */
    int32_t tile_rows;       /* host plan: largest light tile; an expert with 1..tile_rows rows
                                is one light tile, a heavier one heavy tiles (FP8 when every
                                expert fits 8 light tiles: ceil(c / tile_rows) light tiles)  */
    int32_t heavy_tiles;     /* row tiles of the experts cut into heavy tiles               */
    int32_t heavy_rows;      /* largest heavy tile: 256 rows, an expert with c rows getting
                                ceil(c / 256) tiles of about equal size; 320 when the grouping
                                step cut every expert of 257..320 rows as one tile (bf16)    */
    int32_t light_rows;      /* rows of the light tiles                                     */
    int32_t split_light_tiles; /* light tiles whose gate/up GEMM ran on the split-reduction
                                kernel because they held few rows on average (the grouping's
                                choice from the real counts; 0: the streaming kernel or the
                                host plan's kernel took them)                                  */
} fmoe_stats;

int fmoe_abi_version(void);
const char* fmoe_status_string(int status);

/* Bytes of workspace a call with this shape needs: the worst case over all routings (every
 * assignment local, any per-expert imbalance), computed before any routing is known
 * ([H20] paragraph 3).  Host only. */
int fmoe_workspace_bytes(const fmoe_shape* shape, size_t* bytes);

/* Router linear: logits[t,e] = sum_h x[t,h] * w_r[e,h] in fp32, one fused multiply-add per
 * h in ascending h order starting from 0 (so the result is reproducible bit for bit).
 *   x [T,H] bf16, w_r [E,H] bf16 -> logits [T,E] fp32.  H >= 1, E >= 1. */
int fmoe_router_logits(const void* x, const void* w_r, int32_t T, int32_t H, int32_t E,
                       float* logits, void* stream);

/* Router top-k ([PR39593] Fix): each logit is read as fp32, NaN becomes -FLT_MAX and +-inf
 * become +-FLT_MAX; experts are ordered by that value, larger first, lower index first
 * among equals; the first k are written best first, always k distinct ids.
 *   logits [T,E] (logits_dtype FMOE_BF16 or FMOE_FP32) -> topk_ids [T,k] int32,
 *   topk_weights [T,k] fp32:
 *     softmax: exp(v - max) / sum over all E, or over the k picks when renormalize != 0;
 *     sigmoid: 1/(1+exp(-v)); renormalize != 0 divides by the sum of the k picks
 *              (1/k each when that sum is 0). */
int fmoe_router_topk(const void* logits, int32_t logits_dtype, int32_t T, int32_t E, int32_t k,
                     int32_t scoring, int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                     void* stream);

/* Grouped (group-limited) top-k router.  The experts form n_group groups of E/n_group
 * consecutive indices; a group's key is its largest sanitised logit; the topk_group groups with
 * the largest keys are kept (the lower group first among equal keys); the k ids are then picked
 * as in fmoe_router_topk among the kept groups' experts only, with the same weights (an
 * unrenormalised softmax still divides by all E).  "PR #39593: [Bug]: Fix FlashInfer CUTLASS
 * BF16 + CUDA graphs IMA", Root cause, names this router beside the plain one; the definition
 * is the reading taken here.  Requires E % n_group == 0, 1 <= n_group <= 64,
 * 1 <= topk_group <= n_group and k <= topk_group * E / n_group (FMOE_ERR_ARG otherwise;
 * n_group > 64: FMOE_ERR_UNSUPPORTED), so the k ids are distinct; all-NaN rows give 0..k-1.
 * topk_group == n_group is fmoe_router_topk.  Buffers, dtypes and errors otherwise as
 * fmoe_router_topk. */
int fmoe_router_topk_grouped(const void* logits, int32_t logits_dtype, int32_t T, int32_t E, int32_t k,
                             int32_t n_group, int32_t topk_group, int32_t scoring, int32_t renormalize,
                             int32_t* topk_ids, float* topk_weights, void* stream);

/* Per-expert grouping of the T*k assignments topk_ids [T,k] for this rank.  [H20] paragraph
 * 3: the kernel and tile choice need the rows assigned to each expert, not the token count;
 * [PR39593] Root cause: repeated ids in one token must not break the expert kernels.
 * (shape gives T, E, k, ep_size, ep_rank; H, I and weight_dtype only size the workspace):
 *   counts [E_loc]      rows per local expert
 *   offsets [E_loc+1]   exclusive prefix sum of counts, offsets[E_loc] = R
 *   perm_src [T*k]      first R entries: flat index t*k+j of each grouped row, experts
 *                       ascending, flat index ascending inside an expert (stable)
 *   inv_perm [T*k]      grouped row of each assignment, -1 when not local
 * Ids outside [0,E) are skipped and counted (fmoe_read_stats); repeated ids in a token are
 * legal and give separate rows.  ws/ws_bytes as for fmoe_experts. */
int fmoe_route_permute(const fmoe_shape* shape, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* Expert computation for given routing ([H20] paragraph 2: a fused-experts call that takes the
 * routing, the expert-parallel size and rank and FP8 block scales; [LAB6] intro: w8a8 with
 * [128,128] weight blocks; [PR39593] Root cause: repeated ids, and the e4m3 clamp to +-448):
 *   out[t,:] = sum over j ascending with a local id of
 *   topk_weights[t,j] * W_down[l] (silu(W_gate[l] x[t]) * (W_up[l] x[t])),  l = id - ep_rank*E_loc,
 * computed as grouping -> (FP8: per-token per-128 e4m3 quantisation of x) -> grouped gate/up
 * GEMM with fused SiLU-and-mul -> (FP8: quantisation of the activation) -> grouped down GEMM ->
 * weighted combine in fp32, rounded once to bf16.  Tokens with no local id get zeros.  With bf16
 * weights and at most 64 assignments (T*k <= 64, I <= 1024) the down GEMM and the combine are one
 * launch that keeps each row's down projection in fp32 (no bf16 rounding before the weighted
 * sum); results equal the two-launch path's within the layer's rounding.
 *   x [T,H] bf16 (16-byte aligned); topk_ids [T,k] int32; topk_weights [T,k] fp32;
 *   out [T,H] bf16 (16-byte aligned); ws of at least fmoe_workspace_bytes(shape). */
int fmoe_experts(const fmoe_shape* shape, const void* x, const int32_t* topk_ids,
                 const float* topk_weights, const fmoe_weights* w, void* out,
                 void* ws, size_t ws_bytes, void* stream);

/* Whole layer: the router of [PR39593] Fix (fmoe_router_topk) on logits [T,E], then the
 * expert computation of [H20] paragraph 2 (fmoe_experts), with the tile plan from the
 * rows-per-expert estimate of [H20] paragraph 3.  topk_ids_out [T,k] and topk_weights_out
 * [T,k] receive the routing when not NULL (otherwise it stays in ws). */
int fmoe_forward(const fmoe_shape* shape, const void* x, const void* logits, int32_t logits_dtype,
                 int32_t scoring, int32_t renormalize, const fmoe_weights* w, void* out,
                 int32_t* topk_ids_out, float* topk_weights_out, void* ws, size_t ws_bytes,
                 void* stream);

/* Tile plan for tuning harnesses (the tile-space sweep of bench.py).  The host heuristic picks
 * the largest light row tile from the rows-per-expert estimate max(1, ceil(T*top_k/E)) ("vLLM
 * Community Traces H20 MoE Scheduling Inefficiency to Expert-Load Kernel Selection",
 * paragraphs 3-4) and the reduction split from the expected task count; a nonzero field here
 * replaces that choice:
 *   tile_rows      largest rows of a light row tile: 16 or 32 (experts with more rows are cut
 *                  into heavy tiles on the device)
 *   split_gate_up  wavefronts that split the reduction of a light tile in the gate/up GEMM:
 *                  1 (the streaming kernel), 2 or 4
 *   split_down     the same for the down GEMM
 *   light_tiles    light tiles one expert may take: 1 (experts above tile_rows rows are cut
 *                  into heavy tiles) or 8 (experts of up to 8*tile_rows rows are cut into
 *                  light tiles, and the heavy-tile launches are left out when no expert can
 *                  hold more: at most T rows for router ids, T*top_k for caller ids); the
 *                  heuristic takes 8 for FP8 weights and 1 for bf16
 *   heavy_rows     largest heavy tile: 256, or 320 (bf16 weights only): an expert of 257..320
 *                  rows is then one tile of five 64-row groups instead of two tiles.  The
 *                  heuristic decides on the device from the real counts: 320 when the heavy
 *                  tiles of 256 rows give every compute unit at least four tasks in both
 *                  GEMMs (a throughput-bound launch, where one task in place of two saves
 *                  copies), else 256 (a longer task would lengthen the launch) */
typedef struct {
    int32_t tile_rows, split_gate_up, split_down, light_tiles, heavy_rows;
} fmoe_plan;

/* fmoe_forward with the nonzero fields of *plan (NULL: none) in place of the heuristic's
 * choices.  FMOE_ERR_ARG for a field outside the values above; FMOE_ERR_UNSUPPORTED when an
 * FP8 layer's 32-row tile would not fit the activation scales of a split tile in 64 KB of LDS
 * (the limit the heuristic also applies), or for heavy_rows 320 with FP8 weights.  fmoe_workspace_bytes(shape) fits every plan.
 * Results equal fmoe_forward's within the layer's rounding (the reduction order of a split
 * tile differs). */
int fmoe_forward_planned(const fmoe_shape* shape, const void* x, const void* logits,
                         int32_t logits_dtype, int32_t scoring, int32_t renormalize,
                         const fmoe_weights* w, void* out, int32_t* topk_ids_out,
                         float* topk_weights_out, void* ws, size_t ws_bytes, void* stream,
                         const fmoe_plan* plan);

/* Per-row, per-128-column e4m3 quantisation of activations (the w8a8 activation scheme of
 * [LAB6] intro; the saturating fminf/fmaxf clamp of [PR39593] Root cause), the code the
 * layer runs on x and on the gate/up activation:
 *   for every row r and group g of 128 columns: amax = max |x| over the group (NaN ignored);
 *   s[r,g] = amax/448 (1 when amax == 0); inv = 1/s; q = e4m3(max(min(x*inv, 448), -448))
 *   (round to nearest even; a NaN value becomes +448).  IEEE fp32 division and product.
 *   x [rows, cols] bf16 (x_dtype FMOE_BF16) or fp32 (FMOE_FP32) -> q [rows, cols] e4m3 codes,
 *   s [rows, cols/128] fp32.  cols a positive multiple of 128, at most FMOE_MAX_DIM;
 *   rows >= 0 (0: no-op); x, q 16-byte aligned. */
int fmoe_act_quant(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, uint8_t* q, float* s,
                   void* stream);

/* Byte offsets of the layer's intermediate buffers inside a workspace of
 * fmoe_workspace_bytes(shape) bytes, for tests and inspection (0: the buffer does not exist
 * for this weight dtype).  After fmoe_forward / fmoe_experts on ws (stream synchronised):
 *   x_codes [T,H] e4m3, x_scales [T,H/128] fp32 (FP8): the quantised x;
 *   h_f32 [T*k,I] fp32 (FP8): the gate/up activation of grouped row p, when the layer
 *       quantised it in a separate pass (some expert could take a heavy row tile);
 *   h_codes [T*k,I] e4m3, h_scales [T*k,I/128] fp32 (FP8): the quantised activation;
 *   h_bf16 [T*k,I] bf16 (bf16 weights): the activation;
 *   y [T*k,H] bf16: the down projection of grouped row p (before the routing weight); not
 *       written when the down GEMM and the combine ran as one launch (bf16, T*k <= 64);
 *   perm_src, inv_perm [T*k] int32: the grouping (as fmoe_route_permute).
 * Only the first R grouped rows (fmoe_read_stats local_rows) hold data. */
typedef struct {
    size_t x_codes, x_scales, h_f32, h_codes, h_scales, h_bf16, y, perm_src, inv_perm, total;
} fmoe_layout;
int fmoe_workspace_layout(const fmoe_shape* shape, fmoe_layout* out);

/* One grouped GEMM stage of fmoe_experts on operands the caller gives, for tests of the GEMM
 * kernels (integer data makes every kernel's result exact) and for tuning.  topk_ids [T,k]
 * are grouped as fmoe_route_permute does (caller ids: repeats legal, out-of-range dropped),
 * the row tiles are cut from the real counts with the tile plan (*plan, NULL: the heuristic;
 * fields as for fmoe_forward_planned), and the kernels fmoe_experts would launch run:
 *   stage 0 (gate/up): a = activation rows [T,H]: bf16, or e4m3 codes with a_scale [T,H/128];
 *     grouped row p (token t = perm_src[p] / k, local expert l) gets
 *     silu(a[t] . W_gate[l]^T) * (a[t] . W_up[l]^T) in out [T*k, I] as
 *       out_dtype FMOE_BF16 (bf16 weights), FMOE_FP32 (FP8 weights), or FMOE_FP8_E4M3 (FP8
 *       weights: codes, with out_scale [T*k, I/128] as fmoe_act_quant computes them);
 *   stage 1 (down): a = grouped rows [T*k, I]: bf16, or codes with a_scale [T*k, I/128];
 *     out [T*k, H] bf16: row p = a[p] . W_down[l]^T  (out_dtype FMOE_BF16).
 * FP8 operands are used as code * scale per 128-deep block (weights per [128,128] block).
 * Rows p >= R are not written.  ws: fmoe_workspace_bytes(shape) bytes.  Errors as
 * fmoe_experts; FMOE_ERR_ARG for a stage or out_dtype that does not fit the weights. */
int fmoe_grouped_gemm(const fmoe_shape* shape, const fmoe_plan* plan, int32_t stage, const int32_t* topk_ids,
                      const void* a, const float* a_scale, const fmoe_weights* w, int32_t out_dtype, void* out,
                      float* out_scale, void* ws, size_t ws_bytes, void* stream);

/* Stages of fmoe_forward, in launch order, for fmoe_forward_profiled. */
enum {
    FMOE_STAGE_ROUTER = 0, FMOE_STAGE_GROUP = 1, FMOE_STAGE_QUANT_X = 2,
    FMOE_STAGE_GEMM1 = 3,        /* gate/up GEMM of the light row tiles                       */
    FMOE_STAGE_GEMM1_SPLIT = 4,  /* gate/up GEMM of the light row tiles that the grouping gave
                                    to the split-reduction kernel (few rows per tile on average,
                                    see fmoe_stats.split_light_tiles; may find none)            */
    FMOE_STAGE_GEMM1_HEAVY = 5,  /* gate/up GEMM of the heavy row tiles (may find none)       */
    FMOE_STAGE_QUANT_H = 6, FMOE_STAGE_GEMM2 = 7, FMOE_STAGE_GEMM2_HEAVY = 8, FMOE_STAGE_COMBINE = 9,
    FMOE_NUM_STAGES = 10
};

/* fmoe_forward that also records stage_events[i] (hipEvent_t, created by the caller) on the
 * stream just before stage i, and stage_events[FMOE_NUM_STAGES] after the last one; a stage
 * that does not run for this dtype records its event pair back to back.  NULL entries are
 * skipped (each recorded event adds a few microseconds to the stream).  For timing. */
int fmoe_forward_profiled(const fmoe_shape* shape, const void* x, const void* logits,
                          int32_t logits_dtype, int32_t scoring, int32_t renormalize,
                          const fmoe_weights* w, void* out, int32_t* topk_ids_out,
                          float* topk_weights_out, void* ws, size_t ws_bytes, void* stream,
                          void* const* stage_events);

/* Largest workspace fmoe_forward_noalloc can use: the size of the library's static device
 * buffer (one per GPU the library runs on, held until the process ends). */
#define FMOE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)

/* fmoe_forward without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static device buffer of FMOE_NOALLOC_MAX_WORKSPACE bytes inside the library,
 * one per GPU; the first call on a GPU looks up that GPU's copy (hipGetSymbolAddress, which
 * allocates nothing) and keeps its address.  The call itself allocates nothing and calls no
 * allocating routine.  A shape whose fmoe_workspace_bytes exceeds the buffer returns
 * FMOE_ERR_WORKSPACE and enqueues nothing (the 2048/768/128-expert top-8 layer fits up to
 * T = 1024 in bf16; the 7168-wide FP8 shard at T = 288 fits).  Every call on one GPU shares
 * that GPU's buffer, which keeps the last call's contents; nothing in it needs to start at
 * zero (each call writes every value it later reads).  Calls that overlap on one GPU (two
 * streams or two threads) race on the buffer: the caller must order them.  Works on the
 * current device; the stream must belong to it.  Arguments and results otherwise as
 * fmoe_forward; fmoe_read_stats cannot read this buffer. */
int fmoe_forward_noalloc(const fmoe_shape* shape, const void* x, const void* logits, int32_t logits_dtype,
                         int32_t scoring, int32_t renormalize, const fmoe_weights* w, void* out,
                         int32_t* topk_ids_out, float* topk_weights_out, void* stream);

/* Copies the counters of the last call that used ws into *out.  Synchronises the stream:
 * for tests and benchmarks, not for the hot path. */
int fmoe_read_stats(const void* ws, void* stream, fmoe_stats* out);

#ifdef __cplusplus
}
#endif
#endif /* FMOE_H */
