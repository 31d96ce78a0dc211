/*
 * moe.h -- C ABI of a dropless Mixture-of-Experts layer forward for AMD MI355X (gfx950).
 *
 * The operation is the four-stage MoE forward described on the summary page of
 * "Scalable Training of Mixture-of-Experts Models with Megatron Core" (section
 * "Method", first paragraph): a router (learned linear projection, optionally in
 * FP32, then softmax or sigmoid scores and top-k selection), a dispatcher that
 * permutes tokens so each expert's rows are contiguous, all local experts in one
 * grouped GEMM, and a combine step; an optional shared expert sees every token.
 * "Sync-free execution for dropless MoE" (same page, "Method", second paragraph)
 * and "CUDA-Graph-friendly sync-free execution" (same page, "TL;DR") fix the
 * execution model: nothing here reads device data back to the host.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to row-major, densely packed arrays, owned
 *    by the caller; the library allocates no memory and keeps no per-call state (the one
 *    static device array of moe_forward_static aside).
 *    Pointers must be 16-byte aligned.  Inputs and outputs must not alias.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream),
 *    never synchronise, never copy to the host, and are HIP-graph capturable.
 *  - Arguments are validated on the host before anything is launched; a failed check
 *    returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE /
 *    MOE_ERR_TOO_LARGE and launches nothing.  A launch failure returns MOE_ERR_HIP.  Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - Integer outputs (expert ids, counts, offsets, permutation) are deterministic:
 *    the same inputs give the same bits on every run.  No floating-point atomics are
 *    used anywhere, so floating outputs are run-to-run deterministic as well.
 *  - Limits: 1 <= k <= min(E, 16); E <= 512; T*k < 2^31.
 *  - Readings fixed where the pages are silent: selection ranks the fp32 logit plus
 *    the optional routing bias (one fp32 add); gates use the unbiased logit; ties break
 *    to the lower expert index; slots are ordered by key descending; inside an expert
 *    rows follow increasing token index; the first expert matrix's 2F columns are
 *    [gate | up] and h = SiLU(gate) * up; the shared expert has gate 1.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2
#define MOE_MAX_TOPK 16
#define MOE_MAX_EXPERTS 512

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, size out of range, inconsistent sizes     */
  MOE_ERR_UNSUPPORTED = 2, /* valid request this build does not implement            */
  MOE_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than required     */
  MOE_ERR_HIP = 4,         /* a HIP launch failed (hipGetLastError after the launch) */
  MOE_ERR_TOO_LARGE = 5    /* moe_forward_static: more scratch needed than it holds     */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2, /* OCP E4M3 without infinities ("e4m3fn"), max 448 */
  MOE_MXFP4 = 3     /* OCP MXFP4: FP4 E2M1 elements (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), two per
                       byte (element 2i in the low nibble), one E8M0 scale byte (2^(e - 127)) per 32
                       consecutive elements along the contraction; expert GEMMs only */
} moe_dtype;

typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;

/* ---------------------------------------------------------------------------------------
 * Route (summary page, "Method", first paragraph: the router).
 *   x        [T, H]   x_dt = MOE_F32 or MOE_BF16
 *   w_router [H, E]   fp32
 *   bias     [E] fp32 or NULL: added to the logit (one fp32 add) for SELECTION only
 *   logits   [T, E] fp32 out, or NULL (not written).  When written, these are exactly the
 *            fp32 values the selection used.
 *   topk_ids [T, k] int32 out: the k largest keys per token, slots by key descending,
 *            ties to the lower expert index.
 *   topk_gates [T, k] fp32 out: softmax over all E of the logits, or sigmoid of the
 *            logit, taken at the selected experts; divided by their sum if norm_topk != 0.
 *   workspace device scratch of at least moe_route_workspace_size(T, H, E, logits != NULL)
 *            bytes: the router weight split into bf16 parts, the logits when the caller does
 *            not ask for them, and the partial products of the projection when it is cut
 *            over H or K (few experts and few tokens; many experts and few output tiles).
 *            The size is a function of (T, H, E, logits_given) only.
 * H must be a multiple of 8.
 * ------------------------------------------------------------------------------------- */
size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E, int32_t logits_given);
moe_status moe_route(const void* x, moe_dtype x_dt, const float* w_router, const float* bias,
                     int64_t T, int32_t H, int32_t E, int32_t k, moe_score score, int32_t norm_topk,
                     float* logits, int32_t* topk_ids, float* topk_gates, void* workspace,
                     size_t workspace_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Dispatch (summary page, "Method", first paragraph: tokens permuted so same-expert
 * tokens are contiguous, as the grouped GEMM requires).
 *   topk_ids       [T, k] int32, each in [0, E) and distinct within a token.  Not checked on
 *                  the host (device data); the kernels take an id outside [0, E) as expert 0 and
 *                  stay in bounds either way, but the outputs are then meaningless.
 *   expert_counts  [E] int32 out, or NULL: rows per expert (sum = T*k)
 *   expert_offsets [E+1] int32 out: exclusive prefix sum of the counts
 *   row_map        [T, k] int32 out: permuted row of (t, j)
 *   src_token      [T*k] int32 out: token of permuted row p (inverse of row_map)
 *   x_perm         [T*k, H] out: x_perm[row_map[t, j]] = x[t].  perm_dt = x_dt copies the
 *                  bits; perm_dt = MOE_FP8_E4M3 (x_dt = MOE_BF16, H % 128 == 0) quantises
 *                  each row in 1x128 blocks: scale = the smallest power of two 2^q with
 *                  448 * 2^q >= amax, q in [-127, 127] (1 for an all-zero block),
 *                  code = e4m3_rne(clamp(x / scale, +-448)); scales go to
 *   x_perm_scales  [T*k, H/128] fp32 out (FP8 only, else ignored).  perm_dt = MOE_MXFP4 (x_dt =
 *                  MOE_BF16, H % 32 == 0) quantises each row in 1x32 blocks: scale = the smallest
 *                  power of two 2^q with 6 * 2^q >= amax, q in [-127, 127] (2^0 for an all-zero
 *                  block), element = the nearest E2M1 value of x / scale (ties to the even-mantissa
 *                  code); x_perm [T*k, H/2] bytes, x_perm_scales [T*k, H/32] E8M0 bytes.
 *   x_perm may be NULL to build only the maps.
 *   workspace      device scratch of at least moe_permute_workspace_size(T, E, k) bytes.
 * ------------------------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k);
moe_status moe_permute(const void* x, moe_dtype x_dt, const int32_t* topk_ids, int64_t T, int32_t H,
                       int32_t E, int32_t k, void* x_perm, moe_dtype perm_dt, void* x_perm_scales,
                       int32_t* row_map, int32_t* src_token, int32_t* expert_counts,
                       int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                       moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Compute (summary page, "Method", first paragraph: all local experts in one grouped GEMM;
 * SwiGLU experts): for every expert e and every row p in [offsets[e], offsets[e+1]):
 *     u = x_perm[p] . W1[e]          W1 [E, H, 2F]   (columns [0,F) gate, [F,2F) up)
 *     h = SiLU(u[:F]) * u[F:]        SiLU(z) = z / (1 + exp(-z))
 *     y_perm[p] = h . W2[e]          W2 [E, F, H]
 * Per-expert row counts are read from expert_offsets in DEVICE memory only; `rows` is the
 * host-known bound T*k used to size the launch (offsets non-decreasing from 0 with
 * offsets[E] <= rows is required; offsets breaking this are clamped into [0, rows], which keeps
 * every access in bounds but makes the results meaningless).
 *   dt = MOE_F32:  x_perm, w1, w2 fp32; h fp32; y_perm fp32 (out_dt MOE_F32).
 *   dt = MOE_BF16: x_perm, w1, w2 bf16; h rounded to bf16; y_perm bf16 or fp32.
 *   dt = MOE_FP8_E4M3: x_perm e4m3 with x_perm_scales [rows, H/128]; w1/w2 e4m3 with
 *        w1_scales [E, H/128, 2F/128], w2_scales [E, F/128, H/128] (128x128 blocks); h is
 *        quantised to e4m3 in 1x128 blocks inside the path; y_perm bf16 or fp32.  Scales are
 *        any positive finite fp32 values; when all of them are powers of two (as the ones
 *        moe_permute writes) the scaled MFMA applies them exactly as exponents, otherwise a
 *        slower path multiplies them in fp32 (chosen on the device, no host sync).
 *   dt = MOE_MXFP4: both operands of both GEMMs 4-bit, every matrix stored contraction-contiguous
 *        with one E8M0 byte per 32 elements: x_perm [rows, H/2] + x_perm_scales [rows, H/32];
 *        W1[e] (the logical [H, 2F] above) as w1 [E, 2F, H/2] + w1_scales [E, 2F, H/32]; W2[e]
 *        (logical [F, H]) as w2 [E, H, F/2] + w2_scales [E, H, F/32]; h is re-quantised to MXFP4
 *        in 1x32 blocks inside the path (the moe_permute rule); y_perm bf16 or fp32.
 * Sizes: bf16: H a multiple of 64 and F of 128; e4m3: both multiples of 128; MXFP4: both of 256;
 * fp32: both of 32.
 * workspace: at least moe_grouped_swiglu_workspace_size(rows, F, dt) bytes (holds h).
 * Rows beyond offsets[E] are not written.
 * ------------------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_workspace_size(int64_t rows, int32_t F, moe_dtype dt);
moe_status moe_grouped_swiglu(const void* x_perm, const void* x_perm_scales, moe_dtype dt,
                              const int32_t* expert_offsets, int64_t rows, int32_t E, int32_t H,
                              int32_t F, const void* w1, const void* w1_scales, const void* w2,
                              const void* w2_scales, void* y_perm, moe_dtype out_dt,
                              void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Combine (summary page, "Method", first paragraph):
 *     y[t] = sum_{j<k} topk_gates[t, j] * y_perm[row_map[t, j]]  (+ shared_out[t], gate 1)
 * accumulated in fp32 over j ascending and rounded once to out_dt.
 *   y_perm [T*k, H] y_dt (MOE_F32 | MOE_BF16); shared_out [T, H] y_dt or NULL;
 *   y [T, H] out_dt (MOE_F32 | MOE_BF16).
 *   row_map entries must lie in [0, T*k); an entry outside is read as row 0 (in bounds, but
 *   the result is then meaningless).
 * ------------------------------------------------------------------------------------- */
moe_status moe_unpermute_combine(const void* y_perm, moe_dtype y_dt, const int32_t* row_map,
                                 const float* topk_gates, const void* shared_out, int64_t T,
                                 int32_t H, int32_t k, void* y, moe_dtype out_dt, moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * The whole layer in one call: route -> permute -> grouped SwiGLU -> (shared expert) ->
 * combine, launched in that order on `stream` (summary page, "Method", first paragraph, the
 * four stages; second paragraph, sync-free dropless execution).
 * ------------------------------------------------------------------------------------- */
typedef struct {
  int32_t H, E, k, F;
  int32_t Fs;           /* shared expert hidden size, 0 = no shared expert                */
  moe_dtype x_dt;       /* activations x and y: MOE_F32 or MOE_BF16                      */
  moe_dtype w_dt;       /* expert weights: MOE_F32 (x_dt F32), MOE_BF16, MOE_FP8_E4M3,   */
                        /* MOE_MXFP4 (stored as in moe_grouped_swiglu; shared: ws1       */
                        /* [2Fs, H/2] + [2Fs, H/32], ws2 [H, Fs/2] + [H, Fs/32])          */
  moe_dtype out_dt;     /* y: MOE_F32 or MOE_BF16                                        */
  moe_score score;
  int32_t norm_topk;
  const float* w_router; /* [H, E] fp32                                                  */
  const float* bias;     /* [E] selection bias or NULL                                   */
  const void* w1;        /* [E, H, 2F]                                                   */
  const void* w2;        /* [E, F, H]                                                    */
  const void* ws1;       /* [H, 2Fs] or NULL                                             */
  const void* ws2;       /* [Fs, H] or NULL                                              */
  const void* w1_scales, *w2_scales, *ws1_scales, *ws2_scales;  /* FP8: fp32; MXFP4: E8M0 */
                                                                 /* bytes; else NULL       */
  int32_t gate_in_expert; /* 0: combine weights the expert rows by their gates.  1: the gate  */
                          /* is folded into the experts: the first GEMM's SwiGLU epilogue     */
                          /* multiplies each permuted row's h by its gate before rounding, so */
                          /* y_perm rows come out gate-weighted and combine sums the k rows   */
                          /* unweighted (summary page, "Method", second paragraph: memory-    */
                          /* efficient permutation, kernel fusion).  The shared expert keeps  */
                          /* gate 1 either way; moe_backward does not depend on it.           */
} moe_layer;

/* Optional views of the intermediates: every non-NULL pointer receives that stage's
 * output (shapes as in the stage calls; x_perm / y_perm in the dtypes moe_forward uses:
 * x_perm in w_dt (e4m3 codes for FP8, with x_perm_scales, which is then required), y_perm in
 * x_dt; with gate_in_expert, y_perm rows are the gate-weighted ones the experts wrote).  moe_forward itself does not materialise x_perm: its first grouped GEMM reads the
 * token rows of x (for FP8: of x quantised once per token) through src_token; x_perm is
 * written only when requested here.  All pointers 16-byte aligned.
 * stage_events: optional hipEvent_t handles recorded on `stream` at the stage boundaries
 * (0 before route, 1 after route, 2 after permute, 3 after the first grouped GEMM,
 * 4 after the second, 5 after the shared expert, 6 after combine); NULL entries are skipped. */
#define MOE_NUM_STAGE_EVENTS 7
typedef struct {
  float* logits;
  int32_t* topk_ids;
  float* topk_gates;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* row_map;
  int32_t* src_token;
  void* x_perm;
  void* x_perm_scales;
  void* y_perm;
  void* stage_events[MOE_NUM_STAGE_EVENTS];
} moe_debug;

size_t moe_workspace_size(const moe_layer* L, int64_t T);
moe_status moe_forward(const moe_layer* L, const void* x, int64_t T, void* y, const moe_debug* dbg,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Backward of the whole layer.  The pages measure this layer in training ("Scalable Training
 * of Mixture-of-Experts Models with Megatron Core": abstract; summary page, "Method", second
 * paragraph: fine-grained activation recomputation).  Given dy = dL/dy for one moe_forward
 * call, it writes the gradients of L with respect to x and every weight, by the chain rule
 * through the forward's stages:
 *   combine  dL/dg_tj = <dy_t, y_perm[row_map(t, j)]>; each expert row receives g_tj dy_t
 *   experts  u = x_perm W1[e] (recomputed: the forward keeps no activations), a | b = u,
 *            h = SiLU(a) b; dh = dyp W2[e]^T, dW2[e] = h^T dyp,
 *            du = [dh b SiLU'(a) | dh SiLU(a)], dx_perm = du W1[e]^T, dW1[e] = x_perm^T du
 *   dispatch dx_t = sum_j dx_perm[row_map(t, j)]
 *   route    dL/dlogits through softmax (over all E) or sigmoid, and the renormalisation
 *            when norm_topk; top-k selection and the selection bias pass no gradient;
 *            dx += dlogits W_r^T, dW_r = x^T dlogits
 *   shared   the expert rule on all T rows with gate 1
 *   L        the layer as given to moe_forward; w_dt = x_dt = MOE_F32 or MOE_BF16
 *            (MOE_FP8_E4M3 and MOE_MXFP4 return MOE_ERR_UNSUPPORTED).  out_dt is not used.
 *   x        [T, H] x_dt, the forward's input
 *   dy       [T, H] x_dt
 *   r        the forward's routing, as written through moe_debug: logits [T, E] fp32,
 *            topk_ids [T, k], topk_gates [T, k] fp32, expert_offsets [E+1], row_map [T, k],
 *            src_token [T*k].  src_token entries must lie in [0, T), as moe_forward writes
 *            them (the recomputation of u gathers x rows through them unchecked); the other
 *            index entries are clamped into range on the device.
 *   g        outputs, all written in full: dx [T, H] x_dt; dw_router [H, E], dw1 [E, H, 2F],
 *            dw2 [E, F, H], dws1 [H, 2Fs], dws2 [Fs, H] fp32 (the shared pair only when
 *            Fs > 0, else ignored).  An expert that received no rows gets zero gradients.
 *   stage_events NULL or MOE_NUM_BWD_STAGE_EVENTS hipEvent_t handles (NULL entries skipped),
 *            recorded on `stream`: 0 at the start; after the routed experts' recomputed u (1),
 *            dh (2), SwiGLU backward (3), dW2 (4), dx_perm (5) and dW1 (6); after the shared
 *            expert (7); at the end (8).
 *   workspace at least moe_backward_workspace_size(L, T) bytes: u [T*k, 2F] and
 *            dy W2^T [T*k, F] fp32, du [T*k + 64, 2F], g h [T*k, F] and dx_perm [T*k, H] in
 *            x_dt, dg [T*k], dlogits [T, E], dlogits W_r^T [T, H] fp32, and the shared
 *            expert's counterparts, and with many tokens per router-gradient tile up to 32
 *            row slices of partial router-weight gradients [slices, H, E] fp32; for bf16
 *            also the weight gradients' operands: one activation transposed per expert with
 *            each expert's rows padded to a multiple of 64 ([max(H, F, Fs), T*k + 64 E] bf16),
 *            dy in expert-row order ([T*k + 64, H] bf16) and two small index tables.  For bf16
 *            with E a multiple of 32 and H of 64 the router's two products run as bf16 products
 *            of split operands, as accurate as fp32 (dlogits and W_r each as three bf16 parts,
 *            each the rounding of what the parts before it leave): in place of the fp32 row
 *            slices, dlogits' parts [T, 6E] and [T + 64, 3E], W_r's parts [H, 6E] (bf16), and
 *            up to 6 row slices of partial products [slices, H, 3E] fp32 with their offsets.
 * Accumulation is fp32 throughout (fp32 MFMA for fp32 operands, bf16 MFMA with fp32 accumulate
 * for bf16 ones); du and g h are rounded to x_dt before their GEMMs, and the per-row input
 * gradients dx_perm (and the shared expert's) to x_dt before dx sums them in fp32, as the forward
 * rounds y_perm before combine.  Sizes as for moe_forward.
 * ------------------------------------------------------------------------------------- */
#define MOE_NUM_BWD_STAGE_EVENTS 9
typedef struct {
  const float* logits;
  const int32_t* topk_ids;
  const float* topk_gates;
  const int32_t* expert_offsets;
  const int32_t* row_map;
  const int32_t* src_token;
} moe_routing;

typedef struct {
  void* dx;
  float* dw_router;
  float* dw1;
  float* dw2;
  float* dws1;
  float* dws2;
} moe_grads;

size_t moe_backward_workspace_size(const moe_layer* L, int64_t T);
moe_status moe_backward(const moe_layer* L, const void* x, const void* dy, int64_t T, const moe_routing* r,
                        const moe_grads* g, void* const* stage_events, void* workspace, size_t workspace_bytes,
                        moe_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * The fused forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, stages and results as moe_forward (same kernels, so bit-identical outputs for
 * the same inputs); the caller still owns x, y and every moe_debug buffer.  The workspace is a
 * static device array of MOE_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; nothing is allocated or freed by any call.
 *   Limit: a call needing more than MOE_STATIC_SCRATCH_BYTES of workspace, i.e.
 *   moe_workspace_size(L, T) > MOE_STATIC_SCRATCH_BYTES, returns MOE_ERR_TOO_LARGE, launching
 *   nothing.  Decode-sized batches fit: up to 292 tokens of a DeepSeek-V3-shaped bf16 layer
 *   (H 7168, 256 experts, top-8, F 2048, shared expert), 620 of a Qwen3-235B-shaped one, 900 of a
 *   Mixtral-8x7B-shaped one.
 *   Sharing: every call on one GPU uses that GPU's one array, and no kernel relies on its previous
 *   contents; calls that overlap in time on one GPU (different streams or threads without
 *   ordering between them) race on it and must not be issued.
 *   The first call on each device looks up the array's device address (hipGetSymbolAddress) and
 *   keeps it; make that first call outside a graph capture.
 * ------------------------------------------------------------------------------------- */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_static(const moe_layer* L, const void* x, int64_t T, void* y, const moe_debug* dbg,
                              moe_stream_t stream);

const char* moe_status_str(moe_status s);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
