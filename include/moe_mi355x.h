/*
 * moe_mi355x.h -- C ABI of the Stable LatentMoE forward layer for MI355X (gfx950).
 *
 * The layer (sources by page title and section):
 *   - sigmoid router on the full-width token; a per-expert bias picks the
 *     top-k experts, the mixture weights are the chosen raw scores
 *     renormalised, the bias acts on selection only
 *     ("Kimi K3 模型结构（5）：宽度维度，Stable LatentMoE", Q&A on routing);
 *   - Quantile Balancing: per-expert bias from the (1-k/n) quantile of the
 *     expert's margin minus a common offset, exact target load per expert
 *     (same page, Q&A on Quantile Balancing; 延伸解读 "Quantile Balancing与
 *     DeepSeek-V3路由的异同": coordinate descent on the dual of the balanced
 *     assignment problem);
 *   - shared latent down-projection d -> d/2, routed GLU experts with
 *     SiTU-GLU h = SiLU(4 tanh(g/4)) * 25 tanh(u/25), weighted sum, RMSNorm,
 *     up-projection, plus the merged shared-expert MLP at full width
 *     ("Kimi K3 — LatentMoE" (dimsnsums.com), section "Why does the router
 *     need three moves?"; xhh.club page, Q&A on SiTU-GLU, RMSNorm and the
 *     shared expert);
 *   - routed-expert weights in MXFP4 for deployment (xhh.club page,
 *     延伸解读 "参数规模与部署要点").
 *
 * Conventions for every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller unless
 *     stated otherwise.  The library never frees or retains caller memory.
 *     State kept between calls: loaded code objects; per device, one
 *     auxiliary non-blocking stream (default priority) with two events,
 *     created on first use, on which moe_latent_forward runs the
 *     routing-independent shared branch (forked from and joined back into
 *     `stream`, under a per-device mutex held for the call); per device, the
 *     compute-unit count and wall-clock rate that size the routing loop's
 *     grid and its wait limit; the opt-in stage-timing records.
 *   - Matrices are row-major [out_features][in_features] (K contiguous);
 *     activations are [T][features].  bf16 values are passed as raw 16-bit
 *     patterns.  MXFP4 weights: codes uint8 [rows][K/2] (element 2i in the
 *     low nibble of byte i, 2i+1 in the high nibble, bit 3 = sign, E2M1
 *     magnitudes 0,.5,1,1.5,2,3,4,6) and one E8M0 scale byte per 32
 *     consecutive K elements, uint8 [rows][K/32] (value * 2^(byte-127)).
 *     Every byte 0..254 is decoded exactly; a product above the bf16 range
 *     (bytes 253 and 254 with large codes) becomes an infinity, and byte 255
 *     (NaN in the format) gives NaN.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Work is enqueued on it and no call waits on the host.  Routing (every
 *     mode) runs as one persistent launch of at most one block per compute
 *     unit whose blocks wait for each other through device-memory
 *     barriers; work on other streams may delay it but must not depend on
 *     it.  A barrier wait longer than 2 s ends the loop with qb_info status
 *     3 (aborted) and leaves the routing outputs undefined.
 *   - Return value: MOE_OK or a negative moe_status for invalid arguments,
 *     unsupported combinations, a too-small workspace or a HIP error.  Nothing
 *     is launched when validation fails.  The outcome of balancing (rounds,
 *     balanced or not) is reported through `qb_info`, not the return value.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad shape, NULL where a buffer is required, k > n, ... */
  MOE_EUNSUPPORTED = -2,  /* valid but not implemented (dtype combination, n > 1024) */
  MOE_EWORKSPACE = -3,    /* workspace smaller than the *_workspace_bytes query */
  MOE_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_MXFP4 = 2,    /* routed weights: E2M1 codes + E8M0 scales per 32 (bf16 activations) */
  MOE_MXFP4_A8 = 3, /* routed weights as MOE_MXFP4; the routed experts' inputs z and h are
                       quantised on the fly from bf16 to MXFP8 (E4M3 + E8M0 per 32) and
                       multiplied with gfx950's scaled MFMA (W4A8).  latent and inter must be
                       multiples of 128 (else MOE_EUNSUPPORTED) */
  MOE_MXFP4_A4 = 4  /* as MOE_MXFP4_A8 with z and h quantised to MXFP4 (E2M1 + E8M0 per 32,
                       shared exponent floor(log2 amax) - 2): W4A4 on the scaled MFMA with
                       E2M1 on both operands; same size limits */
} moe_dtype;

typedef enum {
  MOE_QB_FROZEN = 0,  /* use the given bias as is (inference: bias frozen) */
  MOE_QB_BATCH = 1    /* Quantile Balancing on this batch, bias in/out */
} moe_qb_mode;

/* qb_info[4] (int32, device): rounds of quantile coordinate updates, status
 * (0 balanced / frozen, 1 not balanced within the limits, 2 bias left the
 * representable range), max |load - target| at exit, augmenting-path moves.
 * Status 1 means that no bias balances the batch (equal scores on both sides
 * of a target, e.g. duplicated tokens), or that the step cap was reached.
 * That includes score rows so flat that more than 64 of one token's experts
 * sit within the needed path length of its threshold, where the sparse edge
 * list cannot hold the token's candidates.  The routing outputs are still
 * the top-k under the returned bias. */
enum {
  MOE_QB_STATUS_OK = 0,
  MOE_QB_STATUS_NOT_BALANCED = 1,
  MOE_QB_STATUS_BIAS_RANGE = 2,
  MOE_QB_STATUS_ABORTED = 3 /* a grid-barrier wait timed out: outputs undefined */
};

/* Largest batch any entry point takes (2^20 tokens; larger T returns
 * MOE_EUNSUPPORTED).  Far above what one GPU's memory holds for the K3 layer,
 * and small enough that every slot, tile and edge count of the kernels fits in
 * 32 bits. */
#define MOE_MAX_TOKENS (1 << 20)

typedef struct {
  int32_t T;             /* tokens in the batch, 0..MOE_MAX_TOKENS */
  int32_t d;             /* model width (7168 for K3), multiple of 64 */
  int32_t latent;        /* latent width (d/2 = 3584 for K3), multiple of 64 */
  int32_t n_experts;     /* routed experts (896), 1..1024 */
  int32_t top_k;         /* experts per token (16), 1..n_experts */
  int32_t inter;         /* routed intermediate width m, multiple of 64 */
  int32_t shared_inter;  /* merged shared-expert intermediate (2 x 3072), multiple of 64 */
  int32_t act_dtype;     /* MOE_F32 or MOE_BF16: x, out and the dense weights */
  int32_t routed_dtype;  /* act_dtype, or MOE_MXFP4 / _A8 / _A4 with MOE_BF16 activations */
  float rms_eps;         /* RMSNorm epsilon (1e-6) */
  int32_t qb_mode;       /* moe_qb_mode */
  int32_t qb_max_rounds; /* cap on quantile coordinate rounds (<= 0: 64) */
} moe_shape_t;

typedef struct {
  const float* w_router;            /* [n][d] f32 */
  const float* router_logit_offset; /* [n] f32 added to the logits, or NULL */
  const void* w_down;               /* [latent][d]  act dtype: latent down-projection */
  const void* w_up;                 /* [d][latent]  act dtype: latent up-projection */
  const void* w_gate;               /* [n][inter][latent] routed gate (codes if MXFP4) */
  const void* w_uproj;              /* [n][inter][latent] routed up   (codes if MXFP4) */
  const void* w_dn;                 /* [n][latent][inter] routed down (codes if MXFP4) */
  const uint8_t* s_gate;            /* MXFP4 scales [n][inter][latent/32], else NULL */
  const uint8_t* s_uproj;           /* MXFP4 scales [n][inter][latent/32], else NULL */
  const uint8_t* s_dn;              /* MXFP4 scales [n][latent][inter/32], else NULL */
  const float* rms_gamma;           /* [latent] f32 RMSNorm gain */
  const void* ws_gate;              /* [shared_inter][d] act dtype */
  const void* ws_up;                /* [shared_inter][d] act dtype */
  const void* ws_down;              /* [d][shared_inter] act dtype */
} moe_weights_t;

/* Bytes of device workspace moe_route_qb needs for (T, n, k); 0 on bad input. */
size_t moe_route_workspace_bytes(int32_t T, int32_t n, int32_t k);

/*
 * moe_route_qb -- routing of T tokens given their sigmoid scores.
 *   scores   [T][n] f32 in [0, 1] (read only)
 *   mode     moe_qb_mode; max_rounds caps the quantile rounds (<= 0: 64)
 *   bias     [n] f64, in: starting (BATCH) or frozen (FROZEN) bias; out (BATCH):
 *            the balancing bias, exact multiples of 2^-40, common offset removed
 *            (sum in [0, n) * 2^-40).  |bias| must stay below 1024.
 *   topk_idx [T][k] i32: chosen experts by descending raw score, ties to the
 *            lower expert index
 *   topk_w   [T][k] f32: chosen raw scores divided by their sum
 *   loads    [n] i32: tokens per expert; qb_info [4] i32 as described above
 *   workspace/workspace_bytes: device scratch of at least
 *            moe_route_workspace_bytes(T, n, k) bytes, 256-byte aligned
 * Scores and biases are compared exactly on a 2^-40 fixed-point grid; with
 * QB the chosen sets are the unique balanced optimum, independent of how the
 * bias was reached.
 */
int moe_route_qb(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
                 int32_t max_rounds, double* bias, int32_t* topk_idx, float* topk_w,
                 int32_t* loads, int32_t* qb_info, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * moe_route_qb_noalloc -- moe_route_qb for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same arguments and results without
 * workspace/workspace_bytes.  The scratch is a device array of
 * MOE_ROUTE_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call allocates nothing.  Batches whose
 * moe_route_workspace_bytes(T, n, k) exceeds that size are rejected with
 * MOE_EWORKSPACE (at n = 896, k = 16: up to about 6600 tokens).  All calls on
 * one GPU share its array: calls that overlap on one GPU (concurrent
 * streams, threads) race and give undefined results.
 */
#define MOE_ROUTE_SCRATCH_BYTES (32u << 20)
int moe_route_qb_noalloc(const float* scores, int32_t T, int32_t n, int32_t k, int32_t mode,
                         int32_t max_rounds, double* bias, int32_t* topk_idx, float* topk_w,
                         int32_t* loads, int32_t* qb_info, void* stream);

/*
 * moe_route_sign -- the fixed-step sign update of the routing bias
 * (DeepSeek-V3's rule), run on one batch as the baseline Quantile Balancing
 * is compared with: sign descent on the same dual objective with a
 * hand-tuned step (xhh.club page above, 延伸解读 "Quantile Balancing与
 * DeepSeek-V3路由的异同").  Each round takes the top-k of the biased keys
 * (exactly as moe_route_qb) and then moves every expert's bias by
 * step * sign(C_e - L_e); the loop stops at exact balance or after
 * max_rounds updates.
 *   scores, topk_idx, topk_w, loads, workspace: as for moe_route_qb
 *   step     bias step in score units, > 0; used as rint(step * 2^40) grid
 *            units (at least one unit, below 2^50)
 *   max_rounds  updates at most (>= 0; 0 = plain top-k under the given bias)
 *   bias     [n] f64 in: the start; out: the bias after the last update
 *            (no common offset removed)
 *   qb_info  [4] i32: updates made, status (0 balanced, 1 not balanced after
 *            max_rounds, 2 bias left the representable range), max
 *            |load - target| at exit, 0
 */
int moe_route_sign(const float* scores, int32_t T, int32_t n, int32_t k, double step,
                   int32_t max_rounds, double* bias, int32_t* topk_idx, float* topk_w,
                   int32_t* loads, int32_t* qb_info, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Bytes of device workspace moe_latent_forward needs for this shape; 0 on bad input. */
size_t moe_forward_workspace_bytes(const moe_shape_t* shape);

/*
 * moe_latent_forward -- one forward pass of the layer.
 *   shape, weights : host pointers to the structs above (read during the call)
 *   x   [T][d] act dtype (read only); out [T][d] act dtype
 *   bias [n] f64 in/out exactly as for moe_route_qb
 *   scores_in  [T][n] f32 or NULL: when given, these scores replace the router
 *              (e.g. scores computed elsewhere); when NULL the router runs
 *   scores_out [T][n] f32 or NULL: receives the scores used for routing
 *   topk_idx, topk_w, loads, qb_info: as for moe_route_qb; each may be NULL
 *   workspace : >= moe_forward_workspace_bytes(shape) bytes, 256-byte aligned
 */
int moe_latent_forward(const moe_shape_t* shape, const moe_weights_t* weights, const void* x,
                       void* out, double* bias, const float* scores_in, float* scores_out,
                       int32_t* topk_idx, float* topk_w, int32_t* loads, int32_t* qb_info,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_mxfp8_quantize -- the on-the-fly MXFP8 rounding of the routed experts'
 * inputs in MOE_MXFP4_A8 (deployment of the routed experts in microscaling
 * formats: xhh.club page, 延伸解读 "参数规模与部署要点"; element and scale
 * formats of the OCP Microscaling v1.0 specification).
 *   x      [rows][K] bf16 (raw 16-bit patterns), 16-byte aligned, read only
 *   codes  [rows][K] u8 E4M3 codes (sign bit 7, 4-bit exponent with bias 7,
 *          3-bit mantissa), 8-byte aligned
 *   scales [rows][K/32] u8 E8M0 (value 2^(byte-127))
 *   K      a multiple of 32; rows >= 0 (0: nothing is launched)
 * Per block of 32 consecutive elements of a row: X = floor(log2 amax) - 8,
 * scale byte X + 127 clamped to [0, 254] (0 for an all-zero block); each
 * element v / 2^(byte-127) rounded to the nearest E4M3 value, ties to the
 * even mantissa, magnitudes beyond 448 saturating to 448.  Enqueued on
 * `stream`; returns MOE_EINVAL for bad sizes, NULL or misaligned pointers.
 */
int moe_mxfp8_quantize(const void* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                       void* stream);

/*
 * moe_mxfp4_quantize -- the on-the-fly MXFP4 rounding of the routed experts'
 * inputs in MOE_MXFP4_A4 (the same deployment passage and OCP format as the
 * routed weights).
 *   x      [rows][K] bf16 (raw 16-bit patterns), 16-byte aligned, read only
 *   codes  [rows][K/2] u8 E2M1 codes, element 2i in the low nibble of byte i
 *          (sign bit 3, magnitudes 0,.5,1,1.5,2,3,4,6), 4-byte aligned
 *   scales [rows][K/32] u8 E8M0 (value 2^(byte-127))
 *   K      a multiple of 32; rows >= 0 (0: nothing is launched)
 * Per block of 32 consecutive elements of a row: X = floor(log2 amax) - 2,
 * scale byte X + 127 clamped to [0, 254] (0 for an all-zero block); each
 * element v / 2^(byte-127) rounded to the nearest E2M1 value, ties to the
 * even code, magnitudes beyond 6 saturating to 6.  Enqueued on `stream`;
 * returns MOE_EINVAL for bad sizes, NULL or misaligned pointers.
 */
int moe_mxfp4_quantize(const void* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                       void* stream);

/* Gradients written by moe_latent_backward (DEVICE pointers, caller-owned).
 * Weight gradients are fp32 in the layout of the weights; dx has the
 * activation dtype.  d_router_logit_offset must be NULL exactly when the
 * weights have no router_logit_offset. */
typedef struct {
  void* dx;                     /* [T][d] */
  float* d_w_router;            /* [n][d] */
  float* d_router_logit_offset; /* [n] or NULL */
  float* d_w_down;              /* [latent][d] */
  float* d_w_up;                /* [d][latent] */
  float* d_w_gate;              /* [n][inter][latent] */
  float* d_w_uproj;             /* [n][inter][latent] */
  float* d_w_dn;                /* [n][latent][inter] */
  float* d_rms_gamma;           /* [latent] */
  float* d_ws_gate;             /* [shared_inter][d] */
  float* d_ws_up;               /* [shared_inter][d] */
  float* d_ws_down;             /* [d][shared_inter] */
} moe_grads_t;

/* Bytes of device workspace moe_latent_backward needs; 0 on a shape it does
 * not take (bf16 activations and bf16 routed weights only). */
size_t moe_backward_workspace_bytes(const moe_shape_t* shape);

/*
 * moe_latent_backward -- gradients of sum(out * dout) for one forward call,
 * the expert selection held fixed: the QB bias acts on selection only, so
 * gradients reach the router through the renormalised raw scores of the
 * chosen experts, and every step after routing is differentiated as written
 * (xhh.club page above, Q&A on routing, SiTU-GLU, RMSNorm and the shared
 * expert).
 *   shape, weights : as for the forward call (act_dtype and routed_dtype
 *                    MOE_BF16, else MOE_EUNSUPPORTED; qb_mode is ignored)
 *   x        [T][d] bf16, the forward's input
 *   scores   [T][n] f32, the forward's router scores (its scores_out)
 *   topk_idx [T][k] i32 and topk_w [T][k] f32, the forward's routing
 *   dout     [T][d] bf16, the gradient of the output
 *   grads    host pointer to the gradient buffers (overwritten, not
 *            accumulated)
 *   workspace: >= moe_backward_workspace_bytes(shape) bytes, 256-byte aligned
 * The forward activations are recomputed from x and the routing.  Products
 * run on the bf16 MFMA with fp32 accumulation; intermediate gradients that
 * feed a product are rounded to bf16.  Results are deterministic (fixed
 * reduction orders, no floating-point atomics).  Enqueued on `stream`.
 */
int moe_latent_backward(const moe_shape_t* shape, const moe_weights_t* weights, const void* x,
                        const float* scores, const int32_t* topk_idx, const float* topk_w,
                        const void* dout, const moe_grads_t* grads, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * moe_sgd_step -- one plain gradient-descent step on every weight of the
 * layer, in place: w <- w - lr * g, the optimizer step that completes a
 * training step after moe_latent_backward (the pages place QB in training,
 * where the bias is set again for every batch: dimsnsums.com "Kimi K3 --
 * LatentMoE", Quantile Balancing paragraph; they name no optimizer for the
 * layer's weights, and the plainest one is taken).
 *   shape   : as for moe_latent_backward (bf16 layers only)
 *   weights : the layer's weights; the buffers it points to are updated in
 *             place (router, its offset when present, latent down and up,
 *             routed gate, up and down, RMSNorm gain, shared gate, up, down)
 *   grads   : their gradients (moe_latent_backward's output)
 *   lr      : step size, finite
 * Every element is computed as fp32 operations, each rounded to nearest
 * even: t = lr * g, then w - t, then the weight's own type (fp32 for the
 * router, its offset and the gain; bf16, round to nearest even, for the
 * rest).  No contraction into a fused multiply-add, so results are exactly
 * defined.  Enqueued on `stream`; NULL required buffers return MOE_EINVAL.
 */
int moe_sgd_step(const moe_shape_t* shape, const moe_weights_t* weights, const moe_grads_t* grads,
                 float lr, void* stream);

/*
 * moe_latent_backward_sgd -- moe_latent_backward followed by moe_sgd_step,
 * with the same results bit for bit, but the routed experts' weight
 * gradients (the three largest tensors, fp32 [n][inter][latent] and
 * [n][latent][inter]) are never stored: each is applied to its weight inside
 * the kernel that forms it, after every read of that weight.  Arguments as
 * for moe_latent_backward plus lr (finite); grads->d_w_gate, d_w_uproj and
 * d_w_dn are not used (may be NULL), every other gradient is written and
 * applied.  Every weight buffer is updated in place.  T = 0: the gradients
 * are left as they are and no weight moves.
 */
int moe_latent_backward_sgd(const moe_shape_t* shape, const moe_weights_t* weights, const void* x,
                            const float* scores, const int32_t* topk_idx, const float* topk_w,
                            const void* dout, const moe_grads_t* grads, float lr, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Training forward and backward: the forward keeps the activations the
 * backward would otherwise recompute (bf16 layers).
 *
 * moe_saved_activations_bytes -- size of the buffer they need (at least 256
 * bytes); 0 on a shape the training calls do not take.  The buffer holds z [T][latent] bf16, the
 * routed experts' gate and up pre-activations [T*k][inter] fp32 and h bf16,
 * their outputs [T*k][latent] fp32, and the shared expert's pre-activations
 * [T][shared_inter] fp32 and hs bf16, slots in the forward's permutation
 * order.  Its content is private to these calls.
 *
 * moe_latent_forward_train -- moe_latent_forward (same arguments, same
 * results bit for bit) that also fills `saved` (>= the size above, 256-byte
 * aligned, caller-owned).
 *
 * moe_latent_backward_train -- moe_latent_backward (apply_sgd = 0) or
 * moe_latent_backward_sgd (apply_sgd = 1, step size lr) for that forward
 * call: x, scores, topk_idx, topk_w as it returned them, `saved` as it
 * filled it (read only).  Workspace as for moe_latent_backward.  The
 * results match those of the recomputing calls to within the rounding of
 * the activations: the forward may split a small product's K range where
 * the recompute does not, which can move a stored bf16 activation by one
 * unit.
 */
size_t moe_saved_activations_bytes(const moe_shape_t* shape);

int moe_latent_forward_train(const moe_shape_t* shape, const moe_weights_t* weights, const void* x,
                             void* out, double* bias, const float* scores_in, float* scores_out,
                             int32_t* topk_idx, float* topk_w, int32_t* loads, int32_t* qb_info,
                             void* saved, size_t saved_bytes, void* workspace,
                             size_t workspace_bytes, void* stream);

int moe_latent_backward_train(const moe_shape_t* shape, const moe_weights_t* weights, const void* x,
                              const float* scores, const int32_t* topk_idx, const float* topk_w,
                              const void* dout, const void* saved, size_t saved_bytes,
                              const moe_grads_t* grads, int apply_sgd, float lr, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Static description of a moe_status value; never NULL. */
const char* moe_status_str(int status);

/*
 * Stage timing (diagnostics; not a part of the layer's arithmetic).
 * moe_stage_timing(1) makes later moe_latent_forward / moe_route_qb calls
 * record a pair of HIP events around each stage on their stream, and clears
 * the totals; moe_stage_timing(0) stops recording.  After the caller has
 * synchronised those streams, moe_stage_times writes the summed milliseconds
 * and the number of timed launches per stage (arrays of max_stages entries,
 * either may be NULL) and returns the number of stages, or MOE_EHIP if an
 * event has not completed.  Stages, in order: router, latent_down,
 * shared_gate_up, routing, permute, routed_gate_up, routed_down,
 * combine_rmsnorm, up_proj_shared_down; moe_stage_name gives these names
 * (static strings, "unknown" out of range).  Host-side state, guarded by a
 * mutex; events are created on first use and reused.
 */
int moe_stage_timing(int enable);
int moe_stage_times(double* total_ms, int32_t* counts, int32_t max_stages);
const char* moe_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
