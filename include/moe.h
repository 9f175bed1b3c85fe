/*
 * moe.h — C ABI of libmoe.so: the forward pass of one Mixture-of-Experts FFN
 * layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer (moe-200m-qwen3-100b README, "Architecture diagram" and
 * "SigmoidRouter"; SpecForge PR #930, "What this adds"):
 *   1. router, always in fp32 (README, "Per-layer numerics"):
 *        logits = x W_r^T; scores = sigmoid(logits) or softmax over all
 *        experts; an optional per-expert bias is added to the scores for
 *        the choice of experts only; top-k by descending value; combine
 *        weights are the unbiased scores of the chosen experts, divided by
 *        their sum (plus 1e-9 for sigmoid) when renormalising;
 *        counts[e] = tokens that chose expert e;
 *   2. dispatch of the (token, slot) pairs into expert-contiguous order;
 *   3. SwiGLU experts on their rows, weights stacked [E, out, in]
 *        (PR #930, "Why FSDP is enough here"): h = silu(x W_gate[e]^T) *
 *        (x W_up[e]^T), out = h W_down[e]^T; the names w1 / w3 / w2 of the
 *        pages' per-expert checkpoint keys are gate / up / down;
 *      plus an optional shared expert that every token uses with weight 1;
 *   4. combine back to token order: y[t] = sum_j w[t,j] out_{e_j}(x_t)
 *        (+ shared(x_t)).
 *
 * Determinism. Expert ids, counts, dispatch order and combine weights are
 * bit-reproducible: the gate product is one fp32 fma chain per (token,
 * expert) over features in ascending order; exp inside the router is a fixed
 * sequence of IEEE operations; ties go to the lower expert id; rows of one
 * expert are ordered by token id. Outputs are bitwise repeatable from call to
 * call (no floating-point atomics anywhere).
 *
 * Conventions for every entry point.
 *   - Pointers to tensors are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or keeps them. Size out-parameters are
 *     host pointers.
 *   - Tensors are row-major and contiguous. bf16 data is stored as 16-bit
 *     bf16 bit patterns; fp32 as IEEE binary32.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream). Calls return after enqueueing; none synchronises the stream,
 *     except moe_timing_read.
 *   - Arguments are validated before anything is enqueued; an invalid call
 *     returns a status other than MOE_OK and leaves every buffer untouched.
 *     MOE_ERR_HIP reports a launch error; faults inside kernels surface at
 *     the caller's next synchronisation.
 *   - Outputs must not alias inputs. Scratch space comes from the caller's
 *     workspace `ws` of `ws_bytes` bytes (256-byte aligned); its contents
 *     after a call are unspecified.
 *   - No exception crosses this interface. Calls on different streams with
 *     different workspaces may run concurrently.
 */
#ifndef MOE_MI355X_MOE_H
#define MOE_MI355X_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* null required pointer, k < 1, k > E, T < 0, inconsistent shared expert, ... */
    MOE_ERR_UNSUPPORTED = 2, /* d_model or d_ff not a multiple of 64, E > 1024, k > 32, unknown dtype/score */
    MOE_ERR_WORKSPACE = 3,   /* ws_bytes below the size the matching *_workspace_size query returns */
    MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status;

/* dtype of x, of the expert weights and of the internal SwiGLU activations.
 * The router weight and the selection bias are fp32 in every case. */
#define MOE_F32 0
#define MOE_BF16 1

/* router score */
#define MOE_SOFTMAX 0 /* softmax over all experts (SpecForge PR #930, qwen3 preset) */
#define MOE_SIGMOID 1 /* sigmoid per expert (README, "SigmoidRouter") */

/* One MoE FFN layer: shapes, recipe and device pointers to its weights.
 * The counterpart of the pages' MoEModelConfig (README, "Config") restricted
 * to the fields of one layer. Stating the shared expert inconsistently (some
 * but not all of its three weights, or a width without weights) is an error,
 * as conflicting statements of the expert count are on the pages
 * (PR #930, "What this adds": num_experts vs n_routed_experts). */
typedef struct moe_layer {
    int32_t d_model;     /* d: features per token; multiple of 64 */
    int32_t d_ff;        /* width of each routed expert; multiple of 64 */
    int32_t n_experts;   /* E: routed experts, 1..1024 */
    int32_t top_k;       /* k: experts per token, 1..min(E, 32) */
    int32_t score;       /* MOE_SOFTMAX or MOE_SIGMOID */
    int32_t renorm;      /* nonzero: combine weights renormalised over the k chosen experts */
    int32_t dtype;       /* MOE_F32 or MOE_BF16 */
    int32_t d_ff_shared; /* width of the shared expert; 0 when there is none; multiple of 64 */
    int32_t bias_on_logits; /* 0: sel_bias is added to the score (PR #930 noaux_tc selection bias);
                               nonzero: to the logit (README, "SigmoidRouter": logits + bias select) */
    const float *w_router; /* [E, d] fp32 (nn.Linear layout) */
    const float *sel_bias; /* [E] fp32 selection bias, or NULL; moves selection only */
    const void *w_gate;    /* [E, d_ff, d]  (w1) */
    const void *w_up;      /* [E, d_ff, d]  (w3) */
    const void *w_down;    /* [E, d, d_ff]  (w2) */
    const void *ws_gate;   /* [d_ff_shared, d] or NULL */
    const void *ws_up;     /* [d_ff_shared, d] or NULL */
    const void *ws_down;   /* [d, d_ff_shared] or NULL */
} moe_layer;

/* Router losses and health metrics (README, "SigmoidRouter": z_loss,
 * aux_loss, router_cv, router_entropy_bits; PR #931, "What to watch":
 * moe/load_max_ratio and the share of experts that receive no token).
 * Indices into the fp64 metrics array of moe_route_opts:
 *   Z_LOSS        mean over tokens of logsumexp(logits)^2
 *   AUX_LOSS      E * sum_e f_e P_e, f_e = counts_e / T, P_e = mean unbiased score of e
 *   CV            unbiased std(counts) / max(mean(counts), 1); 0 when E = 1
 *   ENTROPY_BITS  -sum p log2 p over p = max(P, 1e-9), normalised to sum 1
 *   LOAD_MAX_RATIO max(counts) / mean(counts)
 *   UNUSED_FRAC   share of experts with counts = 0
 * Scores are the sigmoid or the softmax over all experts, never biased. */
#define MOE_METRIC_Z_LOSS 0
#define MOE_METRIC_AUX_LOSS 1
#define MOE_METRIC_CV 2
#define MOE_METRIC_ENTROPY_BITS 3
#define MOE_METRIC_LOAD_MAX_RATIO 4
#define MOE_METRIC_UNUSED_FRAC 5
#define MOE_N_METRICS 6

/* Per-call router options for training-time use; a NULL moe_route_opts*
 * means both off.
 *   sel_noise  [T, E] fp32 DEVICE array or NULL: added to every selection
 *              value after the bias (README, "SigmoidRouter": exploration
 *              noise during training, none at evaluation). The caller draws
 *              it (randn * std); the library draws no random numbers.
 *   metrics    [MOE_N_METRICS] fp64 DEVICE array or NULL: written with the
 *              router metrics of this call, bitwise repeatable. */
typedef struct moe_route_opts {
    const float *sel_noise;
    double *metrics;
} moe_route_opts;

/* Human-readable name of a status code (static storage). */
const char *moe_status_str(moe_status s);

/* Workspace bytes that moe_forward, moe_route, moe_permute and moe_combine
 * need for this layer and T tokens (one size serves all four). */
moe_status moe_workspace_size(const moe_layer *layer, int64_t T, size_t *bytes);

/*
 * Router (README "SigmoidRouter"; PR #930 qwen3 preset).
 *   x        [T, d] in layer->dtype
 *   topk_idx [T, k] int32 out: expert ids, slot 0 has the largest selection value
 *   topk_w   [T, k] fp32 out: combine weights
 *   counts   [E] int32 out: tokens per expert (may be NULL)
 *   ws       workspace of at least moe_workspace_size bytes (required when T > 0)
 * Selection value: the logit when sel_bias is NULL; otherwise the score plus
 * the bias (sigmoid: 1/(1+exp(-l)); softmax: exp(l-m)/sum exp(l-m), summed in
 * expert order), or the logit plus the bias when layer->bias_on_logits.
 * Weights: softmax renorm exp(l_j - M)/sum_i exp(l_i - M) over the chosen
 * logits; sigmoid renorm s_j/(sum_i s_i + 1e-9); without renorm the score
 * itself. T = 0 zeroes counts.
 */
moe_status moe_route(const moe_layer *layer, const void *x, int64_t T, int32_t *topk_idx, float *topk_w,
                     int32_t *counts, void *ws, size_t ws_bytes, void *stream);

/* moe_route with training options (noise, metrics; opts may be NULL).
 * opts->metrics needs T > 0 (MOE_ERR_INVALID otherwise). */
moe_status moe_route_ex(const moe_layer *layer, const void *x, int64_t T, const moe_route_opts *opts,
                        int32_t *topk_idx, float *topk_w, int32_t *counts, void *ws, size_t ws_bytes, void *stream);

/*
 * One step of the aux-loss-free balance controller (README, "SigmoidRouter",
 * step_bias_update; PR #930, "Tests": the update is applied after the
 * forward pass, so the next pass selects with the new bias). In fp32:
 *   p_e = counts_e / max(sum counts, 1);  err_e = 1/E - p_e;
 *   err_e += 0.5 where p_e < 0.1/E (starved expert);
 *   bias_e = clamp(bias_e + err_e * rate, -10, 10).
 *   counts [n_experts] int32 DEVICE (e.g. from moe_forward; summed over all
 *          data-parallel ranks by the caller first)
 *   bias   [n_experts] fp32 DEVICE, updated in place (the layer's sel_bias)
 */
moe_status moe_bias_update(int32_t n_experts, const int32_t *counts, float rate, float *bias, void *stream);

/*
 * Dispatch into expert-contiguous order ("SigmoidRouter" one-hot counts;
 * PR #930 grouped_mm over rows grouped by expert).
 *   x        [T, d] in layer->dtype
 *   topk_idx [T, k] int32 in (from moe_route; every id in [0, E), the k ids of
 *            a token distinct)
 *   x_perm   [T*k, d] out: x_perm[row_of[t, j]] = x[t]; may be NULL
 *   offsets  [E+1] int32 out: exclusive prefix sum of the per-expert counts
 *   row_of   [T, k] int32 out: row of pair (t, j) in x_perm; rows of one
 *            expert are in ascending token order
 */
moe_status moe_permute(const moe_layer *layer, const void *x, int64_t T, const int32_t *topk_idx, void *x_perm,
                       int32_t *offsets, int32_t *row_of, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for moe_grouped_swiglu. */
moe_status moe_grouped_swiglu_workspace_size(int32_t dtype, int32_t n_groups, int32_t d_in, int32_t d_ff,
                                             int64_t rows, size_t *bytes);

/*
 * SwiGLU experts over row groups (README "Architecture diagram": SwiGLU
 * experts; PR #930 "Why FSDP is enough here": stacked [E, out, in]).
 *   a        [rows, d_in] in dtype; group g owns rows offsets[g]..offsets[g+1]-1
 *   offsets  [n_groups+1] int32 DEVICE array, nondecreasing, offsets[0] = 0,
 *            offsets[n_groups] = rows (not checked on the host: it is device data)
 *   w_gate, w_up [n_groups, d_ff, d_in]; w_down [n_groups, d_in, d_ff]
 *   out      [rows, d_in] fp32: W_down[g] (silu(W_gate[g] a) * (W_up[g] a))
 * The intermediate activation is rounded to dtype (bf16 for MOE_BF16)
 * before the down projection; accumulation is fp32.
 */
moe_status moe_grouped_swiglu(int32_t dtype, int32_t n_groups, int32_t d_in, int32_t d_ff, int64_t rows,
                              const void *a, const int32_t *offsets, const void *w_gate, const void *w_up,
                              const void *w_down, float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Weighted combine back to token order (README "Architecture diagram":
 * weighted sum of the routed experts and the shared expert).
 *   y_perm   [T*k, d] fp32: expert outputs in dispatch order
 *   row_of   [T, k] int32 (from moe_permute)
 *   topk_w   [T, k] fp32
 *   y_shared [T, d] fp32 or NULL: added with weight 1 after the routed terms
 *   y        [T, d] fp32 out: y[t] = sum_j topk_w[t,j] y_perm[row_of[t,j]] (+ y_shared[t]),
 *            slots summed in order, no atomics
 */
moe_status moe_combine(const moe_layer *layer, int64_t T, const float *y_perm, const int32_t *row_of,
                       const float *topk_w, const float *y_shared, float *y, void *stream);

/*
 * The whole layer: route, dispatch, routed and shared SwiGLU experts, combine.
 *   x   [T, d] in layer->dtype
 *   y   [T, d] fp32 out
 *   topk_idx [T, k], topk_w [T, k], counts [E]: optional outputs (NULL: kept
 *   in the workspace only)
 * Routed rows are gathered from x inside the expert GEMM; no permuted copy of
 * x is written. T = 0 zeroes counts and returns.
 */
moe_status moe_forward(const moe_layer *layer, const void *x, int64_t T, float *y, int32_t *topk_idx,
                       float *topk_w, int32_t *counts, void *ws, size_t ws_bytes, void *stream);

typedef struct moe_timing moe_timing; /* opaque: one hipEvent per phase boundary */

/* moe_forward with router options (opts may be NULL) and, when `timing` is
 * not NULL, an event recorded on `stream` at every phase boundary (see
 * moe_timing_read). */
moe_status moe_forward_ex(const moe_layer *layer, const void *x, int64_t T, const moe_route_opts *opts, float *y,
                          int32_t *topk_idx, float *topk_w, int32_t *counts, void *ws, size_t ws_bytes,
                          void *stream, moe_timing *timing);

/*
 * moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results as moe_forward, with the scratch space
 * taken from a fixed array inside the library instead of a caller
 * workspace. The caller still passes x, y and the optional topk_idx,
 * topk_w and counts. No hipMalloc, hipFree or other allocation happens in
 * the call.
 *   - The array holds MOE_NOALLOC_BYTES (256 MiB) per GPU, from the first
 *     call on that GPU until the process ends. A layer and T whose
 *     moe_workspace_size exceeds it return MOE_ERR_WORKSPACE before anything
 *     is enqueued (for example: the 640-wide 16-expert layer up to 8192
 *     tokens fits; a 7168-wide 256-expert layer up to about 900).
 *   - Every call on one GPU uses that GPU's one array, whose contents persist
 *     from call to call: calls that overlap on one GPU (other streams,
 *     other host threads) race and must be ordered by the caller.
 */
#define MOE_NOALLOC_BYTES ((size_t)256 << 20)
moe_status moe_forward_noalloc(const moe_layer *layer, const void *x, int64_t T, float *y, int32_t *topk_idx,
                               float *topk_w, int32_t *counts, void *stream);

/* ---------------------------------------------------------------------- */
/* Backward pass (training)                                                */
/* ---------------------------------------------------------------------- */

/* Gradients written by moe_backward: fp32 DEVICE arrays owned by the caller,
 * each 16-byte aligned (MOE_ERR_INVALID otherwise). */
typedef struct moe_grads {
    float *dx;          /* [T, d] */
    float *dw_router;   /* [E, d] */
    float *dw_gate;     /* [E, d_ff, d] */
    float *dw_up;       /* [E, d_ff, d] */
    float *dw_down;     /* [E, d, d_ff] */
    float *dws_gate;    /* [d_ff_shared, d], or NULL without a shared expert */
    float *dws_up;      /* [d_ff_shared, d], or NULL */
    float *dws_down;    /* [d, d_ff_shared], or NULL */
    float *d_topk_w;    /* [T, k] gradient of the combine weights, or NULL */
} moe_grads;

/* Workspace bytes for moe_backward. */
moe_status moe_backward_workspace_size(const moe_layer *layer, int64_t T, size_t *bytes);

/*
 * Backward pass of the layer for the routing of its forward pass (README,
 * "SigmoidRouter" and "Architecture diagram"; PR #930, "Tests"): given
 * dy = dL/dy [T, d] fp32, writes dL/dx, the weight gradients and the
 * combine-weight gradients, for
 *   L' = L + z_loss_coef * z_loss + aux_loss_coef * aux_loss
 * (the SigmoidRouter z-loss and aux loss, one-hot counts taken as constants;
 * coefficients 0 leave them out). The expert choice passes no gradient; the
 * router's gradient flows through the combine weights, computed from the
 * unbiased scores as in the forward pass. The selection bias and any noise
 * have no gradient.
 *   x        [T, d] layer dtype (the forward's input)
 *   topk_idx [T, k], topk_w [T, k]: the forward's outputs
 * The gate/up activations are recomputed (no forward state is kept); the
 * expert outputs are not needed (d_w = <h, dy W_down>). bf16 layers round dy,
 * w dy, dG/dU and H to bf16 as GEMM operands; every accumulation is fp32. A
 * shared expert must have the routed width (MOE_ERR_UNSUPPORTED otherwise).
 * T must be positive. Deterministic: no atomics; fixed reduction orders.
 */
moe_status moe_backward(const moe_layer *layer, const void *x, int64_t T, const int32_t *topk_idx,
                        const float *topk_w, const float *dy, float z_loss_coef, float aux_loss_coef,
                        const moe_grads *grads, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* Phase timing (measurement only)                                         */
/* ---------------------------------------------------------------------- */

/* Phases of moe_forward, in launch order. */
#define MOE_PHASE_ROUTE 0          /* gate product, scores, top-k, weights, block histograms */
#define MOE_PHASE_SCAN 1           /* counts, offsets, per-block bases, GEMM tile list, router metrics */
#define MOE_PHASE_SCATTER 2        /* row_of and the row -> token map */
#define MOE_PHASE_GATEUP 3         /* routed gate/up grouped GEMM with the SwiGLU epilogue */
#define MOE_PHASE_DOWN 4           /* routed down grouped GEMM */
#define MOE_PHASE_SHARED_GATEUP 5  /* shared expert gate/up (empty without one) */
#define MOE_PHASE_SHARED_DOWN 6    /* shared expert down (empty without one) */
#define MOE_PHASE_COMBINE 7        /* weighted combine */
#define MOE_N_PHASES 8

/* Create / destroy a timing record (creates hipEvents on the current device,
 * without a system-scope fence, so recording them does not flush caches
 * between the phases they time). */
moe_status moe_timing_create(moe_timing **out);
moe_status moe_timing_destroy(moe_timing *t);

/* Time only the phases in phase_mask (bit p = phase p; default all). Each
 * event recorded between two kernels costs a few microseconds of stream
 * time, so a caller timing one phase records only that phase's two
 * boundaries. MOE_ERR_INVALID for an empty mask or bits past the last phase. */
moe_status moe_timing_select(moe_timing *t, uint32_t phase_mask);

/* Milliseconds spent in each phase by the last moe_forward_ex call that
 * used `t`; waits for its events. phase_ms: host array of MOE_N_PHASES;
 * phases outside the mask read -1. */
moe_status moe_timing_read(moe_timing *t, float *phase_ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_MOE_H */
