/*
 * moe_gemv.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts layer.
 *
 * The layer is the routed MoE FFN half of a decoder layer, as the
 * turbospark-runtime 0.3.0 source pages describe it:
 *
 *   logits[t][e] = x_t . router[e]                  (llama/state.rs,
 *                                                    RealLlamaState.router_logits_f32)
 *   s = logits + bias (bias before the top-k)        (gptoss/state.rs,
 *                                                    RealGptOssState.router_bias)
 *   ids[t] = top-k of s, ties to the lower id
 *   w[t]   = softmax over the k selected              (gptoss/state.rs,
 *                                                    RealGptOssState.per_expert_ones)
 *          | softmax over all E, read at the k, no renormalisation
 *                                                    (deepseek2/state.rs, module doc)
 *   act    = silu(clamp(gate.x)) * clamp(up.x)        (gptoss/state.rs, module doc:
 *                                                    the clamped SwiGLU)
 *   y_t    = shared(x_t) + sum_j w[t][j] * down[ids[t][j]] . act_(t,j)
 *                                                    (deepseek2/state.rs,
 *                                                    RealDeepseek2State.shared_out;
 *                                                    gptoss/state.rs, BatchedRoutedScratch:
 *                                                    phase 1 = gate/up/SwiGLU per route,
 *                                                    phase 2 = down + weighted combine)
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers named x, weights, outputs, workspace are DEVICE pointers owned by
 *    the caller; moe_config, moe_weights (the struct itself) and moe_plan are
 *    host memory.  The library never allocates or frees device memory and
 *    never synchronises: every call enqueues kernels on `stream` (a
 *    hipStream_t; NULL = the default stream) and returns.
 *  - Matrices are row-major with the reduction dimension contiguous: router
 *    [E][H], gate and up [E][I][H], down [E][H][I], shared gate and up [Is][H],
 *    shared down [H][Is].  Token rows: x [M][H], y [M][H] (fp32).
 *  - Q8_0 weights are passed as two planes: int8 values with the matrix's shape
 *    (e.g. gate [E][I][H] int8) and fp16 scales, one per 32 consecutive
 *    elements along the reduction dimension (gate_scale [E][I][H/32]).  Value =
 *    scale * q.  moe_q8_0_split converts 34-byte GGUF-style blocks into them.
 *    Weight planes must be 16-byte aligned and scale planes 4-byte aligned
 *    (MOE_ERR_INVALID otherwise).
 *  - MXFP4 weights (expert_dtype MOE_MXFP4) are passed as two planes too:
 *    FP4 E2M1 codes, two per byte with the even element in the low nibble
 *    (gate [E][I][H/2] bytes), and E8M0 scale bytes, one per 32 consecutive
 *    elements along the reduction dimension (gate_scale [E][I][H/32]).  Value
 *    = 2^(scale - 127) * element.  moe_mxfp4_split converts 17-byte blocks
 *    into them.  Code planes must be 16-byte aligned and scale planes 2-byte
 *    aligned (MOE_ERR_INVALID otherwise).
 *  - Routes: route r = t*top_k + j is slot j of token t.  "Sorted position" p
 *    is the route's index in expert-major order (experts ascending, routes
 *    ascending inside an expert), as produced by moe_permute.
 *  - Errors: a non-OK status is returned before anything is enqueued, outputs
 *    are then untouched, and moe_last_error() holds a message (per thread).
 *    MOE_ERR_HIP reports a failed kernel launch; work enqueued before it may
 *    have run.
 *  - Workspace: `ws` must hold moe_workspace_bytes(plan, M) bytes, 256-byte
 *    aligned.  It needs no initialisation and carries nothing between calls.
 *    Calls that share one workspace must be ordered on one stream; calls on
 *    different streams need different workspaces.
 *  - M = 0 is a no-op returning MOE_OK.
 */
#ifndef MOE_GEMV_H
#define MOE_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* bad argument: NULL pointer, M out of range, bad config */
    MOE_ERR_UNSUPPORTED = 2, /* valid layer this library does not implement */
    MOE_ERR_WORKSPACE = 3,   /* ws_bytes < moe_workspace_bytes(plan, M) */
    MOE_ERR_HIP = 4          /* HIP runtime error; moe_last_error() has its text */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_Q8_0 = 2, MOE_MXFP4 = 3 } moe_dtype;

typedef enum {
    MOE_TOPK_SOFTMAX = 0,         /* softmax over the k selected logits */
    MOE_SOFTMAX_ALL_NORENORM = 1, /* softmax over all E, read at the k, not renormalised */
    MOE_SIGMOID_NORM = 2          /* scores sigmoid(logit); the bias (MOE_BIAS_SELECT_ONLY)
                                     is added to the score for the selection; weights are
                                     the selected scores divided by their sum
                                     (llama/state.rs, RealLlamaState::build, MiniMax branch) */
} moe_select;

typedef enum {
    MOE_BIAS_NONE = 0,
    MOE_BIAS_LOGIT = 1,      /* bias added to the logits: selection and softmax */
    MOE_BIAS_SELECT_ONLY = 2 /* bias shifts the selection only; softmax of raw logits */
} moe_bias_mode;

typedef enum {
    MOE_PATH_AUTO = 0, /* GEMV kernels for small batches, MFMA grouped GEMM for large */
    MOE_PATH_GEMV = 1, /* always the bandwidth-bound GEMV kernels */
    MOE_PATH_MFMA = 2  /* always the MFMA grouped GEMM (bf16 x; bf16, Q8_0 or MXFP4 experts;
                          H, I and Is multiples of 64) */
} moe_path;

/* Layer description.  Validated once by moe_plan_create (fail at open). */
typedef struct moe_config {
    int32_t hidden;       /* H, > 0, multiple of 32 */
    int32_t num_experts;  /* E, 1..256 */
    int32_t top_k;        /* k, 1..min(8, E): the 8-slot limit of the pages' Q8_0 MoE kernels */
    int32_t expert_inter; /* I, > 0, multiple of 32 */
    int32_t shared_inter; /* Is, 0 (no shared expert) or > 0 and a multiple of 32 */
    int32_t max_tokens;   /* largest M a call may pass, >= 1 */
    int32_t select;       /* moe_select */
    int32_t bias_mode;    /* moe_bias_mode */
    float swiglu_limit;   /* > 0: clamp gate and up pre-activations to [-limit, limit]; 0: off */
    float rms_eps;        /* > 0: x_t / sqrt(mean(x_t^2) + eps) feeds router and experts; 0: off */
    int32_t x_dtype;      /* MOE_F32 or MOE_BF16 */
    int32_t router_dtype; /* MOE_F32, MOE_BF16 or MOE_Q8_0 (the INT8 router: int8 rows plus
                             fp16 scales per 32 elements, weights.router_scale) */
    int32_t expert_dtype; /* MOE_F32, MOE_BF16, MOE_Q8_0 or MOE_MXFP4 */
    int32_t shared_dtype; /* the expert_dtype (ignored when shared_inter = 0) */
    int32_t path;         /* moe_path */
} moe_config;

/* Device pointers to one layer's weights.  Unused fields may be NULL. */
typedef struct moe_weights {
    const void *router;          /* [E][H] in router_dtype */
    const float *bias;           /* [E] fp32; required unless bias_mode = MOE_BIAS_NONE */
    const void *gate;            /* [E][I][H] (int8 plane for Q8_0) */
    const void *up;              /* [E][I][H] */
    const void *down;            /* [E][H][I] */
    const void *gate_scale;      /* Q8_0: fp16 [E][I][H/32]; MXFP4: E8M0 bytes [E][I][H/32] */
    const void *up_scale;        /* the same for up */
    const void *down_scale;      /* Q8_0: fp16 [E][H][I/32]; MXFP4: E8M0 bytes [E][H][I/32] */
    const void *shared_gate;     /* [Is][H]; required iff shared_inter > 0 */
    const void *shared_up;       /* [Is][H] */
    const void *shared_down;     /* [H][Is] */
    const void *shared_gate_scale; /* Q8_0 / MXFP4 only: [Is][H/32] */
    const void *shared_up_scale;   /* [Is][H/32] */
    const void *shared_down_scale; /* [H][Is/32] */
    /* The INT8 router (llama/state.rs, RealLlamaState.router_ones: the INT8
     * router kernel scales each element of its input by an effective scale,
     * identically 1 where the architecture has no router scale):
     * logits[t][e] = sum_i x[t][i] * router_x_scale[i] * router[e][i]. */
    const void *router_scale;      /* router_dtype Q8_0: fp16 block scales [E][H/32] (2-byte
                                      aligned); the router plane is then int8 [E][H] */
    const void *router_x_scale;    /* bf16 [H] (16-byte aligned), or NULL for ones */
} moe_weights;

typedef struct moe_plan moe_plan; /* host-side, library-owned */

/* Validate `cfg` and build a plan.  MOE_ERR_INVALID for inconsistent values
 * (E or k < 1, k > E, H, I <= 0, Is < 0, max_tokens < 1, unknown enums);
 * MOE_ERR_UNSUPPORTED for k > 8, E > 256, H, I or Is not a multiple of 32, a
 * dtype combination the kernels do not cover, or MOE_PATH_MFMA without bf16 x,
 * bf16, Q8_0 or MXFP4 experts and H, I, Is multiples of 64.  Refusal happens here,
 * before any device work, in the
 * manner of the pages' state constructors (llama/state.rs and
 * deepseek2/state.rs, the `build` functions' open-time checks).
 * On success *plan owns host memory only; free it with moe_plan_destroy. */
moe_status moe_plan_create(const moe_config *cfg, moe_plan **plan);
void moe_plan_destroy(moe_plan *plan);

/* Workspace bytes needed by any entry point called with this M (0 <= M <=
 * max_tokens); returns 0 for M out of range.  Regions for unused features
 * (shared expert, pre-norm, the MFMA path) take no space; plans with the
 * pre-norm on hold room for moe_forward_fused's normed rows. */
size_t moe_workspace_bytes(const moe_plan *plan, int32_t M);

/* Text of the last non-OK status returned on the calling thread. */
const char *moe_last_error(void);

#define MOE_LOGITS_IN 1 /* moe_route flag: `logits` is an input; skip the router GEMV */

/* Router GEMV, bias, top-k and softmax weights (steps a1, a2).
 * x [M][H] (x_dtype); logits [M][E] fp32: written, or read if flags has
 * MOE_LOGITS_IN (NULL allowed when not wanted and not an input).
 * ids [M][k] int32 out, experts in descending key order; w [M][k] fp32 out.
 * With MOE_LOGITS_IN the selection is exact comparison of the given fp32
 * values, so ids are bit-exact. */
moe_status moe_route(const moe_plan *plan, const void *x, const moe_weights *wts, int32_t M,
                     float *logits, int32_t flags, int32_t *ids, float *w, void *ws,
                     size_t ws_bytes, void *stream);

/* Expert histogram, exclusive scan and stable scatter of the routes (a3),
 * the on-device form of the pages' route list (gptoss/state.rs,
 * BatchedRoutedScratch.batch_routes).  ids [M][k] int32 in 0..E-1, distinct
 * within a token.  Out: counts [E], offsets [E+1] (exclusive scan of counts),
 * sorted_routes [M*k] (routes in expert-major, then ascending order) and
 * route_pos [M*k] (its inverse).  Integer-exact. */
moe_status moe_permute(const moe_plan *plan, const int32_t *ids, int32_t M, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_routes, int32_t *route_pos, void *ws,
                       size_t ws_bytes, void *stream);

/* Gate/up projection with the (clamped) SwiGLU, per route (a4; the pages'
 * phase 1, gptoss/state.rs, BatchedRoutedScratch.batch_acts).
 * offsets and sorted_routes as from moe_permute.  act [M*k][I] fp32 out, row p
 * = the route at sorted position p. */
moe_status moe_expert_ffn(const moe_plan *plan, const void *x, const moe_weights *wts,
                          int32_t M, const int32_t *offsets, const int32_t *sorted_routes,
                          float *act, void *ws, size_t ws_bytes, void *stream);

/* Down projection and deterministic weighted combine (a5, a6; the pages'
 * phase 2, gptoss/state.rs, BatchedRoutedScratch.batch_y / batch_zero):
 * y[t] = seed[t] + sum_j w[t][j] * down[e] . act[route_pos[t*k+j]], summed in
 * a fixed order.  seed [M][H] fp32 or NULL (zeros).  act as from
 * moe_expert_ffn; w [M][k] fp32; y [M][H] fp32 out (may not alias act). */
moe_status moe_combine(const moe_plan *plan, const float *act, const moe_weights *wts,
                       int32_t M, const int32_t *offsets, const int32_t *sorted_routes,
                       const int32_t *route_pos, const float *w, const float *seed, float *y,
                       void *ws, size_t ws_bytes, void *stream);

/* The whole layer (a0-a7): y [M][H] fp32 out.  The shared expert, if any,
 * seeds the sum with weight 1 (deepseek2/state.rs,
 * RealDeepseek2State.shared_out).  ids_out [M][k], w_out [M][k] and
 * counts_out [E] are optional copies of the routing (NULL = not wanted).
 * With one expert (E = 1, k = 1: a dense layer) every route is expert 0 with
 * weight 1 whatever its logit, so no router runs and the router weights are
 * not read. */
moe_status moe_forward(const moe_plan *plan, const void *x, const moe_weights *wts, int32_t M,
                       float *y, int32_t *ids_out, float *w_out, int32_t *counts_out, void *ws,
                       size_t ws_bytes, void *stream);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The kernels use a static scratch array
 * of the library (32 MiB of device memory on each GPU the library runs on,
 * held until the process ends) in place of `ws`; the call allocates
 * nothing.  MOE_ERR_WORKSPACE when moe_workspace_bytes(plan, M) exceeds
 * 32 MiB (then call moe_forward with a workspace).  The first call on a
 * device looks the array's device address up.  Every call on one GPU shares
 * that GPU's array: calls that
 * overlap on one GPU (concurrent streams, or threads) race and must be
 * serialised by the caller, as calls sharing one workspace must.  Other
 * arguments and results as moe_forward. */
moe_status moe_forward_noalloc(const moe_plan *plan, const void *x, const moe_weights *wts, int32_t M,
                               float *y, int32_t *ids_out, float *w_out, int32_t *counts_out,
                               void *stream);

/* The layer with its neighbours fused (deepseek2/state.rs, module doc: the
 * post-attention RMSNorm with its weight feeds the router and the experts,
 * and the routed sum plus the shared expert is added to the residual
 * stream;
 * gptoss/state.rs, BatchedRoutedScratch: the routed sum reaches the stream
 * through one residual add):
 *   f_t = x_t / sqrt(mean_i x_ti^2 + rms_eps) * norm_weight,
 *   y_t = residual_t + shared(f_t) + sum_j w_j expert_j(f_t).
 * norm_weight: [H] stored like x (16-byte aligned), or NULL for unit gain;
 * a non-NULL norm_weight needs a plan with rms_eps > 0 (MOE_ERR_INVALID
 * otherwise).  residual: [M][H] fp32 (16-byte aligned) or NULL (zeros); it
 * may be y itself, which then updates the stream in place.  The normed rows
 * are computed once (fp32) into the workspace, which for plans with
 * rms_eps > 0 holds room for them.  Other arguments as moe_forward; with
 * both NULL this is moe_forward. */
moe_status moe_forward_fused(const moe_plan *plan, const void *x, const void *norm_weight,
                             const float *residual, const moe_weights *wts, int32_t M, float *y,
                             int32_t *ids_out, float *w_out, int32_t *counts_out, void *ws,
                             size_t ws_bytes, void *stream);

/* Kernels of moe_forward, in launch order, as reported by moe_forward_timed. */
typedef enum {
    MOE_STAGE_RMS = 0,     /* pre-norm scale (only when rms_eps > 0) */
    MOE_STAGE_ROUTER = 1,  /* router GEMV */
    MOE_STAGE_TOPK = 2,    /* bias, top-k, softmax */
    MOE_STAGE_PERMUTE = 3, /* histogram, scan, stable scatter */
    MOE_STAGE_GATEUP = 4,  /* gate/up + SwiGLU */
    MOE_STAGE_DOWN = 5,    /* down projection (+ combine on the fused GEMV form) */
    MOE_STAGE_COMBINE = 6  /* weighted combine (unfused forms only) */
} moe_stage;

/* moe_forward with timing: the same kernels on the same stream, each launched
 * with hipExtLaunchKernel so that events[2i] is recorded when the i-th stage's
 * kernel starts and events[2i+1] when it ends (the dispatch gap between
 * kernels is outside every pair, as in a profiler's kernel trace).  events are
 * hipEvent_t handles created by the caller; max_events >= 14 is always enough
 * (MOE_ERR_INVALID when a stage finds no free pair).  stages[i] (moe_stage)
 * names the i-th stage and *n_stages receives their number.  Not for use
 * under stream capture.  Used to attribute time to kernels. */
moe_status moe_forward_timed(const moe_plan *plan, const void *x, const moe_weights *wts,
                             int32_t M, float *y, int32_t *ids_out, float *w_out,
                             int32_t *counts_out, void *ws, size_t ws_bytes, void *stream,
                             void **events, int32_t max_events, int32_t *stages,
                             int32_t *n_stages);

/* Kernel family moe_forward launches for an M-token call under this plan. */
typedef enum {
    MOE_RUN_SINGLE = 0, /* one token: router, then two self-routing expert GEMVs */
    MOE_RUN_GEMV = 1,   /* routing + permutation, then gathered GEMV kernels */
    MOE_RUN_MFMA = 2    /* routing + permutation, then the MFMA grouped GEMM */
} moe_run;

/* The moe_run value for M tokens, or -1 (moe_last_error set) when the plan is
 * NULL or M is outside [1, max_tokens].  Pure host logic, no device work. */
int32_t moe_forward_path(const moe_plan *plan, int32_t M);

/* Convert Q8_0 blocks (34 bytes: little-endian fp16 scale, then 32 int8) of a
 * [rows][cols] matrix, cols a multiple of 32, into the two planes the layer
 * reads: qs [rows][cols] int8 and scales [rows][cols/32] fp16.  The block
 * format is the one the pages' GGUF MoE kernels walk (deepseek2/state.rs,
 * RealDeepseek2State::build).  Device pointers; blocks need only 2-byte
 * alignment; MOE_ERR_INVALID for rows < 0, cols <= 0 or cols % 32 != 0. */
moe_status moe_q8_0_split(const void *blocks, int64_t rows, int32_t cols, int8_t *qs,
                          uint16_t *scales, void *stream);

/* Convert MXFP4 blocks (17 bytes: the E8M0 scale byte, then 16 bytes of FP4
 * E2M1 codes, byte j holding element 2j in its low nibble and element 2j+1 in
 * its high nibble) of a [rows][cols] matrix, cols a multiple of 32, into the
 * two planes the layer reads: codes [rows][cols/2] bytes (the 16 code bytes of
 * each block, in order) and scales [rows][cols/32] E8M0 bytes.  Element and
 * scale encodings are those of the OCP Microscaling (MX) v1.0 formats, value =
 * 2^(scale - 127) * element; gptoss/state.rs (module doc and
 * BatchedRoutedScratch) names MXFP4 as the format of gpt-oss's routed expert
 * pair, and the 17-byte block layout is a reading of that.  Device pointers;
 * codes 16-byte aligned, blocks and scales any alignment (the layer
 * reads scale planes 2-byte aligned); MOE_ERR_INVALID for
 * rows < 0, cols <= 0 or cols % 32 != 0. */
moe_status moe_mxfp4_split(const void *blocks, int64_t rows, int32_t cols, uint8_t *codes,
                           uint8_t *scales, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GEMV_H */
