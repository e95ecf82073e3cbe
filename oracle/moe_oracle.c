/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct fp64 CPU implementation of the routed
 * mixture-of-experts FFN of one decoder layer.  It exists to check the HIP
 * path: only the tests, the smoke check and the bench's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, and where the turbospark-runtime 0.3.0 pages state it:
 *
 *   router logits   l[t][e] = sum_i x[t][i] * s[i] * Wr[e][i]
 *       llama/state.rs, RealLlamaState.router_logits_f32 (fp32 logits, one
 *       [num_experts] row per token) and deepseek2/state.rs module doc
 *       (the normed rows times the router).  s is the INT8 router's per-element input scale
 *       (llama/state.rs, RealLlamaState.router_ones; ones when absent) and
 *       Wr may be Q8_0 blocks (the INT8 router's rows).
 *   router bias     added to the logits BEFORE top-k
 *       gptoss/state.rs, RealGptOssState.router_bias.
 *   selection       top-k of the (biased) logits, then either
 *       - softmax over the selected k: gptoss/state.rs,
 *         RealGptOssState.per_expert_ones (unit per-expert weights change
 *         nothing, so the weights are a softmax restricted to the k), or
 *       - softmax over all experts, then top-k with NO renormalisation:
 *         deepseek2/state.rs module doc (decoder-layer sketch), or
 *       - sigmoid scores: llama/state.rs, RealLlamaState::build (the
 *         MiniMax branch requires sigmoid router scoring and a finite fp32
 *         per-expert e_score_correction_bias).  Reading: the correction bias
 *         is added to the sigmoid score for the selection only, and the
 *         weights are the selected experts' sigmoid scores divided by their
 *         sum.
 *   expert          SwiGLU down(silu(gate.x) * (up.x)) per selected expert,
 *       optionally clamped: gptoss/state.rs module doc (clamped SwiGLU).
 *   combine         y = shared + sum_j w_j * expert_j(x), seeded with zeros
 *       when there is no shared expert: deepseek2/state.rs,
 *       RealDeepseek2State.shared_out; gptoss/state.rs,
 *       BatchedRoutedScratch.batch_zero.
 *   Q8_0            32-element blocks, fp16 scale then 32 int8:
 *       deepseek2/state.rs, RealDeepseek2State::build (Q8_0 dots walk whole
 *       32-element blocks).
 *   MXFP4           gpt-oss's routed expert pair is MXFP4: gptoss/state.rs
 *       module doc (the clamp rides inside the MXFP4 routed pair),
 *       BatchedRoutedScratch.wide_blobs and RealGptOssState::ensure_batched
 *       (the MXFP4 batched pair and its argument buffer).  The pages
 *       give no encoding, so the element and scale formats are those of the
 *       OCP Microscaling (MX) v1.0 specification: 32 FP4 E2M1 elements share
 *       one E8M0 scale, value = 2^(E - 127) * element, E = 255 is NaN.
 *       Reading for the byte layout: a 17-byte block per 32 elements along
 *       the reduction, the E8M0 byte first, then 16 bytes of codes, byte j
 *       holding element 2j in its low nibble and element 2j+1 in its high
 *       nibble.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes): ties in the top-k go to the lower expert id; the clamp
 * limits both the gate and the up pre-activation to [-limit, limit]; the
 * selection key is the biased logit in both modes (softmax is monotone); the
 * optional pre-norm is RMS with unit gain; the shared expert is one SwiGLU of
 * width Is with weight 1 and no clamp.
 *
 * Every stored value is widened exactly to double (bf16, fp16, fp32; Q8_0 as
 * d*q; MXFP4 as 2^(E-127) times the E2M1 value) and every sum is taken in
 * double; no intermediate is rounded.
 *
 * Parity pins for every function here live in tests/pins.py.  The mutant
 * switch below exists only so that tests can prove those pins catch plausible
 * mistakes; it is 0 (off) unless a test sets it.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q8_0 = 2, ORC_MXFP4 = 3 };
enum { ORC_TOPK_SOFTMAX = 0, ORC_SOFTMAX_ALL_NORENORM = 1, ORC_SIGMOID_NORM = 2 };
enum { ORC_BIAS_NONE = 0, ORC_BIAS_LOGIT = 1, ORC_BIAS_SELECT_ONLY = 2 };

typedef struct {
    int hidden, num_experts, top_k, expert_inter, shared_inter;
    int select, bias_mode;
    double swiglu_limit; /* 0 = no clamp */
    double rms_eps;      /* 0 = no pre-norm */
    int x_fmt, router_fmt, expert_fmt, shared_fmt;
} orc_layer;

/* ---- deliberate mistakes, for the pin-strength tests only ---- */
enum {
    MUT_NONE = 0,
    MUT_TOPK_SOFTMAX_OVER_ALL = 1,  /* softmax-over-selected divides by the all-expert sum */
    MUT_SWAP_GATE_UP = 2,           /* SiLU applied to up instead of gate */
    MUT_BIAS_NOT_IN_SELECTION = 3,  /* logit bias ignored by the top-k */
    MUT_TIES_TO_HIGHER_ID = 4,
    MUT_CLAMP_GATE_ONLY = 5,
    MUT_DOWN_TRANSPOSED = 6,        /* down read as [I][H] */
    MUT_ALL_MODE_RENORMALISES = 7,
    MUT_DROP_SHARED = 8,
    MUT_RMS_SUM_NOT_MEAN = 9,
    MUT_UNSTABLE_PERMUTE = 10,
    MUT_Q8_NEXT_BLOCK_SCALE = 11,
    MUT_SILU_SIGN = 12,
    MUT_COMBINE_UNWEIGHTED = 13,
    MUT_SELECT_ONLY_BIAS_IN_SOFTMAX = 14,
    MUT_CLAMP_GATE_UPPER_ONLY = 15,
    MUT_NORM_ROUTER_ONLY = 16,
    MUT_SIGMOID_BIAS_BEFORE = 17,   /* sigmoid mode: correction bias added to the logit, not the score */
    MUT_SIGMOID_NO_RENORM = 18,     /* sigmoid mode: weights are the raw scores */
    MUT_FP4_NIBBLE_SWAP = 19,       /* MXFP4: element 2j read from the high nibble */
    MUT_E8M0_BIAS_128 = 20,         /* MXFP4: scale exponent bias 128 instead of 127 */
    MUT_FP4_NO_SUBNORMAL = 21,      /* MXFP4: exponent field 0 given an implicit leading one */
    MUT_MX_NEXT_BLOCK_SCALE = 22,   /* MXFP4: the next block's scale */
    MUT_NORM_WEIGHT_ROUTER_ONLY = 23, /* fused norm: the experts see the unit-gain rows */
    MUT_RESIDUAL_DROPPED = 24,      /* fused: the residual stream is not added */
    MUT_ROUTER_SCALE_IGNORED = 25,  /* INT8 router: the input scale is not applied */
    MUT_ROUTER_SCALE_ON_EXPERTS = 26, /* INT8 router: the input scale also reaches the experts */
    MUT_COUNT = 27
};
static int orc_mutant = MUT_NONE;

void orc_set_mutant(int m) { orc_mutant = m; }
int orc_mutant_count(void) { return MUT_COUNT; }

/* ---- exact widening of stored values ---- */
static double orc_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double orc_f16(uint16_t h)
{
    int sign = h >> 15, ex = (h >> 10) & 31, man = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);               /* subnormal */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);  /* (1 + m/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

/* An FP4 E2M1 code (OCP MX v1.0): bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa.  Exponent field 0 is subnormal: 0.5 * m. */
static double orc_e2m1(unsigned code)
{
    const unsigned sign = (code >> 3) & 1, ex = (code >> 1) & 3, m = code & 1;
    double v;
    if (ex == 0 && orc_mutant != MUT_FP4_NO_SUBNORMAL)
        v = 0.5 * m;
    else
        v = ldexp(1.0 + 0.5 * m, (int)ex - 1);
    return sign ? -v : v;
}

/* An E8M0 scale (OCP MX v1.0): 2^(e - 127); e = 255 is NaN. */
static double orc_e8m0(unsigned e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - (orc_mutant == MUT_E8M0_BIAS_128 ? 128 : 127));
}

/* Element (r, c) of a row-major matrix with `cols` columns stored in `fmt`. */
static double orc_at(const void *base, int fmt, size_t r, size_t cols, size_t c)
{
    switch (fmt) {
    case ORC_F32:
        return (double)((const float *)base)[r * cols + c];
    case ORC_BF16:
        return orc_bf16(((const uint16_t *)base)[r * cols + c]);
    case ORC_Q8_0: {
        size_t nb = cols / 32;
        const uint8_t *row = (const uint8_t *)base + r * nb * 34;
        size_t blk = c / 32;
        if (orc_mutant == MUT_Q8_NEXT_BLOCK_SCALE)
            blk = (blk + 1) % nb;
        uint16_t d = (uint16_t)(row[blk * 34] | (row[blk * 34 + 1] << 8));
        int8_t q = (int8_t)row[(c / 32) * 34 + 2 + c % 32];
        return orc_f16(d) * (double)q;
    }
    case ORC_MXFP4: {
        size_t nb = cols / 32;
        const uint8_t *row = (const uint8_t *)base + r * nb * 17;
        size_t blk = c / 32, j = c % 32;
        size_t sblk = orc_mutant == MUT_MX_NEXT_BLOCK_SCALE ? (blk + 1) % nb : blk;
        uint8_t byte = row[blk * 17 + 1 + j / 2];
        int high = (j % 2 == 1) != (orc_mutant == MUT_FP4_NIBBLE_SWAP);
        return orc_e8m0(row[sblk * 17]) * orc_e2m1(high ? byte >> 4 : byte & 15);
    }
    }
    return NAN;
}

/* Row r of a matrix with `cols` columns, dotted with v[cols]. */
static double orc_row_dot(const void *base, int fmt, size_t r, size_t cols, const double *v)
{
    double s = 0.0;
    for (size_t c = 0; c < cols; c++)
        s += orc_at(base, fmt, r, cols, c) * v[c];
    return s;
}

/* ---- step 0 (optional): RMS pre-norm, x / sqrt(mean(x^2) + eps) * gamma ----
 * deepseek2/state.rs module doc: the post-attention RMSNorm's output feeds
 * the router and the experts.  gamma (norm_w, [H] in the x format) is
 * the norm's weight; NULL is unit gain. */
static void norm_tokens(const orc_layer *L, int M, const void *x, const void *norm_w, double *xn)
{
    const int H = L->hidden;
    for (int t = 0; t < M; t++) {
        for (int i = 0; i < H; i++)
            xn[(size_t)t * H + i] = orc_at(x, L->x_fmt, t, H, i);
        if (L->rms_eps > 0.0) {
            double ss = 0.0;
            for (int i = 0; i < H; i++)
                ss += xn[(size_t)t * H + i] * xn[(size_t)t * H + i];
            double mean = (orc_mutant == MUT_RMS_SUM_NOT_MEAN) ? ss : ss / H;
            double r = sqrt(mean + L->rms_eps);
            for (int i = 0; i < H; i++) {
                xn[(size_t)t * H + i] /= r;
                if (norm_w)
                    xn[(size_t)t * H + i] *= orc_at(norm_w, L->x_fmt, 0, H, i);
            }
        }
    }
}

void orc_norm_tokens(const orc_layer *L, int M, const void *x, double *xn)
{
    norm_tokens(L, M, x, NULL, xn);
}

/* ---- step 1: router logits ----
 * l[t][e] = sum_i (xn[t][i] * xs[i]) * Wr[e][i], xs the router's input scale
 * (bf16 [H], or NULL for ones): the INT8 router kernel of llama/state.rs
 * (RealLlamaState.router_ones) scales each element of its input by an
 * effective scale, identically 1 where the architecture has no router scale
 * (gptoss/state.rs and deepseek2/state.rs, router_ones).  The router rows
 * may be Q8_0 blocks like the experts' (the INT8 router's weights). */
void orc_router_logits(const orc_layer *L, int M, const double *xn, const void *router,
                       const uint16_t *xs, double *logits)
{
    const int H = L->hidden, E = L->num_experts;
    double *xr = malloc(sizeof(double) * (size_t)M * H);
    for (size_t i = 0; i < (size_t)M * H; i++)
        xr[i] = (xs && orc_mutant != MUT_ROUTER_SCALE_IGNORED) ? xn[i] * orc_bf16(xs[i % H]) : xn[i];
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < M; t++)
        for (int e = 0; e < E; e++)
            logits[(size_t)t * E + e] = orc_row_dot(router, L->router_fmt, e, H, xr + (size_t)t * H);
    free(xr);
}

/* ---- steps 2-4: bias, top-k, weights for one token ----
 * s = selection key, u = softmax input (sigmoid mode: the score):
 *   NONE: s = u = l;  LOGIT: s = u = l + b;  SELECT_ONLY: s = l + b, u = l;
 *   sigmoid mode: u = sigmoid(l), s = u (+ b with any bias mode).
 * If `forced` is non-NULL its k ids are taken as the selection (slot order
 * kept) and only the weights are computed. */
static void orc_select_token(const orc_layer *L, const double *l, const float *bias,
                             const int32_t *forced, int32_t *ids, double *w)
{
    const int E = L->num_experts, k = L->top_k;
    double *s = malloc(sizeof(double) * E), *u = malloc(sizeof(double) * E);
    char *taken = calloc(E, 1);
    for (int e = 0; e < E; e++) {
        double b = bias ? (double)bias[e] : 0.0;
        s[e] = u[e] = l[e];
        if (L->select == ORC_SIGMOID_NORM) {
            const double bb = L->bias_mode != ORC_BIAS_NONE ? b : 0.0;
            u[e] = 1.0 / (1.0 + exp(-l[e]));
            s[e] = u[e] + bb;
            if (orc_mutant == MUT_SIGMOID_BIAS_BEFORE)
                s[e] = 1.0 / (1.0 + exp(-(l[e] + bb)));
            continue;
        }
        if (L->bias_mode == ORC_BIAS_LOGIT) {
            s[e] = l[e] + b;
            u[e] = l[e] + b;
            if (orc_mutant == MUT_BIAS_NOT_IN_SELECTION)
                s[e] = l[e];
        } else if (L->bias_mode == ORC_BIAS_SELECT_ONLY) {
            s[e] = l[e] + b;
            if (orc_mutant == MUT_SELECT_ONLY_BIAS_IN_SOFTMAX)
                u[e] = l[e] + b;
        }
    }
    for (int j = 0; j < k; j++) {
        int best = -1;
        if (forced) {
            best = forced[j];
        } else {
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                int better = (orc_mutant == MUT_TIES_TO_HIGHER_ID) ? (best < 0 || s[e] >= s[best])
                                                                   : (best < 0 || s[e] > s[best]);
                if (better)
                    best = e;
            }
        }
        ids[j] = best;
        taken[best] = 1;
    }
    int over_all = (L->select == ORC_SOFTMAX_ALL_NORENORM && orc_mutant != MUT_ALL_MODE_RENORMALISES) ||
                   (L->select == ORC_TOPK_SOFTMAX && orc_mutant == MUT_TOPK_SOFTMAX_OVER_ALL);
    if (L->select == ORC_SIGMOID_NORM) {
        /* the selected experts' scores, divided by their sum */
        double z = 0.0;
        for (int j = 0; j < k; j++)
            z += u[ids[j]];
        for (int j = 0; j < k; j++)
            w[j] = orc_mutant == MUT_SIGMOID_NO_RENORM ? u[ids[j]] : u[ids[j]] / z;
    } else if (!over_all) {
        /* softmax restricted to the k selected experts */
        double m = u[ids[0]];
        for (int j = 1; j < k; j++)
            if (u[ids[j]] > m)
                m = u[ids[j]];
        double z = 0.0;
        for (int j = 0; j < k; j++)
            z += exp(u[ids[j]] - m);
        for (int j = 0; j < k; j++)
            w[j] = exp(u[ids[j]] - m) / z;
    } else {
        /* softmax over all experts, read at the selected ones, no renorm */
        double m = u[0];
        for (int e = 1; e < E; e++)
            if (u[e] > m)
                m = u[e];
        double z = 0.0;
        for (int e = 0; e < E; e++)
            z += exp(u[e] - m);
        for (int j = 0; j < k; j++)
            w[j] = exp(u[ids[j]] - m) / z;
    }
    free(s);
    free(u);
    free(taken);
}

void orc_select(const orc_layer *L, int M, const double *logits, const float *bias,
                const int32_t *forced_ids, int32_t *ids, double *w)
{
    const int E = L->num_experts, k = L->top_k;
    for (int t = 0; t < M; t++)
        orc_select_token(L, logits + (size_t)t * E, bias,
                         forced_ids ? forced_ids + (size_t)t * k : NULL,
                         ids + (size_t)t * k, w + (size_t)t * k);
}

/* ---- step 5: counting sort of the routes r = t*k + j by expert ----
 * sorted_routes lists, expert by expert (ascending id), the routes that
 * chose it in ascending r; route_pos is the inverse map. */
void orc_permute(int E, int M, int k, const int32_t *ids, int32_t *counts, int32_t *offsets,
                 int32_t *sorted_routes, int32_t *route_pos)
{
    const int R = M * k;
    offsets[0] = 0;
    for (int e = 0; e < E; e++) {
        counts[e] = 0;
        for (int r = 0; r < R; r++)
            if (ids[r] == e)
                counts[e]++;
        offsets[e + 1] = offsets[e] + counts[e];
    }
    int pos = 0;
    for (int e = 0; e < E; e++) {
        if (orc_mutant == MUT_UNSTABLE_PERMUTE) {
            for (int r = R - 1; r >= 0; r--)
                if (ids[r] == e) {
                    sorted_routes[pos] = r;
                    route_pos[r] = pos++;
                }
        } else {
            for (int r = 0; r < R; r++)
                if (ids[r] == e) {
                    sorted_routes[pos] = r;
                    route_pos[r] = pos++;
                }
        }
    }
}

/* ---- step 6: one SwiGLU expert ----
 * gate/up are [n_mat][width][H] and down is [n_mat][H][width]; `mat` picks
 * the expert.  act[width] = silu(clamp(g)) * clamp(v); out[H] = down . act */
static double orc_silu(double g)
{
    if (orc_mutant == MUT_SILU_SIGN)
        return g / (1.0 + exp(g));
    return g / (1.0 + exp(-g));
}

static double orc_clamp(double v, double lim)
{
    return v < -lim ? -lim : (v > lim ? lim : v);
}

void orc_swiglu_act(int H, int width, int fmt, double limit, const void *gate, const void *up,
                    int mat, const double *xn, double *act)
{
    /* rows are independent; spread them over the threads when the caller's
       token loop is not itself parallel (each row's dot is the same serial
       sum either way) */
#pragma omp parallel for schedule(static) if (!omp_in_parallel() && (long)width * H >= (1L << 18))
    for (int i = 0; i < width; i++) {
        size_t row = (size_t)mat * width + i;
        double g = orc_row_dot(gate, fmt, row, H, xn);
        double v = orc_row_dot(up, fmt, row, H, xn);
        if (orc_mutant == MUT_SWAP_GATE_UP) {
            double tmp = g;
            g = v;
            v = tmp;
        }
        if (limit > 0.0) {
            if (orc_mutant == MUT_CLAMP_GATE_UPPER_ONLY) {
                g = g > limit ? limit : g;
                v = orc_clamp(v, limit);
            } else {
                g = orc_clamp(g, limit);
                if (orc_mutant != MUT_CLAMP_GATE_ONLY)
                    v = orc_clamp(v, limit);
            }
        }
        act[i] = orc_silu(g) * v;
    }
}

void orc_down(int H, int width, int fmt, const void *down, int mat, const double *act, double *out)
{
#pragma omp parallel for schedule(static) if (!omp_in_parallel() && (long)width * H >= (1L << 18))
    for (int h = 0; h < H; h++) {
        if (orc_mutant == MUT_DOWN_TRANSPOSED && fmt != ORC_Q8_0 && fmt != ORC_MXFP4) {
            /* read element (h, i) at flat index i*H + h of the expert's block */
            double s = 0.0;
            for (int i = 0; i < width; i++) {
                size_t flat = (size_t)i * H + h;
                s += orc_at(down, fmt, (size_t)mat * H + flat / width, width, flat % width) * act[i];
            }
            out[h] = s;
        } else {
            out[h] = orc_row_dot(down, fmt, (size_t)mat * H + h, width, act);
        }
    }
}

/* ---- the whole layer ----
 * Outputs (any may be NULL except y): logits[M][E], ids[M][k], w[M][k],
 * counts[E], act[M*k][I] (route-major, r = t*k + j), y[M][H].
 * forced_ids (or NULL) fixes the selection, as described above. */
/* The layer with its neighbours (deepseek2/state.rs module doc: the normed
 * rows feed the router and the experts, and the routed sum plus the shared
 * SwiGLU is added to the residual stream; gptoss/state.rs, BatchedRoutedScratch: the routed sum reaches
 * the stream through one residual add):
 *   y_t = residual_t + shared(f_t) + sum_j w_j expert_j(f_t),
 *   f_t = x_t / sqrt(mean(x_t^2) + eps) * norm_w.
 * norm_w ([H] in the x format) needs rms_eps > 0 (else the call is refused);
 * residual ([M][H] fp32) or NULL for zeros; router_xs (bf16 [H]) or NULL:
 * the router's input scale (step 1).  orc_forward is the case
 * norm_w = residual = router_xs = NULL. */
int orc_forward_fused(const orc_layer *L, int M, const void *x, const void *norm_w,
                      const float *residual, const void *router, const uint16_t *router_xs,
                      const float *bias, const void *gate,
                      const void *up, const void *down, const void *sgate, const void *sup,
                      const void *sdown, const int32_t *forced_ids, double *logits_out,
                      int32_t *ids_out, double *w_out, int32_t *counts_out, double *act_out, double *y)
{
    const int H = L->hidden, E = L->num_experts, k = L->top_k, I = L->expert_inter;
    const int Is = L->shared_inter;
    if (M < 0 || H <= 0 || E <= 0 || k <= 0 || k > E || I <= 0 || Is < 0)
        return 1;
    if (norm_w && !(L->rms_eps > 0.0))
        return 1;
    if (M == 0)
        return 0;
    double *xn = malloc(sizeof(double) * (size_t)M * H);
    double *logits = malloc(sizeof(double) * (size_t)M * E);
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)M * k);
    double *w = malloc(sizeof(double) * (size_t)M * k);
    norm_tokens(L, M, x, norm_w, xn);
    if (orc_mutant == MUT_NORM_ROUTER_ONLY) {
        /* the router sees the normed rows, the experts the raw ones */
        orc_router_logits(L, M, xn, router, router_xs, logits);
        orc_layer raw = *L;
        raw.rms_eps = 0.0;
        norm_tokens(&raw, M, x, NULL, xn);
    } else if (orc_mutant == MUT_NORM_WEIGHT_ROUTER_ONLY) {
        /* the router sees the weighted rows, the experts the unit-gain ones */
        orc_router_logits(L, M, xn, router, router_xs, logits);
        norm_tokens(L, M, x, NULL, xn);
    } else {
        orc_router_logits(L, M, xn, router, router_xs, logits);
    }
    if (orc_mutant == MUT_ROUTER_SCALE_ON_EXPERTS && router_xs)
        for (size_t i = 0; i < (size_t)M * H; i++)
            xn[i] *= orc_bf16(router_xs[i % H]);
    orc_select(L, M, logits, bias, forced_ids, ids, w);

    /* tokens in parallel when there are enough of them; otherwise the expert
       rows of each token are (orc_swiglu_act, orc_down) */
#pragma omp parallel for schedule(dynamic, 1) if (M >= omp_get_max_threads())
    for (int t = 0; t < M; t++) {
        const double *xt = xn + (size_t)t * H;
        double *yt = y + (size_t)t * H;
        int wmax = I > Is ? I : Is;
        double *act = malloc(sizeof(double) * wmax);
        double *out = malloc(sizeof(double) * H);
        /* seed: the residual stream (or zeros), plus the shared expert
           (weight 1, no clamp) */
        for (int h = 0; h < H; h++)
            yt[h] = (residual && orc_mutant != MUT_RESIDUAL_DROPPED) ? (double)residual[(size_t)t * H + h] : 0.0;
        if (Is > 0 && orc_mutant != MUT_DROP_SHARED) {
            orc_swiglu_act(H, Is, L->shared_fmt, 0.0, sgate, sup, 0, xt, act);
            orc_down(H, Is, L->shared_fmt, sdown, 0, act, out);
            for (int h = 0; h < H; h++)
                yt[h] += out[h];
        }
        /* routed experts, summed in slot order */
        for (int j = 0; j < k; j++) {
            int e = ids[(size_t)t * k + j];
            orc_swiglu_act(H, I, L->expert_fmt, L->swiglu_limit, gate, up, e, xt, act);
            if (act_out)
                memcpy(act_out + ((size_t)t * k + j) * I, act, sizeof(double) * I);
            orc_down(H, I, L->expert_fmt, down, e, act, out);
            double wj = (orc_mutant == MUT_COMBINE_UNWEIGHTED) ? 1.0 : w[(size_t)t * k + j];
            for (int h = 0; h < H; h++)
                yt[h] += wj * out[h];
        }
        free(act);
        free(out);
    }

    if (logits_out)
        memcpy(logits_out, logits, sizeof(double) * (size_t)M * E);
    if (ids_out)
        memcpy(ids_out, ids, sizeof(int32_t) * (size_t)M * k);
    if (w_out)
        memcpy(w_out, w, sizeof(double) * (size_t)M * k);
    if (counts_out)
        for (int e = 0; e < E; e++) {
            counts_out[e] = 0;
            for (int r = 0; r < M * k; r++)
                if (ids[r] == e)
                    counts_out[e]++;
        }
    free(xn);
    free(logits);
    free(ids);
    free(w);
    return 0;
}

int orc_forward(const orc_layer *L, int M, const void *x, const void *router, const float *bias,
                const void *gate, const void *up, const void *down, const void *sgate,
                const void *sup, const void *sdown, const int32_t *forced_ids, double *logits_out,
                int32_t *ids_out, double *w_out, int32_t *counts_out, double *act_out, double *y)
{
    return orc_forward_fused(L, M, x, NULL, NULL, router, NULL, bias, gate, up, down, sgate, sup, sdown,
                             forced_ids, logits_out, ids_out, w_out, counts_out, act_out, y);
}

/* The routing half alone, for every token: the (normed, weighted) rows,
 * the logits, the selection and its weights, computed exactly as
 * orc_forward_fused computes them (steps 0-4; router_xs as there).  Lets a test check every
 * token's selection and the per-expert counts of a batch whose expert work
 * is too slow to run whole.  norm_w as in orc_forward_fused; logits may be
 * NULL. */
int orc_route(const orc_layer *L, int M, const void *x, const void *norm_w, const void *router,
              const uint16_t *router_xs, const float *bias, double *logits_out, int32_t *ids, double *w)
{
    const int H = L->hidden, E = L->num_experts;
    if (M < 0 || H <= 0 || E <= 0 || L->top_k <= 0 || L->top_k > E)
        return 1;
    if (norm_w && !(L->rms_eps > 0.0))
        return 1;
    if (M == 0)
        return 0;
    double *xn = malloc(sizeof(double) * (size_t)M * H);
    double *logits = logits_out ? logits_out : malloc(sizeof(double) * (size_t)M * E);
    norm_tokens(L, M, x, norm_w, xn);
    orc_router_logits(L, M, xn, router, router_xs, logits);
    orc_select(L, M, logits, bias, NULL, ids, w);
    if (!logits_out)
        free(logits);
    free(xn);
    return 0;
}

/* Expose the element reader so tests can check the format decoding against
 * independent closed forms. */
double orc_element(const void *base, int fmt, long long r, long long cols, long long c)
{
    return orc_at(base, fmt, (size_t)r, (size_t)cols, (size_t)c);
}

/* Thread count OpenMP would use (for the CPU-baseline report). */
int orc_threads(void)
{
    return omp_get_max_threads();
}
