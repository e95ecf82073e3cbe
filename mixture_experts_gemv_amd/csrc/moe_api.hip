// C ABI of the routed MoE layer: plan creation and validation, workspace
// layout, and the enqueueing of the kernels for each entry point.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "common.h"
#include "launch.h"
#include "moe_gemv.h"
#include "topk.h"

struct moe_plan {
    moe_config cfg;
    moe::Layer L;
    bool mfma_capable;
};

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

moe_status hip_fail(hipError_t e, const char *what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Where each workspace region starts for a call with M tokens.
struct WsLayout {
    size_t tok_scale, logits, ids, w, counts, offsets, sorted, route_pos, active, tiles, hist;
    size_t act, shared_act, y_routes, y_shared, xn, xs, xh, total;
    int max_tiles;
};

bool use_mfma(const moe_plan *p, int M) {
    if (!p->mfma_capable) return false;
    if (p->cfg.path == MOE_PATH_MFMA) return true;
    if (p->cfg.path == MOE_PATH_GEMV) return false;
    // From about two routes per expert on (four with Q8_0 or MXFP4 experts,
    // whose conversion and block scales cost the grouped GEMM more), the
    // grouped GEMM (32-row tiles at small batches) beats the per-row kernels,
    // whose dot-product work grows with the tokens each expert sees.
    const long routes = (long)M * p->L.k;
    const long per_expert = p->L.edt == moe::DT_Q8 || p->L.edt == moe::DT_MX4 ? 4 : 2;
    return M >= 8 && routes >= per_expert * p->L.E;
}

WsLayout layout(const moe_plan *p, int M) {
    const moe::Layer &L = p->L;
    const size_t R = (size_t)M * L.k;
    const bool mfma = use_mfma(p, M);
    WsLayout w{};
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
    w.tok_scale = take(L.eps > 0.f ? (size_t)M * 4 : 0);
    w.logits = take((size_t)M * L.E * 4);
    w.ids = take(R * 4);
    w.w = take(R * 4);
    w.counts = take((size_t)L.E * 4);
    w.offsets = take((size_t)(L.E + 1) * 4);
    w.sorted = take(R * 4);
    w.route_pos = take(R * 4);
    w.active = take((size_t)(L.E + 1) * 4);
    // per-group expert counts of the top-k (batches past the small-batch route)
    w.hist = take((size_t)moe::topk_hist_groups(M) * L.E * 4);
    // tile capacity for the smaller of the two tile heights (the layer call's
    // or the stage-wise entry points')
    const int tile_rows = std::min(moe::mfma_tile_rows(), moe::mfma_tile_rows(L, M));
    w.max_tiles = mfma ? (int)(R / tile_rows + (R < (size_t)L.E ? R : (size_t)L.E) + 1) : 0;
    w.tiles = take(mfma ? (size_t)(2 + L.E + 2 * w.max_tiles) * 4 : 4 * 3);
    w.act = take(R * L.I * 4);
    w.shared_act = take(L.Is > 0 ? (size_t)M * L.Is * 4 : 0);
    // (the most reduction slices of the two tile heights; moe_combine with
    // Q8_0 or MXFP4 experts uses the row kernels' slices even when the layer
    // call takes the grouped GEMM)
    const size_t slices = mfma ? std::max({moe::down_ksplit(L, M, moe::mfma_tile_rows()),
                                           moe::down_ksplit(L, M, moe::mfma_tile_rows(L, M)),
                                           L.edt != moe::DT_BF16 ? moe::down_gemv_slices(L.I, L.edt) : 1})
                               : moe::down_gemv_slices(L.I, L.edt);
    // (the grouped-GEMM router's partial logits [S][M][E] live here until the
    // top-k has read them)
    // (and, for the pre-norm, their partial sums of squares [S][M])
    w.y_routes = take(std::max(slices * R * L.H * 4,
                               mfma ? (size_t)moe::router_slices(L, M) * M * (L.E + 1) * 4 : (size_t)0));
    w.y_shared = take(L.Is > 0 ? (size_t)(mfma ? 1 : moe::down_gemv_slices(L.Is, L.sdt)) * M * L.H * 4 : 0);
    // the weighted pre-norm's rows (moe_forward_fused with a norm weight):
    // fp32, and for the grouped-GEMM path split bf16 (router) and fp16
    // (experts); only plans with the pre-norm on
    w.xn = take(L.eps > 0.f ? (size_t)M * L.H * 4 : 0);
    w.xs = take(L.eps > 0.f && mfma ? (size_t)M * L.H * 4 : 0);
    w.xh = take(L.eps > 0.f && mfma ? (size_t)M * L.H * 2 : 0);
    w.total = o;
    return w;
}

template <class T> T *at(void *ws, size_t off) { return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off); }

moe::Mats routed_mats(const moe_weights *w) {
    return moe::Mats{w->gate, w->up, w->down, w->gate_scale, w->up_scale, w->down_scale};
}
moe::Mats shared_mats(const moe_weights *w) {
    return moe::Mats{w->shared_gate, w->shared_up, w->shared_down, w->shared_gate_scale,
                     w->shared_up_scale, w->shared_down_scale};
}

moe_status check_call(const moe_plan *p, int32_t M, void *ws, size_t ws_bytes) {
    if (!p) return fail(MOE_ERR_INVALID, "plan is NULL");
    if (M < 0 || M > p->cfg.max_tokens)
        return fail(MOE_ERR_INVALID, "M = %d outside 0..max_tokens (%d)", M, p->cfg.max_tokens);
    if (M == 0) return MOE_OK;
    const size_t need = layout(p, M).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace holds %zu bytes; M = %d needs %zu", ws_bytes, M, need);
    if (!ws) return fail(MOE_ERR_INVALID, "workspace is NULL");
    if (!aligned(ws, kAlign)) return fail(MOE_ERR_INVALID, "workspace is not 256-byte aligned");
    return MOE_OK;
}

moe_status need_ptr(const void *ptr, size_t align, const char *name) {
    if (!ptr) return fail(MOE_ERR_INVALID, "%s is NULL", name);
    if (!aligned(ptr, align)) return fail(MOE_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
    return MOE_OK;
}

#define TRY(expr)                                   \
    do {                                            \
        moe_status st_ = (expr);                    \
        if (st_ != MOE_OK) return st_;              \
    } while (0)

#define LAUNCH(expr, what)                          \
    do {                                            \
        hipError_t e_ = (expr);                     \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

moe_status check_experts(const moe_plan *p, const moe_weights *w, bool need_gateup, bool need_down,
                         bool need_shared) {
    if (!w) return fail(MOE_ERR_INVALID, "weights is NULL");
    // block scale planes: Q8_0 fp16 (4-byte aligned), MXFP4 E8M0 bytes (2-byte
    // aligned: the grouped GEMM reads a column's two scales of a stage at once)
    auto scale_align = [](int dt) -> size_t { return dt == moe::DT_Q8 ? 4 : (dt == moe::DT_MX4 ? 2 : 0); };
    const size_t sa = scale_align(p->L.edt);
    if (need_gateup) {
        TRY(need_ptr(w->gate, 16, "weights.gate"));
        TRY(need_ptr(w->up, 16, "weights.up"));
        if (sa) {
            TRY(need_ptr(w->gate_scale, sa, "weights.gate_scale"));
            TRY(need_ptr(w->up_scale, sa, "weights.up_scale"));
        }
    }
    if (need_down) {
        TRY(need_ptr(w->down, 16, "weights.down"));
        if (sa) TRY(need_ptr(w->down_scale, sa, "weights.down_scale"));
    }
    if (need_shared && p->L.Is > 0) {
        const size_t ssa = scale_align(p->L.sdt);
        TRY(need_ptr(w->shared_gate, 16, "weights.shared_gate"));
        TRY(need_ptr(w->shared_up, 16, "weights.shared_up"));
        TRY(need_ptr(w->shared_down, 16, "weights.shared_down"));
        if (ssa) {
            TRY(need_ptr(w->shared_gate_scale, ssa, "weights.shared_gate_scale"));
            TRY(need_ptr(w->shared_up_scale, ssa, "weights.shared_up_scale"));
            TRY(need_ptr(w->shared_down_scale, ssa, "weights.shared_down_scale"));
        }
    }
    return MOE_OK;
}

moe_status check_router(const moe_plan *p, const moe_weights *w, bool need_router) {
    if (!w) return fail(MOE_ERR_INVALID, "weights is NULL");
    if (need_router) {
        TRY(need_ptr(w->router, 16, "weights.router"));
        if (p->L.rdt == moe::DT_Q8) TRY(need_ptr(w->router_scale, 2, "weights.router_scale"));
        if (w->router_x_scale) TRY(need_ptr(w->router_x_scale, 16, "weights.router_x_scale"));
    }
    if (p->L.bias_mode != MOE_BIAS_NONE) TRY(need_ptr(w->bias, 4, "weights.bias"));
    return MOE_OK;
}

moe::RouterW router_w(const moe_plan *p, const moe_weights *w) {
    return moe::RouterW{w->router, p->L.rdt == moe::DT_Q8 ? w->router_scale : nullptr,
                        static_cast<const uint16_t *>(w->router_x_scale)};
}

} // namespace

// ------------------------------------------------------------ static scratch
// The workspace of moe_forward_noalloc: one array in device memory per GPU,
// held until the process ends, for callers that cannot allocate.  In host
// code `scratch` names a host-side stand-in, not device memory: kernels and
// copies take the device address hipGetSymbolAddress gives for the current
// device, looked up once per device and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// Device address of the current device's scratch (looked up on the first
// call on each device).
moe_status device_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || !aligned(ptr, kAlign)) return fail(MOE_ERR_HIP, "static scratch has no usable device address");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}
} // namespace

namespace moe {
StageTimer &stage_timer() {
    static thread_local StageTimer t;
    return t;
}
} // namespace moe

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

moe_status moe_plan_create(const moe_config *c, moe_plan **out) {
    if (!c || !out) return fail(MOE_ERR_INVALID, "config or plan pointer is NULL");
    *out = nullptr;
    if (c->num_experts < 1 || c->top_k < 1)
        return fail(MOE_ERR_INVALID, "num_experts (%d) and top_k (%d) must both be positive", c->num_experts, c->top_k);
    if (c->top_k > c->num_experts)
        return fail(MOE_ERR_INVALID, "top_k %d exceeds num_experts %d", c->top_k, c->num_experts);
    if (c->hidden <= 0 || c->expert_inter <= 0 || c->shared_inter < 0)
        return fail(MOE_ERR_INVALID, "hidden (%d) and expert_inter (%d) must be positive, shared_inter (%d) non-negative",
                    c->hidden, c->expert_inter, c->shared_inter);
    if (c->max_tokens < 1) return fail(MOE_ERR_INVALID, "max_tokens must be >= 1");
    if (c->select != MOE_TOPK_SOFTMAX && c->select != MOE_SOFTMAX_ALL_NORENORM && c->select != MOE_SIGMOID_NORM)
        return fail(MOE_ERR_INVALID, "unknown select mode %d", c->select);
    if (c->bias_mode < MOE_BIAS_NONE || c->bias_mode > MOE_BIAS_SELECT_ONLY)
        return fail(MOE_ERR_INVALID, "unknown bias mode %d", c->bias_mode);
    if (c->path < MOE_PATH_AUTO || c->path > MOE_PATH_MFMA) return fail(MOE_ERR_INVALID, "unknown path %d", c->path);
    if (!(c->swiglu_limit >= 0.f) || !(c->rms_eps >= 0.f))
        return fail(MOE_ERR_INVALID, "swiglu_limit and rms_eps must be >= 0");
    auto known = [](int d) { return d == MOE_F32 || d == MOE_BF16 || d == MOE_Q8_0 || d == MOE_MXFP4; };
    if (!known(c->x_dtype) || !known(c->router_dtype) || !known(c->expert_dtype) ||
        (c->shared_inter > 0 && !known(c->shared_dtype)))
        return fail(MOE_ERR_INVALID, "unknown dtype");
    if (c->select == MOE_SIGMOID_NORM && c->bias_mode == MOE_BIAS_LOGIT)
        return fail(MOE_ERR_UNSUPPORTED, "sigmoid scoring takes its bias for the selection only (MOE_BIAS_SELECT_ONLY)");
    if (c->top_k > 8) return fail(MOE_ERR_UNSUPPORTED, "top_k %d exceeds the 8 routing slots", c->top_k);
    if (c->num_experts > 256) return fail(MOE_ERR_UNSUPPORTED, "num_experts %d exceeds 256", c->num_experts);
    if (c->hidden % 32 || c->expert_inter % 32 || c->shared_inter % 32)
        return fail(MOE_ERR_UNSUPPORTED, "hidden, expert_inter and shared_inter must be multiples of 32");
    if (c->hidden > 16384) return fail(MOE_ERR_UNSUPPORTED, "hidden %d exceeds 16384", c->hidden);
    if (c->x_dtype == MOE_Q8_0 || c->x_dtype == MOE_MXFP4)
        return fail(MOE_ERR_UNSUPPORTED, "x must be fp32 or bf16");
    if (c->router_dtype == MOE_MXFP4)
        return fail(MOE_ERR_UNSUPPORTED, "the router must be fp32, bf16 or Q8_0");
    if (c->shared_inter > 0 && c->shared_dtype != c->expert_dtype)
        return fail(MOE_ERR_UNSUPPORTED, "the shared expert must use the routed experts' dtype");
    if ((long)c->max_tokens * c->top_k > (1L << 30))
        return fail(MOE_ERR_UNSUPPORTED, "max_tokens * top_k too large");
    const moe::Layer L{c->hidden, c->num_experts, c->top_k, c->expert_inter, c->shared_inter,
                       c->select, c->bias_mode, c->swiglu_limit, c->rms_eps,
                       c->x_dtype, c->router_dtype, c->expert_dtype, c->shared_dtype};
    const bool mfma_ok = moe::mfma_supported(L);
    if (c->path == MOE_PATH_MFMA && !mfma_ok)
        return fail(MOE_ERR_UNSUPPORTED,
                    "the MFMA path needs bf16 x, bf16, Q8_0 or MXFP4 experts and hidden, expert_inter, "
                    "shared_inter multiples of 64");
    moe_plan *p = new moe_plan;
    p->cfg = *c;
    p->L = L;
    p->mfma_capable = mfma_ok;
    *out = p;
    return MOE_OK;
}

void moe_plan_destroy(moe_plan *p) { delete p; }

size_t moe_workspace_bytes(const moe_plan *p, int32_t M) {
    if (!p || M < 0 || M > p->cfg.max_tokens) return 0;
    if (M == 0) return 0;
    return layout(p, M).total;
}

moe_status moe_route(const moe_plan *p, const void *x, const moe_weights *wts, int32_t M,
                     float *logits, int32_t flags, int32_t *ids, float *w, void *ws,
                     size_t ws_bytes, void *stream) {
    TRY(check_call(p, M, ws, ws_bytes));
    if (M == 0) return MOE_OK;
    const bool logits_in = flags & MOE_LOGITS_IN;
    if (flags & ~MOE_LOGITS_IN) return fail(MOE_ERR_INVALID, "unknown flags 0x%x", flags);
    TRY(check_router(p, wts, !logits_in));
    if (logits_in) TRY(need_ptr(logits, 4, "logits"));
    else TRY(need_ptr(x, 16, "x"));
    TRY(need_ptr(ids, 4, "ids"));
    TRY(need_ptr(w, 4, "w"));
    const moe::Layer &L = p->L;
    const WsLayout lay = layout(p, M);
    hipStream_t s = (hipStream_t)stream;
    float *lg = logits ? logits : at<float>(ws, lay.logits);
    if (!logits_in) {
        float *sc = nullptr;
        if (L.eps > 0.f) {
            sc = at<float>(ws, lay.tok_scale);
            LAUNCH(moe::launch_rms_scale(L, x, M, sc, s), "rms scale");
        }
        LAUNCH(moe::launch_router(L, x, router_w(p, wts), sc, M, lg, s), "router");
    }
    LAUNCH(moe::launch_topk(L, lg, wts->bias, M, ids, w, s), "top-k");
    return MOE_OK;
}

moe_status moe_permute(const moe_plan *p, const int32_t *ids, int32_t M, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_routes, int32_t *route_pos, void *ws,
                       size_t ws_bytes, void *stream) {
    TRY(check_call(p, M, ws, ws_bytes));
    if (M == 0) return MOE_OK;
    TRY(need_ptr(ids, 4, "ids"));
    TRY(need_ptr(counts, 4, "counts"));
    TRY(need_ptr(offsets, 4, "offsets"));
    TRY(need_ptr(sorted_routes, 4, "sorted_routes"));
    TRY(need_ptr(route_pos, 4, "route_pos"));
    const WsLayout lay = layout(p, M);
    LAUNCH(moe::launch_permute(p->L.E, M * p->L.k, moe::mfma_tile_rows(), ids, counts, offsets,
                               sorted_routes, route_pos, at<int32_t>(ws, lay.active),
                               lay.max_tiles ? at<int32_t>(ws, lay.tiles) : nullptr, (hipStream_t)stream),
           "permute");
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_plan *p, const void *x, const moe_weights *wts, int32_t M,
                          const int32_t *offsets, const int32_t *sorted_routes, float *act,
                          void *ws, size_t ws_bytes, void *stream) {
    TRY(check_call(p, M, ws, ws_bytes));
    if (M == 0) return MOE_OK;
    TRY(need_ptr(x, 16, "x"));
    TRY(check_experts(p, wts, true, false, false));
    TRY(need_ptr(offsets, 4, "offsets"));
    TRY(need_ptr(sorted_routes, 4, "sorted_routes"));
    TRY(need_ptr(act, 16, "act"));
    const moe::Layer &L = p->L;
    const WsLayout lay = layout(p, M);
    hipStream_t s = (hipStream_t)stream;
    int32_t *active = at<int32_t>(ws, lay.active);
    int32_t *tiles = lay.max_tiles ? at<int32_t>(ws, lay.tiles) : nullptr;
    LAUNCH(moe::launch_plan_from_offsets(L.E, moe::mfma_tile_rows(), offsets, active, tiles, s), "plan");
    float *sc = nullptr;
    if (L.eps > 0.f) {
        sc = at<float>(ws, lay.tok_scale);
        LAUNCH(moe::launch_rms_scale(L, x, M, sc, s), "rms scale");
    }
    const moe::Routing rt{offsets, sorted_routes, nullptr, active, tiles};
    const moe::Mats none{};
    if (use_mfma(p, M))
        LAUNCH(moe::launch_gateup_mfma(L, x, sc, routed_mats(wts), none, rt, M, lay.max_tiles, moe::mfma_tile_rows(),
                                       act, nullptr, moe::ACT_F32, s),
               "gate/up (MFMA)");
    else
        LAUNCH(moe::launch_gateup_gemv(L, x, sc, routed_mats(wts), none, rt, M, act, nullptr, s), "gate/up");
    return MOE_OK;
}

moe_status moe_combine(const moe_plan *p, const float *act, const moe_weights *wts, int32_t M,
                       const int32_t *offsets, const int32_t *sorted_routes,
                       const int32_t *route_pos, const float *w, const float *seed, float *y,
                       void *ws, size_t ws_bytes, void *stream) {
    TRY(check_call(p, M, ws, ws_bytes));
    if (M == 0) return MOE_OK;
    TRY(need_ptr(act, 16, "act"));
    TRY(check_experts(p, wts, false, true, false));
    TRY(need_ptr(offsets, 4, "offsets"));
    TRY(need_ptr(sorted_routes, 4, "sorted_routes"));
    TRY(need_ptr(route_pos, 4, "route_pos"));
    TRY(need_ptr(w, 4, "w"));
    if (seed) TRY(need_ptr(seed, 16, "seed"));
    TRY(need_ptr(y, 16, "y"));
    if ((const void *)y == (const void *)act) return fail(MOE_ERR_INVALID, "y aliases act");
    const moe::Layer &L = p->L;
    const WsLayout lay = layout(p, M);
    hipStream_t s = (hipStream_t)stream;
    int32_t *active = at<int32_t>(ws, lay.active);
    int32_t *tiles = lay.max_tiles ? at<int32_t>(ws, lay.tiles) : nullptr;
    LAUNCH(moe::launch_plan_from_offsets(L.E, moe::mfma_tile_rows(), offsets, active, tiles, s), "plan");
    const moe::Routing rt{offsets, sorted_routes, route_pos, active, tiles};
    const moe::Mats none{};
    // (the fp32-act grouped GEMM reads bf16 weights only)
    if (use_mfma(p, M) && L.edt == moe::DT_BF16) {
        float *yr = at<float>(ws, lay.y_routes);
        LAUNCH(moe::launch_down_mfma(L, act, nullptr, routed_mats(wts), none, rt, M, lay.max_tiles, moe::mfma_tile_rows(),
                                     yr, nullptr, moe::ACT_F32, s),
               "down (MFMA)");
        LAUNCH(moe::launch_combine(L, yr, nullptr, route_pos, w, seed, M, y, s,
                                   moe::down_ksplit(L, M, moe::mfma_tile_rows()), 0),
               "combine");
    } else {
        float *yr = at<float>(ws, lay.y_routes);
        LAUNCH(moe::launch_down_gemv(L, act, nullptr, routed_mats(wts), none, rt, M, yr, nullptr, s), "down");
        LAUNCH(moe::launch_combine(L, yr, nullptr, route_pos, w, seed, M, y, s, moe::down_gemv_slices(L.I, L.edt), 0),
               "combine");
    }
    return MOE_OK;
}

// Per-stage timing for moe_forward_timed: events[2i] and events[2i+1] bracket
// the kernels of the i-th stage that launched any (see moe::StageTimer).
struct Recorder {
    hipEvent_t *events = nullptr;
    int max_events = 0, n = 0;
    int32_t *stages = nullptr;
    ~Recorder() {
        if (events) moe::stage_timer() = moe::StageTimer{};
    }
    moe_status arm() {
        if (!events) return MOE_OK;
        if (2 * n + 1 >= max_events) return fail(MOE_ERR_INVALID, "too few timing events");
        moe::stage_timer() = moe::StageTimer{events[2 * n], events[2 * n + 1], 0};
        return MOE_OK;
    }
    void after(int stage) {
        if (!events) return;
        moe::StageTimer &t = moe::stage_timer();
        const bool launched = t.launches > 0;
        t = moe::StageTimer{};
        if (!launched) return;
        if (stages) stages[n] = stage;
        n++;
    }
};

#define STAGE(rec, expr, what, stage)               \
    do {                                            \
        TRY((rec).arm());                           \
        LAUNCH(expr, what);                         \
        (rec).after(stage);                         \
    } while (0)

// norm_w ([H] like x, or null) weights the pre-norm, which must be on;
// residual ([M][H] fp32, or null; may be y) seeds the combine.
static moe_status forward_impl(const moe_plan *p, const void *x, const moe_weights *wts, int32_t M,
                               float *y, int32_t *ids_out, float *w_out, int32_t *counts_out,
                               void *ws, size_t ws_bytes, hipStream_t s, Recorder &rec,
                               const void *norm_w = nullptr, const float *residual = nullptr) {
    TRY(check_call(p, M, ws, ws_bytes));
    if (M == 0) return MOE_OK;
    TRY(need_ptr(x, 16, "x"));
    if (norm_w) {
        if (!(p->L.eps > 0.f))
            return fail(MOE_ERR_INVALID, "a norm weight needs the pre-norm on (rms_eps > 0)");
        TRY(need_ptr(norm_w, 16, "norm_weight"));
    }
    if (residual) TRY(need_ptr(residual, 16, "residual"));
    TRY(check_router(p, wts, true));
    TRY(check_experts(p, wts, true, true, true));
    TRY(need_ptr(y, 16, "y"));
    if (ids_out) TRY(need_ptr(ids_out, 4, "ids_out"));
    if (w_out) TRY(need_ptr(w_out, 4, "w_out"));
    if (counts_out) TRY(need_ptr(counts_out, 4, "counts_out"));
    const WsLayout lay = layout(p, M);
    const bool mfma = use_mfma(p, M);
    // L: what the kernels see.  With a norm weight the normed rows are
    // written once (fp32; on the grouped-GEMM path also split bf16 for the
    // router and fp16 for the experts, as the pages keep the normed rows) and the rest
    // of the layer reads them as fp32 x with the pre-norm done.
    moe::Layer L = p->L;
    float *sc = nullptr;
    uint16_t *xsplit = nullptr, *xhalf = nullptr;
    // the grouped-GEMM router on bf16 rows; without a norm weight it also
    // sums the squares of x for the pre-norm, and the top-k forms the scale
    // one expert (k = 1): every route is expert 0 with weight 1 whatever its
    // logit, so no router runs
    const bool one = L.E == 1;
    const bool mfma_router = mfma && !one && L.rdt == moe::DT_BF16 && !wts->router_x_scale;
    const bool rms_in_router = mfma_router && L.eps > 0.f && !norm_w && L.xdt == moe::DT_BF16;
    if (L.eps > 0.f) {
        sc = at<float>(ws, lay.tok_scale);
        if (!rms_in_router) STAGE(rec, moe::launch_rms_scale(L, x, M, sc, s), "rms scale", MOE_STAGE_RMS);
        if (norm_w) {
            float *xn = at<float>(ws, lay.xn);
            xsplit = mfma ? at<uint16_t>(ws, lay.xs) : nullptr;
            xhalf = mfma ? at<uint16_t>(ws, lay.xh) : nullptr;
            STAGE(rec, moe::launch_norm_apply(L, x, norm_w, sc, M, xn, xsplit, xhalf, s), "norm", MOE_STAGE_RMS);
            x = xn;
            sc = nullptr;
            L.xdt = moe::DT_F32;
            L.eps = 0.f;
        }
    }
    float *lg = at<float>(ws, lay.logits);
    int32_t *ids = ids_out ? ids_out : at<int32_t>(ws, lay.ids);
    float *w = w_out ? w_out : at<float>(ws, lay.w);
    int32_t *counts = counts_out ? counts_out : at<int32_t>(ws, lay.counts);
    int32_t *offsets = at<int32_t>(ws, lay.offsets);
    int32_t *sorted = at<int32_t>(ws, lay.sorted);
    int32_t *rpos = at<int32_t>(ws, lay.route_pos);
    int32_t *active = at<int32_t>(ws, lay.active);
    int32_t *tiles = lay.max_tiles ? at<int32_t>(ws, lay.tiles) : nullptr;
    const int rows = moe::mfma_tile_rows(L, M); // tile height of the grouped GEMMs
    const bool single = M == 1 && !mfma && moe::m1_supported(L);
    // small batches on the streamed gate/up kernel: it runs the selection in
    // its prologue, so only the router runs before it
    const bool fuse_sel = !single && !mfma && !one && M <= moe::route_small_max_tokens() &&
                          moe::gateup_stream_selects(L, M, L.Is > 0);
    if (single) {
        // one token: the gate/up kernel runs the top-k itself from the logits
        if (!one)
            STAGE(rec, moe::launch_router_small(L, x, router_w(p, wts), sc, M, lg, s), "router", MOE_STAGE_ROUTER);
    } else if (one) {
        STAGE(rec, moe::launch_route_one(M, rows, ids, w, counts, offsets, sorted, rpos, active, tiles, s),
              "route (one expert)", MOE_STAGE_ROUTER);
    } else if (fuse_sel) {
        STAGE(rec, moe::launch_router_small(L, x, router_w(p, wts), sc, M, lg, s), "router", MOE_STAGE_ROUTER);
    } else if (M <= moe::route_small_max_tokens() && !mfma) {
        STAGE(rec, moe::launch_route_small(L, x, router_w(p, wts), wts->bias, sc, M, lg, ids, w, counts, offsets,
                                           sorted, rpos, active, s),
              "route", MOE_STAGE_ROUTER);
    } else {
        // (the MFMA router takes bf16 rows and no input scale, and leaves the
        // token scale to the top-k; otherwise the GEMV router)
        const float *part = lg, *part_scale = nullptr;
        float *sqp = nullptr;
        int S = 1;
        if (mfma_router && (L.xdt == moe::DT_BF16 || xsplit)) {
            S = moe::router_slices(L, M);
            float *pw = at<float>(ws, lay.y_routes);
            part = pw;
            if (rms_in_router) sqp = pw + (size_t)S * M * L.E;
            else part_scale = sc;
            STAGE(rec, moe::launch_router_mfma(L, xsplit ? (const void *)xsplit : x, wts->router, M, pw, S, sqp, s,
                                               xsplit != nullptr),
                  "router (MFMA)", MOE_STAGE_ROUTER);
        } else {
            STAGE(rec, moe::launch_router(L, x, router_w(p, wts), sc, M, lg, s), "router", MOE_STAGE_ROUTER);
        }
        int32_t *hist = at<int32_t>(ws, lay.hist);
        STAGE(rec, moe::launch_topk_hist(L, part, S, part_scale, wts->bias, M, ids, w, hist, s, sqp,
                                         sqp ? sc : nullptr),
              "top-k", MOE_STAGE_TOPK);
        STAGE(rec, moe::launch_scatter(L.E, M, L.k, rows, ids, hist, counts, offsets, sorted, rpos, active, tiles, s),
              "permute", MOE_STAGE_PERMUTE);
    }
    const moe::Routing rt{offsets, sorted, rpos, active, tiles};
    float *act = at<float>(ws, lay.act);
    float *sact = L.Is > 0 ? at<float>(ws, lay.shared_act) : nullptr;
    float *yr = at<float>(ws, lay.y_routes);
    float *ysh = L.Is > 0 ? at<float>(ws, lay.y_shared) : nullptr;
    if (mfma) {
        STAGE(rec, moe::launch_gateup_mfma(L, xhalf ? (const void *)xhalf : x, sc, routed_mats(wts),
                                           shared_mats(wts), rt, M, lay.max_tiles, rows, act, sact, moe::ACT_F16, s,
                                           xhalf != nullptr),
              "gate/up (MFMA)", MOE_STAGE_GATEUP);
        STAGE(rec, moe::launch_down_mfma(L, act, sact, routed_mats(wts), shared_mats(wts), rt, M,
                                         lay.max_tiles, rows, yr, ysh, moe::ACT_F16, s),
              "down (MFMA)", MOE_STAGE_DOWN);
        STAGE(rec, moe::launch_combine(L, yr, ysh, rpos, w, residual, M, y, s, moe::down_ksplit(L, M, rows), 1),
              "combine", MOE_STAGE_COMBINE);
    } else if (single) {
        STAGE(rec, moe::launch_gateup_m1(L, x, sc, routed_mats(wts), shared_mats(wts), one ? nullptr : lg,
                                         wts->bias, ids, w,
                                         counts_out, act, sact, s),
              "top-k + gate/up", MOE_STAGE_GATEUP);
        STAGE(rec, moe::launch_down_m1(L, act, sact, routed_mats(wts), shared_mats(wts), ids, w, residual, y, s),
              "down + combine", MOE_STAGE_DOWN);
    } else {
        const moe::SelectSmall sel{lg, L.bias_mode ? wts->bias : nullptr, M, L.E, L.k, L.select, L.bias_mode,
                                   ids, w, counts, offsets, sorted, rpos, active};
        STAGE(rec, moe::launch_gateup_gemv(L, x, sc, routed_mats(wts), shared_mats(wts), rt, M, act, sact, s,
                                           fuse_sel ? &sel : nullptr),
              "gate/up", MOE_STAGE_GATEUP);
        STAGE(rec, moe::launch_down_gemv(L, act, sact, routed_mats(wts), shared_mats(wts), rt, M, yr, ysh, s),
              "down", MOE_STAGE_DOWN);
        STAGE(rec, moe::launch_combine(L, yr, ysh, rpos, w, residual, M, y, s, moe::down_gemv_slices(L.I, L.edt),
                                       moe::down_gemv_slices(L.Is, L.sdt)),
              "combine", MOE_STAGE_COMBINE);
    }
    return MOE_OK;
}

moe_status moe_forward(const moe_plan *p, const void *x, const moe_weights *wts, int32_t M,
                       float *y, int32_t *ids_out, float *w_out, int32_t *counts_out, void *ws,
                       size_t ws_bytes, void *stream) {
    Recorder rec;
    return forward_impl(p, x, wts, M, y, ids_out, w_out, counts_out, ws, ws_bytes, (hipStream_t)stream, rec);
}

moe_status moe_forward_noalloc(const moe_plan *p, const void *x, const moe_weights *wts, int32_t M,
                               float *y, int32_t *ids_out, float *w_out, int32_t *counts_out,
                               void *stream) {
    if (!p) return fail(MOE_ERR_INVALID, "plan is NULL");
    if (M < 0 || M > p->cfg.max_tokens)
        return fail(MOE_ERR_INVALID, "M = %d outside 0..max_tokens (%d)", M, p->cfg.max_tokens);
    if (M == 0) return MOE_OK;
    const size_t need = layout(p, M).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "M = %d needs %zu bytes of workspace; the static scratch holds %zu "
                    "(call moe_forward with a workspace)", M, need, kScratchBytes);
    void *ws = nullptr;
    TRY(device_scratch(&ws));
    Recorder rec;
    return forward_impl(p, x, wts, M, y, ids_out, w_out, counts_out, ws, kScratchBytes, (hipStream_t)stream, rec);
}

moe_status moe_forward_fused(const moe_plan *p, const void *x, const void *norm_weight,
                             const float *residual, const moe_weights *wts, int32_t M, float *y,
                             int32_t *ids_out, float *w_out, int32_t *counts_out, void *ws, size_t ws_bytes,
                             void *stream) {
    Recorder rec;
    return forward_impl(p, x, wts, M, y, ids_out, w_out, counts_out, ws, ws_bytes, (hipStream_t)stream, rec,
                        norm_weight, residual);
}

moe_status moe_forward_timed(const moe_plan *p, const void *x, const moe_weights *wts, int32_t M,
                             float *y, int32_t *ids_out, float *w_out, int32_t *counts_out, void *ws,
                             size_t ws_bytes, void *stream, void **events, int32_t max_events,
                             int32_t *stages, int32_t *n_stages) {
    if (!events || max_events < 2) return fail(MOE_ERR_INVALID, "timing needs at least two events");
    for (int i = 0; i < max_events; i++)
        if (!events[i]) return fail(MOE_ERR_INVALID, "event %d is NULL", i);
    Recorder rec;
    rec.events = reinterpret_cast<hipEvent_t *>(events);
    rec.max_events = max_events;
    rec.stages = stages;
    moe_status st = forward_impl(p, x, wts, M, y, ids_out, w_out, counts_out, ws, ws_bytes,
                                 (hipStream_t)stream, rec);
    if (n_stages) *n_stages = rec.n;
    return st;
}

int32_t moe_forward_path(const moe_plan *p, int32_t M) {
    if (!p) return fail(MOE_ERR_INVALID, "plan is NULL"), -1;
    if (M < 1 || M > p->cfg.max_tokens)
        return fail(MOE_ERR_INVALID, "M = %d outside [1, %d]", M, p->cfg.max_tokens), -1;
    if (use_mfma(p, M)) return MOE_RUN_MFMA;
    return M == 1 && moe::m1_supported(p->L) ? MOE_RUN_SINGLE : MOE_RUN_GEMV;
}

moe_status moe_q8_0_split(const void *blocks, int64_t rows, int32_t cols, int8_t *qs,
                          uint16_t *scales, void *stream) {
    if (rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_INVALID, "rows %lld, cols %d: need rows >= 0 and cols a positive multiple of 32", (long long)rows, cols);
    if (rows == 0) return MOE_OK;
    TRY(need_ptr(blocks, 2, "blocks"));
    TRY(need_ptr(qs, 4, "qs"));
    TRY(need_ptr(scales, 2, "scales"));
    LAUNCH(moe::launch_q8_split(blocks, rows, cols, qs, scales, (hipStream_t)stream), "Q8_0 split");
    return MOE_OK;
}

moe_status moe_mxfp4_split(const void *blocks, int64_t rows, int32_t cols, uint8_t *codes,
                           uint8_t *scales, void *stream) {
    if (rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_INVALID, "rows %lld, cols %d: need rows >= 0 and cols a positive multiple of 32", (long long)rows, cols);
    if (rows == 0) return MOE_OK;
    TRY(need_ptr(blocks, 1, "blocks"));
    TRY(need_ptr(codes, 16, "codes"));
    TRY(need_ptr(scales, 1, "scales"));
    LAUNCH(moe::launch_mxfp4_split(blocks, rows, cols, codes, scales, (hipStream_t)stream), "MXFP4 split");
    return MOE_OK;
}

} // extern "C"

// ---------------------------------------------------------------- Q8_0 split
namespace moe {

// One thread per block: 2-byte scale, then 32 int8 written as 8 dwords.
__global__ __launch_bounds__(256) void k_q8_split(const uint16_t *blocks, int64_t nblocks, int8_t *qs,
                                                  uint16_t *scales) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const uint16_t *src = blocks + b * 17; // 34 bytes = 17 halfwords
    scales[b] = src[0];
    uint32_t *dst = reinterpret_cast<uint32_t *>(qs + b * 32);
#pragma unroll
    for (int i = 0; i < 8; i++) dst[i] = (uint32_t)src[1 + 2 * i] | ((uint32_t)src[2 + 2 * i] << 16);
}

hipError_t launch_q8_split(const void *blocks, int64_t rows, int cols, int8_t *qs, uint16_t *scales,
                           hipStream_t s) {
    const int64_t nb = rows * (cols / 32);
    launch_kernel(k_q8_split, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t *>(blocks), nb, qs, scales);
    return hipGetLastError();
}

} // namespace moe

// ---------------------------------------------------------------- MXFP4 split
namespace moe {

// One thread per block: the E8M0 byte, then the 16 code bytes (as stored:
// element 2j in the low nibble of byte j) written as one 16-byte store.
__global__ __launch_bounds__(256) void k_mxfp4_split(const uint8_t *blocks, int64_t nblocks, uint8_t *codes,
                                                     uint8_t *scales) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const uint8_t *src = blocks + b * 17;
    scales[b] = src[0];
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        w[i] = (uint32_t)src[1 + 4 * i] | ((uint32_t)src[2 + 4 * i] << 8) | ((uint32_t)src[3 + 4 * i] << 16) |
               ((uint32_t)src[4 + 4 * i] << 24);
    reinterpret_cast<u32x4 *>(codes)[b] = u32x4{w[0], w[1], w[2], w[3]};
}

hipError_t launch_mxfp4_split(const void *blocks, int64_t rows, int cols, uint8_t *codes, uint8_t *scales,
                              hipStream_t s) {
    const int64_t nb = rows * (cols / 32);
    launch_kernel(k_mxfp4_split, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s,
                  reinterpret_cast<const uint8_t *>(blocks), nb, codes, scales);
    return hipGetLastError();
}

} // namespace moe
