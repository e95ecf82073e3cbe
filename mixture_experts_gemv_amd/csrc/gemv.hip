// Bandwidth-bound GEMV path of the routed MoE layer (decode and small batches).
//
// gate/up: one workgroup per (touched expert, tile of kPairsPerWG rows of I).
//   The tokens routed to the expert are staged in LDS as fp32, kTB at a time;
//   each wave streams kRowPairs gate rows and the matching up rows with 16-byte
//   loads, dequantising in registers (bf16 -> fp32, Q8_0 q * block scale), and
//   writes act = silu(clamp(g)) * clamp(v) for every staged token.
// down:    one workgroup per tile of rows of H.  For M <= 64 each wave owns kRH
//   output rows and loops over every touched expert in ascending id (then the
//   shared expert), so every y element is summed by one wave in a fixed order:
//   no atomics, bitwise-repeatable.  Lane t accumulates token t.
//   For M > 64 the per-route results go to y_routes and a combine kernel sums
//   them in slot order.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowPairs = 2;                         // gate/up row pairs per wave pass
constexpr int kPairsPerWave = 4;
constexpr int kPairsPerWG = kWaves * kPairsPerWave;  // rows of I per workgroup

struct GateUpArgs {
    const void *x;
    const float *tok_scale;
    Mats routed, shared;
    const int32_t *offsets, *sorted, *active;
    int M, H, k, I, Is;
    int seg_routed;  // workgroup slots for routed experts (>= touched experts)
    int tiles_I, tiles_Is;
    float limit;
    float *act, *shared_act;
};

template <int XDT>
__device__ __forceinline__ void stage_token(const void *x, int t, int H, float *dst, float scale) {
    if constexpr (XDT == DT_BF16) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(x) + (size_t)t * H);
        for (int c = threadIdx.x; c < H / 8; c += kThreads) {
            u32x4 q = src[c];
            f32x4 a = {bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y)};
            f32x4 b = {bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w)};
            reinterpret_cast<f32x4 *>(dst)[2 * c] = a * scale;
            reinterpret_cast<f32x4 *>(dst)[2 * c + 1] = b * scale;
        }
    } else {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(x) + (size_t)t * H);
        for (int c = threadIdx.x; c < H / 4; c += kThreads) reinterpret_cast<f32x4 *>(dst)[c] = src[c] * scale;
    }
}

template <int XDT, int WDT, int TB>
__global__ __launch_bounds__(kThreads) void k_gateup_gemv(GateUpArgs a) {
    extern __shared__ float xs[]; // [TB][H]
    constexpr int N = Chunk<WDT>::N;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int H = a.H;

    // ---- which rows of which expert this workgroup owns
    int b = blockIdx.x;
    const void *gbase, *ubase;
    const uint16_t *gsb = nullptr, *usb = nullptr;
    int width, row0, ntok, p0 = 0;
    bool is_shared;
    if (b < a.seg_routed * a.tiles_I) {
        const int u = b / a.tiles_I;
        if (u >= a.active[0]) return;
        const int e = a.active[1 + u];
        width = a.I;
        row0 = (b % a.tiles_I) * kPairsPerWG;
        p0 = a.offsets[e];
        ntok = a.offsets[e + 1] - p0;
        const size_t mat = (size_t)e * a.I * H;
        gbase = reinterpret_cast<const char *>(a.routed.gate) + mat * elem_bytes<WDT>();
        ubase = reinterpret_cast<const char *>(a.routed.up) + mat * elem_bytes<WDT>();
        if constexpr (WDT == DT_Q8) {
            gsb = a.routed.gate_s + mat / 32;
            usb = a.routed.up_s + mat / 32;
        }
        is_shared = false;
    } else {
        b -= a.seg_routed * a.tiles_I;
        width = a.Is;
        row0 = b * kPairsPerWG;
        ntok = a.M;
        gbase = a.shared.gate;
        ubase = a.shared.up;
        if constexpr (WDT == DT_Q8) {
            gsb = a.shared.gate_s;
            usb = a.shared.up_s;
        }
        is_shared = true;
    }
    const size_t row_bytes = (size_t)H * elem_bytes<WDT>();

    for (int tok0 = 0; tok0 < ntok; tok0 += TB) {
        __syncthreads();
#pragma unroll
        for (int tb = 0; tb < TB; tb++) {
            if (tok0 + tb < ntok) {
                const int t = is_shared ? tok0 + tb : a.sorted[p0 + tok0 + tb] / a.k;
                const float sc = a.tok_scale ? a.tok_scale[t] : 1.0f;
                stage_token<XDT>(a.x, t, H, xs + tb * H, sc);
            } else {
                for (int c = threadIdx.x; c < H; c += kThreads) xs[tb * H + c] = 0.f;
            }
        }
        __syncthreads();

        for (int q = 0; q < kPairsPerWave; q += kRowPairs) {
            const int ib = row0 + wave * kPairsPerWave + q;
            if (ib >= width) break; // uniform per wave
            const char *grow[kRowPairs], *urow[kRowPairs];
            const uint16_t *gsr[kRowPairs], *usr[kRowPairs];
#pragma unroll
            for (int r = 0; r < kRowPairs; r++) {
                const int i = min(ib + r, width - 1);
                grow[r] = reinterpret_cast<const char *>(gbase) + (size_t)i * row_bytes;
                urow[r] = reinterpret_cast<const char *>(ubase) + (size_t)i * row_bytes;
                if constexpr (WDT == DT_Q8) {
                    gsr[r] = gsb + (size_t)i * (H / 32);
                    usr[r] = usb + (size_t)i * (H / 32);
                }
            }
            float ag[kRowPairs][TB], au[kRowPairs][TB];
#pragma unroll
            for (int r = 0; r < kRowPairs; r++)
#pragma unroll
                for (int tb = 0; tb < TB; tb++) ag[r][tb] = au[r][tb] = 0.f;

            for (int c = lane; c < H / N; c += kWave) {
                float wg[kRowPairs][N], wu[kRowPairs][N];
                float sg[kRowPairs], su[kRowPairs];
#pragma unroll
                for (int r = 0; r < kRowPairs; r++) {
                    load_chunk<WDT>(grow[r], c, wg[r]);
                    load_chunk<WDT>(urow[r], c, wu[r]);
                    if constexpr (WDT == DT_Q8) {
                        sg[r] = f16_bits_to_f32(gsr[r][c >> 1]);
                        su[r] = f16_bits_to_f32(usr[r][c >> 1]);
                    }
                }
#pragma unroll
                for (int tb = 0; tb < TB; tb++) {
                    float xv[N];
#pragma unroll
                    for (int n4 = 0; n4 < N / 4; n4++) {
                        f32x4 v = reinterpret_cast<const f32x4 *>(xs + tb * H + c * N)[n4];
                        xv[4 * n4] = v.x; xv[4 * n4 + 1] = v.y; xv[4 * n4 + 2] = v.z; xv[4 * n4 + 3] = v.w;
                    }
#pragma unroll
                    for (int r = 0; r < kRowPairs; r++) {
                        float pg = 0.f, pu = 0.f;
#pragma unroll
                        for (int n = 0; n < N; n++) {
                            pg = fmaf(wg[r][n], xv[n], pg);
                            pu = fmaf(wu[r][n], xv[n], pu);
                        }
                        if constexpr (WDT == DT_Q8) {
                            ag[r][tb] = fmaf(sg[r], pg, ag[r][tb]);
                            au[r][tb] = fmaf(su[r], pu, au[r][tb]);
                        } else {
                            ag[r][tb] += pg;
                            au[r][tb] += pu;
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < kRowPairs; r++) {
#pragma unroll
                for (int tb = 0; tb < TB; tb++) {
                    float g = wave_sum(ag[r][tb]);
                    float v = wave_sum(au[r][tb]);
                    if (a.limit > 0.f) {
                        g = clampf(g, a.limit);
                        v = clampf(v, a.limit);
                    }
                    const int i = ib + r;
                    if (lane == 0 && i < width && tok0 + tb < ntok) {
                        const float h = silu_mul(g, v);
                        if (is_shared)
                            a.shared_act[(size_t)(tok0 + tb) * a.Is + i] = h;
                        else
                            a.act[(size_t)(p0 + tok0 + tb) * a.I + i] = h;
                    }
                }
            }
        }
    }
}

template <int XDT, int WDT>
static void gateup_dispatch(const GateUpArgs &a, int grid, int tb, size_t lds, hipStream_t s) {
    if (tb == 1)
        launch_kernel((k_gateup_gemv<XDT, WDT, 1>), dim3(grid), dim3(kThreads), lds, s, a);
    else
        launch_kernel((k_gateup_gemv<XDT, WDT, 4>), dim3(grid), dim3(kThreads), lds, s, a);
}

hipError_t launch_gateup_gemv(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                              const Mats &shared, const Routing &rt, int M, float *act,
                              float *shared_act, hipStream_t s) {
    GateUpArgs a;
    a.x = x;
    a.tok_scale = tok_scale;
    a.routed = routed;
    a.shared = shared;
    a.offsets = rt.offsets;
    a.sorted = rt.sorted;
    a.active = rt.active;
    a.M = M;
    a.H = L.H;
    a.k = L.k;
    a.I = L.I;
    a.Is = shared_act ? L.Is : 0;
    a.seg_routed = act ? (L.E < M * L.k ? L.E : M * L.k) : 0;
    a.tiles_I = (L.I + kPairsPerWG - 1) / kPairsPerWG;
    a.tiles_Is = (a.Is + kPairsPerWG - 1) / kPairsPerWG;
    a.limit = L.limit;
    a.act = act;
    a.shared_act = shared_act;
    const int grid = a.seg_routed * a.tiles_I + a.tiles_Is;
    if (grid == 0) return hipSuccess;
    const int tb = (M == 1 || 4 * L.H > 16384) ? 1 : 4;   // staged tokens must fit 64 KB of LDS
    const size_t lds = (size_t)tb * L.H * sizeof(float);
    if (L.xdt == DT_BF16) {
        if (L.edt == DT_BF16) gateup_dispatch<DT_BF16, DT_BF16>(a, grid, tb, lds, s);
        else if (L.edt == DT_Q8) gateup_dispatch<DT_BF16, DT_Q8>(a, grid, tb, lds, s);
        else gateup_dispatch<DT_BF16, DT_F32>(a, grid, tb, lds, s);
    } else {
        if (L.edt == DT_BF16) gateup_dispatch<DT_F32, DT_BF16>(a, grid, tb, lds, s);
        else if (L.edt == DT_Q8) gateup_dispatch<DT_F32, DT_Q8>(a, grid, tb, lds, s);
        else gateup_dispatch<DT_F32, DT_F32>(a, grid, tb, lds, s);
    }
    return hipGetLastError();
}

// -------------------------------------------------------------------- down
constexpr int kRH = 2;                     // output rows per wave
constexpr int kRowsPerWG = kWaves * kRH;   // rows of H per workgroup
constexpr int kDTB = 4;                    // routes per inner step

struct DownArgs {
    const float *act, *shared_act;
    Mats routed, shared;
    const int32_t *offsets, *sorted, *active;
    const float *w, *seed;
    int M, H, k, I, Is;
    float *y;
    float *y_routes, *y_shared; // unfused form
    int seg_routed;             // unfused: workgroup slots for routed experts
    int tiles_H;                // unfused: row tiles of H per segment
};

// dot[r][tb] = sum_i down_row_r[i] * act_tb[i] over one expert's rows, for
// kDTB consecutive act rows starting at arow (rows past n are skipped).
template <int WDT>
__device__ __forceinline__ void down_dots(const char *const *drow, const uint16_t *const *dsr, int width,
                                          const float *arow, int n, int lane, float (&dot)[kRH][kDTB]) {
    constexpr int N = Chunk<WDT>::N;
#pragma unroll
    for (int r = 0; r < kRH; r++)
#pragma unroll
        for (int tb = 0; tb < kDTB; tb++) dot[r][tb] = 0.f;
    for (int c = lane; c < width / N; c += kWave) {
        float wd[kRH][N], sd[kRH];
#pragma unroll
        for (int r = 0; r < kRH; r++) {
            load_chunk<WDT>(drow[r], c, wd[r]);
            if constexpr (WDT == DT_Q8) sd[r] = f16_bits_to_f32(dsr[r][c >> 1]);
        }
#pragma unroll
        for (int tb = 0; tb < kDTB; tb++) {
            if (tb < n) {
                float av[N];
#pragma unroll
                for (int n4 = 0; n4 < N / 4; n4++) {
                    f32x4 v = reinterpret_cast<const f32x4 *>(arow + (size_t)tb * width + c * N)[n4];
                    av[4 * n4] = v.x; av[4 * n4 + 1] = v.y; av[4 * n4 + 2] = v.z; av[4 * n4 + 3] = v.w;
                }
#pragma unroll
                for (int r = 0; r < kRH; r++) {
                    float p = 0.f;
#pragma unroll
                    for (int i = 0; i < N; i++) p = fmaf(wd[r][i], av[i], p);
                    if constexpr (WDT == DT_Q8) dot[r][tb] = fmaf(sd[r], p, dot[r][tb]);
                    else dot[r][tb] += p;
                }
            }
        }
    }
}

// Fused down + combine for M <= 64.
template <int WDT>
__global__ __launch_bounds__(kThreads) void k_down_combine_gemv(DownArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int H = a.H;
    const int h0 = (blockIdx.x * kWaves + wave) * kRH;
    if (h0 >= H) return;
    float yacc[kRH];
    int hr[kRH];
#pragma unroll
    for (int r = 0; r < kRH; r++) {
        hr[r] = min(h0 + r, H - 1);
        yacc[r] = (a.seed && lane < a.M) ? a.seed[(size_t)lane * H + hr[r]] : 0.f;
    }
    const char *drow[kRH];
    const uint16_t *dsr[kRH];
    float dot[kRH][kDTB];
    // shared expert: weight 1, route = token
    if (a.Is > 0) {
#pragma unroll
        for (int r = 0; r < kRH; r++) {
            drow[r] = reinterpret_cast<const char *>(a.shared.down) + (size_t)hr[r] * a.Is * elem_bytes<WDT>();
            if constexpr (WDT == DT_Q8) dsr[r] = a.shared.down_s + (size_t)hr[r] * (a.Is / 32);
        }
        for (int t0 = 0; t0 < a.M; t0 += kDTB) {
            const int n = min(kDTB, a.M - t0);
            down_dots<WDT>(drow, dsr, a.Is, a.shared_act + (size_t)t0 * a.Is, n, lane, dot);
#pragma unroll
            for (int tb = 0; tb < kDTB; tb++)
                if (tb < n) {
#pragma unroll
                    for (int r = 0; r < kRH; r++) {
                        const float d = wave_sum(dot[r][tb]);
                        if (lane == t0 + tb) yacc[r] += d;
                    }
                }
        }
    }
    const int n_active = a.active[0];
    for (int u = 0; u < n_active; u++) {
        const int e = a.active[1 + u];
        const int p0 = a.offsets[e], p1 = a.offsets[e + 1];
#pragma unroll
        for (int r = 0; r < kRH; r++) {
            const size_t row = (size_t)e * H + hr[r];
            drow[r] = reinterpret_cast<const char *>(a.routed.down) + row * a.I * elem_bytes<WDT>();
            if constexpr (WDT == DT_Q8) dsr[r] = a.routed.down_s + row * (a.I / 32);
        }
        for (int p = p0; p < p1; p += kDTB) {
            const int n = min(kDTB, p1 - p);
            down_dots<WDT>(drow, dsr, a.I, a.act + (size_t)p * a.I, n, lane, dot);
#pragma unroll
            for (int tb = 0; tb < kDTB; tb++)
                if (tb < n) {
                    const int route = a.sorted[p + tb];
                    const int t = route / a.k;
                    const float wt = a.w[route];
#pragma unroll
                    for (int r = 0; r < kRH; r++) {
                        const float d = wave_sum(dot[r][tb]);
                        if (lane == t) yacc[r] = fmaf(wt, d, yacc[r]);
                    }
                }
        }
    }
    if (lane < a.M) {
#pragma unroll
        for (int r = 0; r < kRH; r++)
            if (h0 + r < H) a.y[(size_t)lane * H + h0 + r] = yacc[r];
    }
}

// Unfused down for M > 64: y_routes[p][h] and y_shared[t][h].
template <int WDT>
__global__ __launch_bounds__(kThreads) void k_down_routes_gemv(DownArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int H = a.H;
    int b = blockIdx.x;
    int width, p0, n_rows;
    const char *dbase;
    const uint16_t *dsb = nullptr;
    const float *abase;
    float *out;
    if (b < a.seg_routed * a.tiles_H) {
        const int u = b / a.tiles_H;
        if (u >= a.active[0]) return;
        const int e = a.active[1 + u];
        b %= a.tiles_H;
        width = a.I;
        p0 = a.offsets[e];
        n_rows = a.offsets[e + 1] - p0;
        dbase = reinterpret_cast<const char *>(a.routed.down) + (size_t)e * H * a.I * elem_bytes<WDT>();
        if constexpr (WDT == DT_Q8) dsb = a.routed.down_s + (size_t)e * H * (a.I / 32);
        abase = a.act;
        out = a.y_routes;
    } else {
        b -= a.seg_routed * a.tiles_H;
        width = a.Is;
        p0 = 0;
        n_rows = a.M;
        dbase = reinterpret_cast<const char *>(a.shared.down);
        if constexpr (WDT == DT_Q8) dsb = a.shared.down_s;
        abase = a.shared_act;
        out = a.y_shared;
    }
    const int h0 = (b * kWaves + wave) * kRH;
    if (h0 >= H) return;
    const char *drow[kRH];
    const uint16_t *dsr[kRH];
#pragma unroll
    for (int r = 0; r < kRH; r++) {
        const int h = min(h0 + r, H - 1);
        drow[r] = dbase + (size_t)h * width * elem_bytes<WDT>();
        if constexpr (WDT == DT_Q8) dsr[r] = dsb + (size_t)h * (width / 32);
    }
    float dot[kRH][kDTB];
    for (int p = 0; p < n_rows; p += kDTB) {
        const int n = min(kDTB, n_rows - p);
        down_dots<WDT>(drow, dsr, width, abase + (size_t)(p0 + p) * width, n, lane, dot);
#pragma unroll
        for (int tb = 0; tb < kDTB; tb++)
            if (tb < n) {
#pragma unroll
                for (int r = 0; r < kRH; r++) {
                    const float d = wave_sum(dot[r][tb]);
                    if (lane == 0 && h0 + r < H) out[(size_t)(p0 + p + tb) * H + h0 + r] = d;
                }
            }
    }
}

static DownArgs down_args(const Layer &L, const float *act, const float *shared_act, const Mats &routed,
                          const Mats &shared, const Routing &rt, const float *w, const float *seed, int M,
                          float *y, float *y_routes, float *y_shared) {
    DownArgs a;
    a.act = act;
    a.shared_act = shared_act;
    a.routed = routed;
    a.shared = shared;
    a.offsets = rt.offsets;
    a.sorted = rt.sorted;
    a.active = rt.active;
    a.w = w;
    a.seed = seed;
    a.M = M;
    a.H = L.H;
    a.k = L.k;
    a.I = L.I;
    a.Is = shared_act ? L.Is : 0;
    a.y = y;
    a.y_routes = y_routes;
    a.y_shared = y_shared;
    a.seg_routed = act ? (L.E < M * L.k ? L.E : M * L.k) : 0;
    a.tiles_H = (L.H + kRowsPerWG - 1) / kRowsPerWG;
    return a;
}

hipError_t launch_down_routes_gemv(const Layer &L, const float *act, const float *shared_act,
                                   const Mats &routed, const Mats &shared, const Routing &rt, int M,
                                   float *y_routes, float *y_shared, hipStream_t s) {
    const DownArgs a = down_args(L, act, shared_act, routed, shared, rt, nullptr, nullptr, M, nullptr,
                                 y_routes, y_shared);
    const dim3 grid(a.seg_routed * a.tiles_H + (a.Is > 0 ? a.tiles_H : 0));
    if (grid.x == 0) return hipSuccess;
    if (L.edt == DT_BF16) launch_kernel(k_down_routes_gemv<DT_BF16>, grid, dim3(kThreads), 0, s, a);
    else if (L.edt == DT_Q8) launch_kernel(k_down_routes_gemv<DT_Q8>, grid, dim3(kThreads), 0, s, a);
    else launch_kernel(k_down_routes_gemv<DT_F32>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_gemv(const Layer &L, const float *act, const float *shared_act,
                            const Mats &routed, const Mats &shared, const Routing &rt,
                            const float *w, const float *seed, int M, float *y, float *y_routes,
                            float *y_shared, hipStream_t s) {
    if (M > kWave) {
        hipError_t err = launch_down_routes_gemv(L, act, shared_act, routed, shared, rt, M, y_routes,
                                                 y_shared, s);
        if (err != hipSuccess) return err;
        return launch_combine(L, y_routes, shared_act ? y_shared : nullptr, rt.route_pos, w, seed, M, y, s);
    }
    const DownArgs a = down_args(L, act, shared_act, routed, shared, rt, w, seed, M, y, y_routes, y_shared);
    const dim3 grid(a.tiles_H);
    if (L.edt == DT_BF16) launch_kernel(k_down_combine_gemv<DT_BF16>, grid, dim3(kThreads), 0, s, a);
    else if (L.edt == DT_Q8) launch_kernel(k_down_combine_gemv<DT_Q8>, grid, dim3(kThreads), 0, s, a);
    else launch_kernel(k_down_combine_gemv<DT_F32>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// ================================================================ M = 1 decode
// With one token every touched expert sees the same x, and the sorted
// position of the route to the u-th touched expert is u.
//
// gate/up: each wave holds x in registers (lane l owns chunks l, l+64, ...)
// and streams a contiguous range of (slot, row) pairs, RP pairs at a time,
// issuing all 2*RP*CPL 16-byte loads of a group before using them.
// Both kernels run the token's top-k from the router logits in their prologue
// (one wave's DPP rounds, overlapped with the first loads), so the single-token
// path needs no routing kernel of its own and no cross-workgroup handoff.
struct M1Route {
    const float *logits, *bias;
    int E, k, select, bias_mode;
};

// Slot -> expert table of the k picks in ascending expert id (wave-uniform).
// (Named fields rather than an array, so the table stays in scalar registers.)
struct M1Slots {
    int e0, e1, e2, e3, e4, e5, e6, e7;
    __device__ int expert(int s) const {
        return s == 0 ? e0 : s == 1 ? e1 : s == 2 ? e2 : s == 3 ? e3 : s == 4 ? e4 : s == 5 ? e5 : s == 6 ? e6 : e7;
    }
    __device__ void set(int s, int v) {
        e0 = s == 0 ? v : e0; e1 = s == 1 ? v : e1; e2 = s == 2 ? v : e2; e3 = s == 3 ? v : e3;
        e4 = s == 4 ? v : e4; e5 = s == 5 ? v : e5; e6 = s == 6 ? v : e6; e7 = s == 7 ? v : e7;
    }
};

__device__ __forceinline__ M1Slots m1_slots(const M1Route &rt, int lane, int *my_id, float *my_w, int *my_rank) {
    topk_wave_core(rt.logits, rt.bias, rt.E, rt.k, rt.select, rt.bias_mode, lane, my_id, my_w);
    *my_rank = pick_rank(*my_id, rt.k, lane);
    M1Slots s{0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < rt.k; j++)
        s.set(__builtin_amdgcn_readlane(*my_rank, j), __builtin_amdgcn_readlane(*my_id, j));
    return s;
}

struct M1GateUpArgs {
    const void *x;
    const float *tok_scale;
    Mats routed, shared;
    M1Route rt;
    int32_t *ids_out, *counts_out; // written by the first wave
    float *w_out;
    int H, I, Is, k;
    int total_pairs, pairs_per_wave;
    float limit;
    float *act, *shared_act;
};

template <int XDT, int WDT, int CPL, int RP>
__global__ __launch_bounds__(kThreads) void k_gateup_m1(M1GateUpArgs a) {
    constexpr int N = Chunk<WDT>::N;
    const int lane = threadIdx.x & 63;
    const int gw = uniform(blockIdx.x * kWaves + (threadIdx.x >> 6));
    const int p_begin = gw * a.pairs_per_wave;
    if (p_begin >= a.total_pairs) return;
    const int p_end = min(a.total_pairs, p_begin + a.pairs_per_wave);
    const int H = a.H, nch = H / N;
    const float sc = a.tok_scale ? a.tok_scale[0] : 1.0f;
    int my_id, my_rank;
    float my_w;
    const M1Slots slots = m1_slots(a.rt, lane, &my_id, &my_w, &my_rank);
    if (gw == 0) {
        if (lane < a.k) {
            a.ids_out[lane] = my_id;
            a.w_out[lane] = my_w;
        }
        if (a.counts_out)
            for (int e = lane; e < a.rt.E; e += kWave) {
                int c = 0;
                for (int u = 0; u < a.k; u++) c += slots.expert(u) == e;
                a.counts_out[e] = c;
            }
    }
    // x chunks this lane multiplies; lanes past the row end hold zeros and
    // load (harmless) duplicates of the last chunk.
    int cl[CPL];
    float xr[CPL][N];
#pragma unroll
    for (int cc = 0; cc < CPL; cc++) {
        const int c = lane + kWave * cc;
        cl[cc] = min(c, nch - 1);
        const float m = c < nch ? sc : 0.f;
#pragma unroll
        for (int n4 = 0; n4 < N; n4 += 4) {
            if constexpr (XDT == DT_BF16) {
                const u32x2 q = reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(a.x) + cl[cc] * N + n4)[0];
                xr[cc][n4] = bf16_lo(q.x) * m; xr[cc][n4 + 1] = bf16_hi(q.x) * m;
                xr[cc][n4 + 2] = bf16_lo(q.y) * m; xr[cc][n4 + 3] = bf16_hi(q.y) * m;
            } else {
                const f32x4 q = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.x) + cl[cc] * N + n4)[0];
                xr[cc][n4] = q.x * m; xr[cc][n4 + 1] = q.y * m; xr[cc][n4 + 2] = q.z * m; xr[cc][n4 + 3] = q.w * m;
            }
        }
    }
    const int routed_pairs = a.k * a.I;
    const size_t row_bytes = (size_t)H * elem_bytes<WDT>();
    for (int p = p_begin; p < p_end; p += RP) {
        const char *grow[RP], *urow[RP];
        const uint16_t *gsr[RP], *usr[RP];
        int slot[RP], irow[RP];
#pragma unroll
        for (int r = 0; r < RP; r++) {
            const int q = min(p + r, p_end - 1);
            size_t row;
            const Mats *m;
            if (q < routed_pairs) {
                slot[r] = q / a.I;
                irow[r] = q - slot[r] * a.I;
                row = (size_t)slots.expert(slot[r]) * a.I + irow[r];
                m = &a.routed;
            } else {
                slot[r] = -1;
                irow[r] = q - routed_pairs;
                row = irow[r];
                m = &a.shared;
            }
            grow[r] = reinterpret_cast<const char *>(m->gate) + row * row_bytes;
            urow[r] = reinterpret_cast<const char *>(m->up) + row * row_bytes;
            if constexpr (WDT == DT_Q8) {
                gsr[r] = m->gate_s + row * (H / 32);
                usr[r] = m->up_s + row * (H / 32);
            }
        }
        // issue every load of the group first
        u32x4 rg[RP][CPL], ru[RP][CPL];
        uint16_t hg[RP][CPL], hu[RP][CPL];
#pragma unroll
        for (int r = 0; r < RP; r++)
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                rg[r][cc] = load_raw(grow[r], cl[cc]);
                ru[r][cc] = load_raw(urow[r], cl[cc]);
                if constexpr (WDT == DT_Q8) {
                    hg[r][cc] = gsr[r][cl[cc] >> 1];
                    hu[r][cc] = usr[r][cl[cc] >> 1];
                }
            }
#pragma unroll
        for (int r = 0; r < RP; r++) {
            float g = 0.f, v = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                float wg[N], wu[N];
                decode_chunk<WDT>(rg[r][cc], wg);
                decode_chunk<WDT>(ru[r][cc], wu);
                float pg = 0.f, pu = 0.f;
#pragma unroll
                for (int n = 0; n < N; n++) {
                    pg = fmaf(wg[n], xr[cc][n], pg);
                    pu = fmaf(wu[n], xr[cc][n], pu);
                }
                if constexpr (WDT == DT_Q8) {
                    g = fmaf(f16_bits_to_f32(hg[r][cc]), pg, g);
                    v = fmaf(f16_bits_to_f32(hu[r][cc]), pu, v);
                } else {
                    g += pg;
                    v += pu;
                }
            }
            g = wave_sum(g);
            v = wave_sum(v);
            if (a.limit > 0.f) {
                g = clampf(g, a.limit);
                v = clampf(v, a.limit);
            }
            if (lane == 0 && p + r < p_end) {
                const float h = silu_mul(g, v);
                if (slot[r] >= 0) a.act[(size_t)slot[r] * a.I + irow[r]] = h;
                else a.shared_act[irow[r]] = h;
            }
        }
    }
}

// down (M = 1): a workgroup owns kM1Rows output rows; its 256 threads stride
// over the concatenated chunks of every touched expert's rows (then the
// shared expert's), kM1Unroll rounds at a time with every load of the rounds
// issued first.  Each chunk's dot is scaled by its route's weight before the
// block reduction, which is done in a fixed order.
constexpr int kM1Rows = 4;
constexpr int kM1Unroll = 2;
constexpr int kMaxSlots = 9; // top-k slots + the shared expert

struct M1DownArgs {
    const float *act, *shared_act;
    Mats routed, shared;
    M1Route rt;
    const float *seed;
    int H, I, Is, k;
    float *y;
};

template <int WDT>
__global__ __launch_bounds__(kThreads) void k_down_m1(M1DownArgs a) {
    constexpr int N = Chunk<WDT>::N;
    __shared__ const char *s_row[kMaxSlots];
    __shared__ const uint16_t *s_sc[kMaxSlots];
    __shared__ const float *s_act[kMaxSlots];
    __shared__ float s_w[kMaxSlots];
    __shared__ int s_width[kMaxSlots];
    __shared__ float s_part[kWaves][kM1Rows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, h0 = blockIdx.x * kM1Rows;
    const int n_routed = a.k; // with M = 1 every slot is a touched expert
    const int nch = a.I / N, nch_s = a.Is / N;
    if (wave == 0) {
        int my_id, my_rank;
        float my_w;
        topk_wave_core(a.rt.logits, a.rt.bias, a.rt.E, a.rt.k, a.rt.select, a.rt.bias_mode, lane, &my_id, &my_w);
        my_rank = pick_rank(my_id, a.k, lane);
        if (lane < n_routed) {
            // slot = rank in ascending expert id, which is the act row of the pick
            const size_t row = (size_t)my_id * H + h0;
            s_row[my_rank] = reinterpret_cast<const char *>(a.routed.down) + row * a.I * elem_bytes<WDT>();
            if constexpr (WDT == DT_Q8) s_sc[my_rank] = a.routed.down_s + row * (a.I / 32);
            s_act[my_rank] = a.act + (size_t)my_rank * a.I;
            s_w[my_rank] = my_w;
            s_width[my_rank] = a.I;
        }
    }
    if (tid == n_routed && a.Is > 0) {
        s_row[tid] = reinterpret_cast<const char *>(a.shared.down) + (size_t)h0 * a.Is * elem_bytes<WDT>();
        if constexpr (WDT == DT_Q8) s_sc[tid] = a.shared.down_s + (size_t)h0 * (a.Is / 32);
        s_act[tid] = a.shared_act;
        s_w[tid] = 1.0f;
        s_width[tid] = a.Is;
    }
    __syncthreads();
    const int n_tasks = n_routed * nch + (a.Is > 0 ? nch_s : 0);
    const int last_row = min(kM1Rows, H - h0) - 1;
    float acc[kM1Rows];
#pragma unroll
    for (int r = 0; r < kM1Rows; r++) acc[r] = 0.f;
    for (int t0 = 0; t0 < n_tasks; t0 += kThreads * kM1Unroll) {
        u32x4 raw[kM1Unroll][kM1Rows];
        uint16_t hs[kM1Unroll][kM1Rows];
        f32x4 av[kM1Unroll][N / 4];
        float wt[kM1Unroll];
#pragma unroll
        for (int u = 0; u < kM1Unroll; u++) {
            const int t = t0 + u * kThreads + tid;
            const int tc = min(t, n_tasks - 1);
            int slot, c;
            if (tc < n_routed * nch) {
                slot = tc / nch;
                c = tc - slot * nch;
            } else {
                slot = n_routed;
                c = tc - n_routed * nch;
            }
            const int width = s_width[slot];
            const size_t rb = (size_t)width * elem_bytes<WDT>();
            const char *row0 = s_row[slot];
            wt[u] = t < n_tasks ? s_w[slot] : 0.f;
#pragma unroll
            for (int r = 0; r < kM1Rows; r++) {
                const int rr = min(r, last_row);
                raw[u][r] = load_raw(row0 + rr * rb, c);
                if constexpr (WDT == DT_Q8) hs[u][r] = s_sc[slot][(size_t)rr * (width / 32) + (c >> 1)];
            }
            const f32x4 *ap = reinterpret_cast<const f32x4 *>(s_act[slot] + c * N);
#pragma unroll
            for (int n4 = 0; n4 < N / 4; n4++) av[u][n4] = ap[n4];
        }
#pragma unroll
        for (int u = 0; u < kM1Unroll; u++) {
#pragma unroll
            for (int r = 0; r < kM1Rows; r++) {
                float wv[N];
                decode_chunk<WDT>(raw[u][r], wv);
                float d = 0.f;
#pragma unroll
                for (int n4 = 0; n4 < N / 4; n4++) {
                    d = fmaf(wv[4 * n4], av[u][n4].x, d);
                    d = fmaf(wv[4 * n4 + 1], av[u][n4].y, d);
                    d = fmaf(wv[4 * n4 + 2], av[u][n4].z, d);
                    d = fmaf(wv[4 * n4 + 3], av[u][n4].w, d);
                }
                if constexpr (WDT == DT_Q8) d *= f16_bits_to_f32(hs[u][r]);
                acc[r] = fmaf(wt[u], d, acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kM1Rows; r++) {
        const float v = wave_sum(acc[r]);
        if (lane == 0) s_part[wave][r] = v;
    }
    __syncthreads();
    if (tid <= last_row) {
        float v = a.seed ? a.seed[h0 + tid] : 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; wv++) v += s_part[wv][tid];
        a.y[h0 + tid] = v;
    }
}

// Chunks per lane of a row of H elements, and the instantiated values.
static int m1_cpl(int H, int N) { return (H / N + kWave - 1) / kWave; }

template <int XDT, int WDT, int RP>
static bool m1_gateup_dispatch(int cpl, const M1GateUpArgs &a, int grid, hipStream_t s) {
#define M1_CASE(C) \
    case C: launch_kernel((k_gateup_m1<XDT, WDT, C, RP>), dim3(grid), dim3(kThreads), 0, s, a); return true;
    switch (cpl) {
        M1_CASE(1) M1_CASE(2) M1_CASE(3) M1_CASE(4) M1_CASE(5) M1_CASE(6) M1_CASE(8)
    default: return false;
    }
#undef M1_CASE
}

bool m1_supported(const Layer &L) {
    const int N = L.edt == DT_Q8 ? 16 : (L.edt == DT_BF16 ? 8 : 4);
    const int c = m1_cpl(L.H, N);
    return c <= 8 && c != 7;
}

static M1Route m1_route(const Layer &L, const float *logits, const float *bias) {
    return M1Route{logits, L.bias_mode ? bias : nullptr, L.E, L.k, L.select, L.bias_mode};
}

hipError_t launch_gateup_m1(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                            const Mats &shared, const float *logits, const float *bias, int32_t *ids_out,
                            float *w_out, int32_t *counts_out, float *act, float *shared_act,
                            hipStream_t s) {
    M1GateUpArgs a;
    a.x = x;
    a.tok_scale = tok_scale;
    a.routed = routed;
    a.shared = shared;
    a.rt = m1_route(L, logits, bias);
    a.ids_out = ids_out;
    a.w_out = w_out;
    a.counts_out = counts_out;
    a.H = L.H;
    a.I = L.I;
    a.Is = shared_act ? L.Is : 0;
    a.k = L.k;
    a.limit = L.limit;
    a.act = act;
    a.shared_act = shared_act;
    a.total_pairs = L.k * L.I + a.Is;
    const int N = L.edt == DT_Q8 ? 16 : (L.edt == DT_BF16 ? 8 : 4);
    const int cpl = m1_cpl(L.H, N);
    const int RP = cpl <= 4 ? 2 : 1; // keep about 16 loads of a group in flight
    const int max_waves = 2048;
    int ppw = (a.total_pairs + max_waves - 1) / max_waves;
    ppw = (ppw + RP - 1) / RP * RP;
    a.pairs_per_wave = ppw;
    const int waves = (a.total_pairs + ppw - 1) / ppw;
    const int grid = (waves + kWaves - 1) / kWaves;
    bool ok;
    if (L.xdt == DT_BF16) {
        if (L.edt == DT_Q8) ok = RP == 2 ? m1_gateup_dispatch<DT_BF16, DT_Q8, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_BF16, DT_Q8, 1>(cpl, a, grid, s);
        else if (L.edt == DT_BF16) ok = RP == 2 ? m1_gateup_dispatch<DT_BF16, DT_BF16, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_BF16, DT_BF16, 1>(cpl, a, grid, s);
        else ok = RP == 2 ? m1_gateup_dispatch<DT_BF16, DT_F32, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_BF16, DT_F32, 1>(cpl, a, grid, s);
    } else {
        if (L.edt == DT_Q8) ok = RP == 2 ? m1_gateup_dispatch<DT_F32, DT_Q8, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_F32, DT_Q8, 1>(cpl, a, grid, s);
        else if (L.edt == DT_BF16) ok = RP == 2 ? m1_gateup_dispatch<DT_F32, DT_BF16, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_F32, DT_BF16, 1>(cpl, a, grid, s);
        else ok = RP == 2 ? m1_gateup_dispatch<DT_F32, DT_F32, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_F32, DT_F32, 1>(cpl, a, grid, s);
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_down_m1(const Layer &L, const float *act, const float *shared_act, const Mats &routed,
                          const Mats &shared, const float *logits, const float *bias, const float *seed,
                          float *y, hipStream_t s) {
    M1DownArgs a;
    a.act = act;
    a.shared_act = shared_act;
    a.routed = routed;
    a.shared = shared;
    a.rt = m1_route(L, logits, bias);
    a.seed = seed;
    a.H = L.H;
    a.I = L.I;
    a.Is = shared_act ? L.Is : 0;
    a.k = L.k;
    a.y = y;
    const dim3 grid((L.H + kM1Rows - 1) / kM1Rows);
    if (L.edt == DT_BF16) launch_kernel(k_down_m1<DT_BF16>, grid, dim3(kThreads), 0, s, a);
    else if (L.edt == DT_Q8) launch_kernel(k_down_m1<DT_Q8>, grid, dim3(kThreads), 0, s, a);
    else launch_kernel(k_down_m1<DT_F32>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// -------------------------------------------------------------------- combine
// One thread per (token, 4 consecutive h); slots summed in order j = 0..k-1,
// each slot's partial slices (a split reduction) summed in slice order first.
__global__ __launch_bounds__(256) void k_combine(const float *y_routes, const float *y_shared,
                                                 const int32_t *route_pos, const float *w,
                                                 const float *seed, int M, int H, int k, int S,
                                                 size_t slab, float *y) {
    const int H4 = H / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)M * H4) return;
    const int t = (int)(idx / H4), c = (int)(idx % H4);
    f32x4 acc = seed ? reinterpret_cast<const f32x4 *>(seed + (size_t)t * H)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    if (y_shared) acc += reinterpret_cast<const f32x4 *>(y_shared + (size_t)t * H)[c];
    for (int j = 0; j < k; j++) {
        const int r = t * k + j;
        const float *row = y_routes + (size_t)route_pos[r] * H;
        f32x4 v = reinterpret_cast<const f32x4 *>(row)[c];
        for (int sl = 1; sl < S; sl++) v += reinterpret_cast<const f32x4 *>(row + sl * slab)[c];
        const float wt = w[r];
        acc.x = fmaf(wt, v.x, acc.x);
        acc.y = fmaf(wt, v.y, acc.y);
        acc.z = fmaf(wt, v.z, acc.z);
        acc.w = fmaf(wt, v.w, acc.w);
    }
    reinterpret_cast<f32x4 *>(y + (size_t)t * H)[c] = acc;
}

hipError_t launch_combine(const Layer &L, const float *y_routes, const float *y_shared,
                          const int32_t *route_pos, const float *w, const float *seed, int M,
                          float *y, hipStream_t s, int slices) {
    const size_t n = (size_t)M * (L.H / 4);
    launch_kernel(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y_routes, y_shared,
                       route_pos, w, seed, M, L.H, L.k, slices, (size_t)M * L.k * L.H, y);
    return hipGetLastError();
}

} // namespace moe
