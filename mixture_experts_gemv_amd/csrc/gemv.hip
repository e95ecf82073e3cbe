// Bandwidth-bound GEMV path of the routed MoE layer (decode and small batches).
//
// After routing and permutation, every touched expert's weight rows are
// streamed from HBM once and dotted with the vectors routed to that expert.
//
// gate/up: a workgroup owns one tile of 16 or 32 rows of one touched expert
//   (or of the shared expert).  The x rows of the expert's tokens are copied
//   into LDS as stored (bf16 or fp32).  Each wave streams its 4 or 8
//   rows RP at a time, issuing every 16-byte load of a group (gate and up)
//   before using any, and dots each row with every staged token (one or four tokens
//   per pass over the loaded rows).  With bf16 x
//   and bf16 or Q8_0 weights the products run on v_dot2c_f32_bf16: bf16
//   weights are used as loaded, Q8_0 int8 values convert to bf16 exactly, and
//   the fp16 block scale multiplies each chunk's dot.  The per-token pre-norm
//   scale multiplies the finished dot.  Epilogue: clamp (routed experts only),
//   silu(g) * v -> act.
// down: a workgroup owns (touched expert, tile of 32 or 64 rows of H, slice of
//   the reduction over I).  The slice of the expert's act rows is copied into
//   LDS (fp32), each wave streams its rows RP at a time (every load of a group
//   issued first), and each row's dots are written to y_routes[slice][route][h]
//   (y_shared[slice][token][h] for the shared expert); the combine kernel sums
//   slices and routes in a fixed order, so results are bitwise repeatable.
// Vectors beyond what LDS holds are taken in further passes over the tile.
// One token (M = 1) has its own kernels further down.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
// Rows per wave of the per-row kernels' tiles depend on the format: gate/up
// 4 for bf16 weights (DeepSeek-V2-Lite shape, M = 16: 131 against 154 us),
// 8 for the others; down as dn_rows_per_wave below.
template <int WDT> constexpr int gu_rows_per_wave() { return WDT == DT_BF16 ? 4 : 8; }
static int gu_rows_tile(int dt) { return kWaves * (dt == DT_BF16 ? 4 : 8); }
// Down rows per wave: 8 for bf16 weights (DeepSeek-V2-Lite shape, M = 16:
// 74 against 85 us), 16 for the others (gpt-oss shape, Q8_0: 66 against 69 us).
template <int WDT> constexpr int dn_rows_per_wave() { return WDT == DT_BF16 ? 8 : 16; }
static int dn_rows_tile(int dt) { return kWaves * (dt == DT_BF16 ? 8 : 16); }
// Vectors dotted per pass over a group's loaded rows: one when a row is one
// chunk block (each staged vector then takes its own pass over the loaded
// registers, with the fewest accumulators), four when a row spans several
// blocks (the sums then run across the blocks, so a stage holds at most that
// many vectors).  Measured at M = 16 against four a pass: gpt-oss-shaped
// Q8_0 gate/up 109 against 132 us, MXFP4 107 against 121 us.
constexpr int kTVMulti = 4;
template <int CPL> constexpr int tokens_per_pass() { return CPL == 8 ? kTVMulti : 1; }
constexpr int kStageMax = 8;             // vectors one LDS stage holds, at most
constexpr size_t kStreamLds = 150 * 1024; // LDS budget of the streamed gate/up kernel
constexpr int kStreamGrid = 256;          // its workgroups: one a CU
constexpr int kStageBytes = 64 * 1024;   // LDS for staged vectors, per workgroup
// Rows per load group of the per-row kernels with MXFP4 weights (gate/up with
// at most two chunks per lane, down with at most four).  Four rows, which
// would keep as many bytes in flight as Q8_0's two, measured slower (the
// register footprint costs occupancy).
constexpr int kMx4RowsGU = 2;
constexpr int kMx4RowsDN = 2;


// The 16 int8 of a Q8_0 chunk as 8 words of bf16 pairs (exact: |q| <= 127).
__device__ __forceinline__ void q8_to_bf16x2(u32x4 v, uint32_t (&o)[8]) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t f0 = __float_as_uint(i8_to_f32<0>(d[i])), f1 = __float_as_uint(i8_to_f32<1>(d[i]));
        const uint32_t f2 = __float_as_uint(i8_to_f32<2>(d[i])), f3 = __float_as_uint(i8_to_f32<3>(d[i]));
        o[2 * i] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        o[2 * i + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    }
}


// ------------------------------------------------------------------ gate/up
struct RowsGateUp {
    const void *x;
    const float *tok_scale;
    Mats routed, shared;
    const int32_t *offsets, *sorted, *active;
    int M, H, k, I, Is;
    int max_routed;           // routed expert slots in the grid (>= touched experts)
    int tiles_I, tiles_Is;    // row tiles per routed / shared expert
    int ncap;                 // token rows one LDS stage holds
    float limit;
    float *act, *shared_act;
};

// The loads of one row group: RP rows of gate and of up, CPL chunks per lane.
template <int WDT, int CPL, int RP>
struct GateUpLoads {
    u32x4 g[RP][CPL], u[RP][CPL];
    uint16_t hg[RP][CPL], hu[RP][CPL];
};

template <int XDT, int WDT, int CPL, int RP>
__global__ __launch_bounds__(kThreads) void k_gateup_rows(RowsGateUp a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_x[]; // [ncap][H] as stored
    constexpr int N = Chunk<WDT>::N;
    constexpr int NG = gu_rows_per_wave<WDT>() / RP;
    constexpr int kTV = tokens_per_pass<CPL>();
    constexpr bool DOT2 = XDT == DT_BF16 && WDT != DT_F32;
    constexpr int XB = XDT == DT_BF16 ? 2 : 4;
    constexpr int NW = N / 2; // bf16 pair words per chunk (dot2 form)
    using Loads = GateUpLoads<WDT, CPL, RP>;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int H = a.H;

    // ---- segment (touched expert or shared expert) and row tile
    int b = blockIdx.x, width, p0 = 0, n, rt;
    bool shared;
    size_t mrow0;
    if (b < a.max_routed * a.tiles_I) {
        const int u = b / a.tiles_I;
        if (u >= a.active[0]) return;
        const int e = a.active[1 + u];
        rt = b - u * a.tiles_I;
        width = a.I;
        p0 = a.offsets[e];
        n = a.offsets[e + 1] - p0;
        shared = false;
        mrow0 = (size_t)e * a.I;
    } else {
        rt = b - a.max_routed * a.tiles_I;
        if (rt >= a.tiles_Is) return;
        width = a.Is;
        n = a.M;
        shared = true;
        mrow0 = 0;
    }
    const Mats &m = shared ? a.shared : a.routed;
    const size_t rbytes = row_bytes<WDT>(H);
    const char *gbase = reinterpret_cast<const char *>(m.gate) + mrow0 * rbytes;
    const char *ubase = reinterpret_cast<const char *>(m.up) + mrow0 * rbytes;
    const void *gsb = nullptr, *usb = nullptr;
    if constexpr (blocked<WDT>()) {
        gsb = scale_at<WDT>(m.gate_s, mrow0 * (H / 32));
        usb = scale_at<WDT>(m.up_s, mrow0 * (H / 32));
    }
    const int row_w = rt * kWaves * gu_rows_per_wave<WDT>() + wave * gu_rows_per_wave<WDT>(); // this wave's first row
    const int nch = H / N;
    const int ncb = (nch + kWave * CPL - 1) / (kWave * CPL); // chunk blocks per row
    const int ng = row_w < width ? min(NG, (width - row_w) / RP) : 0;
    const int nsteps = ng * ncb; // (row group, chunk block) steps of this wave
    const int cpr = H * XB / 16; // 16-byte pieces per staged row

    auto chunks = [&](int cb, int (&cl)[CPL], bool (&ok)[CPL]) {
#pragma unroll
        for (int cc = 0; cc < CPL; cc++) {
            const int c = cb * kWave * CPL + lane + kWave * cc;
            ok[cc] = c < nch;
            cl[cc] = min(c, nch - 1);
        }
    };
    auto load = [&](Loads &B, int st) {
        const int g = st / ncb, cb = st - g * ncb;
        const int i0 = row_w + g * RP;
        int cl[CPL];
        bool ok[CPL];
        chunks(cb, cl, ok);
#pragma unroll
        for (int r = 0; r < RP; r++)
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                B.g[r][cc] = load_raw(gbase + (size_t)(i0 + r) * rbytes, cl[cc]);
                B.u[r][cc] = load_raw(ubase + (size_t)(i0 + r) * rbytes, cl[cc]);
                if constexpr (blocked<WDT>()) {
                    B.hg[r][cc] = scale_bits<WDT>(gsb, (size_t)(i0 + r) * (H / 32) + chunk_block<WDT>(cl[cc]));
                    B.hu[r][cc] = scale_bits<WDT>(usb, (size_t)(i0 + r) * (H / 32) + chunk_block<WDT>(cl[cc]));
                }
            }
    };

    float ag[RP][kTV], au[RP][kTV];
    // dots of the loaded chunks with staged tokens j0..j0+nj-1
    auto dots = [&](const Loads &B, int cb, int j0, int nj) {
        int cl[CPL];
        bool ok[CPL];
        chunks(cb, cl, ok);
#pragma unroll
        for (int cc = 0; cc < CPL; cc++) {
#pragma unroll
            for (int r = 0; r < RP; r++) {
                if constexpr (DOT2) {
                    uint32_t wg[NW], wu[NW];
                    if constexpr (WDT == DT_Q8) {
                        q8_to_bf16x2(B.g[r][cc], wg);
                        q8_to_bf16x2(B.u[r][cc], wu);
                    } else if constexpr (WDT == DT_MX4) {
                        mx4_to_bf16x2(B.g[r][cc], wg);
                        mx4_to_bf16x2(B.u[r][cc], wu);
                    } else {
                        wg[0] = B.g[r][cc].x; wg[1] = B.g[r][cc].y; wg[2] = B.g[r][cc].z; wg[3] = B.g[r][cc].w;
                        wu[0] = B.u[r][cc].x; wu[1] = B.u[r][cc].y; wu[2] = B.u[r][cc].z; wu[3] = B.u[r][cc].w;
                    }
                    const float scg = blocked<WDT>() ? scale_value<WDT>(B.hg[r][cc]) : 1.f;
                    const float scu = blocked<WDT>() ? scale_value<WDT>(B.hu[r][cc]) : 1.f;
#pragma unroll
                    for (int j = 0; j < kTV; j++) {
                        if (j < nj) {
                            const u32x4 *xp = reinterpret_cast<const u32x4 *>(
                                s_x + ((size_t)(j0 + j) * H + (size_t)cl[cc] * N) * 2);
                            uint32_t xw[NW];
#pragma unroll
                            for (int q4 = 0; q4 < NW / 4; q4++) {
                                const u32x4 v = xp[q4];
                                xw[4 * q4] = ok[cc] ? v.x : 0u;
                                xw[4 * q4 + 1] = ok[cc] ? v.y : 0u;
                                xw[4 * q4 + 2] = ok[cc] ? v.z : 0u;
                                xw[4 * q4 + 3] = ok[cc] ? v.w : 0u;
                            }
                            if constexpr (blocked<WDT>()) {
                                float sg = 0.f, su = 0.f;
#pragma unroll
                                for (int q = 0; q < NW; q++) {
                                    sg = dot2_bf16(wg[q], xw[q], sg);
                                    su = dot2_bf16(wu[q], xw[q], su);
                                }
                                ag[r][j] = fmaf(scg, sg, ag[r][j]);
                                au[r][j] = fmaf(scu, su, au[r][j]);
                            } else {
#pragma unroll
                                for (int q = 0; q < NW; q++) {
                                    ag[r][j] = dot2_bf16(wg[q], xw[q], ag[r][j]);
                                    au[r][j] = dot2_bf16(wu[q], xw[q], au[r][j]);
                                }
                            }
                        }
                    }
                } else {
                    float wg[N], wu[N];
                    decode_chunk<WDT>(B.g[r][cc], wg);
                    decode_chunk<WDT>(B.u[r][cc], wu);
                    float scg = ok[cc] ? 1.f : 0.f, scu = scg;
                    if constexpr (blocked<WDT>()) {
                        scg *= scale_value<WDT>(B.hg[r][cc]);
                        scu *= scale_value<WDT>(B.hu[r][cc]);
                    }
#pragma unroll
                    for (int j = 0; j < kTV; j++) {
                        if (j < nj) {
                            float xv[N];
                            const unsigned char *xp = s_x + ((size_t)(j0 + j) * H + (size_t)cl[cc] * N) * XB;
                            if constexpr (XDT == DT_BF16 && N == 4) {
                                const u32x2 v = reinterpret_cast<const u32x2 *>(xp)[0];
                                xv[0] = bf16_lo(v.x); xv[1] = bf16_hi(v.x);
                                xv[2] = bf16_lo(v.y); xv[3] = bf16_hi(v.y);
                            } else {
#pragma unroll
                                for (int q4 = 0; q4 < N * XB / 16; q4++) {
                                    const u32x4 v = reinterpret_cast<const u32x4 *>(xp)[q4];
                                    if constexpr (XDT == DT_BF16) {
                                        xv[8 * q4] = bf16_lo(v.x); xv[8 * q4 + 1] = bf16_hi(v.x);
                                        xv[8 * q4 + 2] = bf16_lo(v.y); xv[8 * q4 + 3] = bf16_hi(v.y);
                                        xv[8 * q4 + 4] = bf16_lo(v.z); xv[8 * q4 + 5] = bf16_hi(v.z);
                                        xv[8 * q4 + 6] = bf16_lo(v.w); xv[8 * q4 + 7] = bf16_hi(v.w);
                                    } else {
                                        xv[4 * q4] = __uint_as_float(v.x); xv[4 * q4 + 1] = __uint_as_float(v.y);
                                        xv[4 * q4 + 2] = __uint_as_float(v.z); xv[4 * q4 + 3] = __uint_as_float(v.w);
                                    }
                                }
                            }
                            float pg = 0.f, pu = 0.f;
#pragma unroll
                            for (int i = 0; i < N; i++) {
                                pg = fmaf(wg[i], xv[i], pg);
                                pu = fmaf(wu[i], xv[i], pu);
                            }
                            ag[r][j] = fmaf(scg, pg, ag[r][j]);
                            au[r][j] = fmaf(scu, pu, au[r][j]);
                        }
                    }
                }
            }
        }
    };
    // one (row, token) result per reduction pair: clamp, SwiGLU, store
    auto epilogue = [&](int i0, int jt, int nj) {
#pragma unroll
        for (int j = 0; j < kTV; j++) {
            if (j < nj) {
                const int jj = jt + j;
                const int t = shared ? jj : a.sorted[p0 + jj] / a.k;
                const float sc = a.tok_scale ? a.tok_scale[t] : 1.0f;
                float gv[2 * RP]; // gate and up of each row, summed together
#pragma unroll
                for (int r = 0; r < RP; r++) {
                    gv[2 * r] = ag[r][j];
                    gv[2 * r + 1] = au[r][j];
                }
                const float sgv = wave_sum_rows<2 * RP>(gv, lane);
#pragma unroll
                for (int r = 0; r < RP; r++) {
                    float g = lane_value(sgv, 2 * r * sum_lanes<2 * RP>()) * sc;
                    float v = lane_value(sgv, (2 * r + 1) * sum_lanes<2 * RP>()) * sc;
                    if (!shared && a.limit > 0.f) { // the shared expert is not clamped
                        g = clampf(g, a.limit);
                        v = clampf(v, a.limit);
                    }
                    if (lane == 0) {
                        const float h = silu_mul(g, v);
                        if (shared) a.shared_act[(size_t)jj * a.Is + i0 + r] = h;
                        else a.act[(size_t)(p0 + jj) * a.I + i0 + r] = h;
                    }
                }
            }
        }
    };
    // a step's work once its loads are in: with one chunk block per row every
    // staged token is done from the registers (kTV at a time); with several,
    // the stage holds at most kTV tokens and the sums run across the blocks.
    auto compute = [&](const Loads &B, int st, int s0, int ns) {
        const int g = st / ncb, cb = st - g * ncb;
        const int i0 = row_w + g * RP;
        if constexpr (DOT2 && WDT == DT_Q8 && kTV == 1) {
            // Q8_0 rows of one chunk block: converted to bf16 pairs once,
            // then dotted with each staged token (the conversion is most of
            // the work a token adds otherwise); chunks past the row end get
            // scale 0
            int cl[CPL];
            bool ok[CPL];
            chunks(cb, cl, ok);
            uint32_t wg[RP][CPL][NW], wu[RP][CPL][NW];
            float scg[RP][CPL], scu[RP][CPL];
#pragma unroll
            for (int r = 0; r < RP; r++)
#pragma unroll
                for (int cc = 0; cc < CPL; cc++) {
                    q8_to_bf16x2(B.g[r][cc], wg[r][cc]);
                    q8_to_bf16x2(B.u[r][cc], wu[r][cc]);
                    scg[r][cc] = ok[cc] ? scale_value<WDT>(B.hg[r][cc]) : 0.f;
                    scu[r][cc] = ok[cc] ? scale_value<WDT>(B.hu[r][cc]) : 0.f;
                }
            for (int j = 0; j < ns; j++) {
#pragma unroll
                for (int r = 0; r < RP; r++) ag[r][0] = au[r][0] = 0.f;
#pragma unroll
                for (int cc = 0; cc < CPL; cc++) {
                    const u32x4 *xp = reinterpret_cast<const u32x4 *>(s_x + ((size_t)j * H + (size_t)cl[cc] * N) * 2);
                    uint32_t xw[NW];
#pragma unroll
                    for (int q4 = 0; q4 < NW / 4; q4++) {
                        const u32x4 v = xp[q4];
                        xw[4 * q4] = v.x; xw[4 * q4 + 1] = v.y; xw[4 * q4 + 2] = v.z; xw[4 * q4 + 3] = v.w;
                    }
#pragma unroll
                    for (int r = 0; r < RP; r++) {
                        float sg = 0.f, su = 0.f;
#pragma unroll
                        for (int q = 0; q < NW; q++) {
                            sg = dot2_bf16(wg[r][cc][q], xw[q], sg);
                            su = dot2_bf16(wu[r][cc][q], xw[q], su);
                        }
                        ag[r][0] = fmaf(scg[r][cc], sg, ag[r][0]);
                        au[r][0] = fmaf(scu[r][cc], su, au[r][0]);
                    }
                }
                epilogue(i0, s0 + j, 1);
            }
            return;
        }
        for (int j0 = 0; j0 < ns; j0 += kTV) {
            const int nj = min(kTV, ns - j0);
            if (cb == 0)
#pragma unroll
                for (int r = 0; r < RP; r++)
#pragma unroll
                    for (int j = 0; j < kTV; j++) ag[r][j] = au[r][j] = 0.f;
            dots(B, cb, j0, nj);
            if (cb == ncb - 1) epilogue(i0, s0 + j0, nj);
        }
    };

    auto stage = [&](int s0, int ns) {
        __syncthreads(); // the previous stage is no longer read
        for (int q = tid; q < ns * cpr; q += kThreads) {
            const int j = q / cpr, c = q - j * cpr;
            const int t = shared ? s0 + j : a.sorted[p0 + s0 + j] / a.k;
            reinterpret_cast<u32x4 *>(s_x)[q] =
                reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.x) + (size_t)t * H * XB)[c];
        }
        __syncthreads();
    };
    // (Issuing the next step's loads before computing the current one
    // measured slower: the extra registers cost more than the overlap.)
    auto steps = [&](int st0, int s0, int ns) {
        for (int st = st0; st < nsteps; st++) {
            Loads B;
            load(B, st);
            compute(B, st, s0, ns);
        }
    };
    // The first step's weights depend on the expert only, so their loads are
    // issued before the first stage is copied and overlap it (gpt-oss-shaped
    // M = 16: Q8_0 gate/up 105.6 against 108.4 us, MXFP4 100.0 against 106.4).
    const int ns0 = min(a.ncap, n);
    {
        Loads B0;
        if (nsteps > 0) load(B0, 0);
        stage(0, ns0);
        if (nsteps > 0) compute(B0, 0, 0, ns0);
    }
    steps(1, 0, ns0);
    for (int s0 = a.ncap; s0 < n; s0 += a.ncap) {
        const int ns = min(a.ncap, n - s0);
        stage(s0, ns);
        steps(0, s0, ns);
    }
}

// Chunks per lane per row for a reduction of `chunks` 16-byte chunks, from the
// instantiated set (larger reductions loop over blocks of 8 * 64 chunks).
static int rows_cpl(int chunks) {
    const int c = (chunks + kWave - 1) / kWave;
    return c <= 4 ? (c < 1 ? 1 : c) : 8;
}

template <int XDT, int WDT>
static void gateup_rows_dispatch(int cpl, const RowsGateUp &a, int grid, size_t lds, hipStream_t s) {
    constexpr int R = WDT == DT_MX4 ? kMx4RowsGU : 2;
    switch (cpl) {
    case 1: launch_kernel((k_gateup_rows<XDT, WDT, 1, R>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    case 2: launch_kernel((k_gateup_rows<XDT, WDT, 2, R>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    case 3: launch_kernel((k_gateup_rows<XDT, WDT, 3, 2>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    case 4: launch_kernel((k_gateup_rows<XDT, WDT, 4, 2>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    default: launch_kernel((k_gateup_rows<XDT, WDT, 8, 1>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    }
}

static int chunk_elems(int dt) { return dt == DT_MX4 ? 32 : (dt == DT_Q8 ? 16 : (dt == DT_BF16 ? 8 : 4)); }

// Token rows one LDS stage of the gate/up kernel holds: up to kStageMax, as
// LDS allows, and at most kTVMulti when a row spans several chunk blocks.
int gemv_stage_tokens(const Layer &L) {
    const int xb = L.xdt == DT_BF16 ? 2 : 4;
    int n = kStageBytes / (L.H * xb);
    if (n > kStageMax) n = kStageMax;
    const int nch = L.H / chunk_elems(L.edt), cpl = rows_cpl(nch);
    if (nch > kWave * cpl && n > kTVMulti) n = kTVMulti;
    return n;
}

// ------------------------------------------------------- gate/up, streamed
// Small batches with bf16 x, when every token row fits in LDS: the waves of
// the grid stream (touched expert, row) pairs, strided by the grid's waves as
// in the one-token kernel.  A pair's gate and up rows are loaded (CPL 16-byte
// chunks a lane), converted to bf16 pairs once, and dotted with each of the
// expert's tokens, read from the workgroup's copy of the batch in LDS.  A
// workgroup is 1024 threads (16 waves, one workgroup a CU) and stages the
// batch, the route-to-token table, the token scales and the routing lists
// once.
struct StreamGateUp {
    const void *x; // bf16 [M][H]
    const float *tok_scale;
    Mats routed, shared;
    const int32_t *offsets, *sorted, *active;
    int M, H, k, E, I, Is;
    float limit;
    float *act, *shared_act;
    // sel.logits non-null (M <= 16): every workgroup runs the batch's
    // selection in its prologue (select_small) instead of reading offsets,
    // sorted and active, and workgroup 0 writes it for the down kernel and
    // the combine, so that no selection kernel runs between the router and
    // this kernel
    SelectSmall sel;
};
constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / kWave;
static_assert(kStreamWaves >= kSelMaxM, "one wave a token for the fused selection");

// LDS bytes of the streamed gate/up kernel for an M-token batch: the batch,
// route tokens, token scales, the touched list and offsets, then (with the
// fused selection, from a 16-byte boundary) the selection's scratch.
static size_t stream_lds_base(const Layer &L, int M) {
    return (size_t)M * L.H * 2 + (size_t)M * L.k * 4 + (size_t)M * 4 + (size_t)(2 * kMaxE + 2) * 4;
}
static size_t stream_lds_bytes(const Layer &L, int M, bool sel) {
    const size_t base = stream_lds_base(L, M);
    if (!sel) return base;
    return (base + 15) / 16 * 16 + (size_t)kStreamWaves * kWave * 8 + (size_t)M * L.E * 4 + (size_t)L.E * 8 +
           (size_t)M * L.k * 4 + 16;
}

template <int WDT, int CPL>
__global__ __launch_bounds__(kStreamThreads) void k_gateup_stream(StreamGateUp a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
    constexpr int N = Chunk<WDT>::N;
    constexpr int NW = N / 2; // bf16 pair words per chunk
    const int tid = threadIdx.x, lane = tid & 63;
    const int H = a.H, nch = H / N, R = a.M * a.k;
    uint16_t *s_x = reinterpret_cast<uint16_t *>(s_dyn);                 // [M][H]
    int *s_tok = reinterpret_cast<int *>(s_dyn + (size_t)a.M * H * 2);    // [R] token of sorted route
    float *s_sc = reinterpret_cast<float *>(s_tok + R);                 // [M] token scales
    int *s_act = reinterpret_cast<int *>(s_sc + a.M);                   // [1 + E] touched experts
    int *s_off = s_act + kMaxE + 1;                                     // [E + 1] offsets
    for (int q = tid; q < a.M * H / 8; q += kStreamThreads)
        reinterpret_cast<u32x4 *>(s_x)[q] = reinterpret_cast<const u32x4 *>(a.x)[q];
    for (int q = tid; q < a.M; q += kStreamThreads) s_sc[q] = a.tok_scale ? a.tok_scale[q] : 1.0f;
    if (a.sel.logits) {
        // the selection's scratch after the offsets (layout as stream_lds_bytes)
        const size_t o = ((size_t)(reinterpret_cast<unsigned char *>(s_off + kMaxE + 1) - s_dyn) + 15) / 16 * 16;
        uint64_t *s_words = reinterpret_cast<uint64_t *>(s_dyn + o);                     // [waves][64]
        float *s_logit = reinterpret_cast<float *>(s_words + kStreamWaves * kWave);        // [M][E]
        float *s_bias = s_logit + a.M * a.E;                                               // [E]
        uint32_t *s_mask = reinterpret_cast<uint32_t *>(s_bias + a.E);                     // [E]
        int *s_ids = reinterpret_cast<int *>(s_mask + a.E);                                // [R]
        int *s_scan = s_ids + R;                                                           // [4]
        select_small(a.sel, blockIdx.x == 0, s_logit, s_bias, s_mask, s_ids, s_scan, s_words, s_off, s_act,
                     s_tok);
    } else {
        for (int q = tid; q < R; q += kStreamThreads) s_tok[q] = a.sorted[q] / a.k;
        for (int q = tid; q <= a.E; q += kStreamThreads) {
            s_act[q] = a.active[q];
            s_off[q] = a.offsets[q];
        }
    }
    __syncthreads();
    const int routed_pairs = s_act[0] * a.I;
    const int total = routed_pairs + a.Is;
    const int nwv = gridDim.x * kStreamWaves;
    const int gw = uniform(blockIdx.x * kStreamWaves + (tid >> 6));
    int cl[CPL];
    bool ok[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; cc++) {
        const int c = lane + kWave * cc;
        ok[cc] = c < nch;
        cl[cc] = min(c, nch - 1);
    }
    const size_t rbytes = row_bytes<WDT>(H);
    for (int p = gw; p < total; p += nwv) {
        // the pair: a touched expert's row, or a shared-expert row (all tokens)
        const bool routed = p < routed_pairs;
        int e = 0, irow, p0 = 0, n = a.M;
        size_t row;
        if (routed) {
            const int u = p / a.I;
            irow = p - u * a.I;
            e = s_act[1 + u];
            p0 = s_off[e];
            n = s_off[e + 1] - p0;
            row = (size_t)e * a.I + irow;
        } else {
            irow = p - routed_pairs;
            row = irow;
        }
        const Mats &m = routed ? a.routed : a.shared;
        const char *grow = reinterpret_cast<const char *>(m.gate) + row * rbytes;
        const char *urow = reinterpret_cast<const char *>(m.up) + row * rbytes;
        u32x4 rg[CPL], ru[CPL];
        uint16_t hg[CPL], hu[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; cc++) {
            rg[cc] = load_raw(grow, cl[cc]);
            ru[cc] = load_raw(urow, cl[cc]);
            if constexpr (blocked<WDT>()) {
                hg[cc] = scale_bits<WDT>(m.gate_s, row * (H / 32) + chunk_block<WDT>(cl[cc]));
                hu[cc] = scale_bits<WDT>(m.up_s, row * (H / 32) + chunk_block<WDT>(cl[cc]));
            }
        }
        // converted once; chunks past the row end get scale 0
        uint32_t wg[CPL][NW], wu[CPL][NW];
        float scg[CPL], scu[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; cc++) {
            if constexpr (WDT == DT_Q8) {
                q8_to_bf16x2(rg[cc], wg[cc]);
                q8_to_bf16x2(ru[cc], wu[cc]);
            } else if constexpr (WDT == DT_MX4) {
                mx4_to_bf16x2(rg[cc], wg[cc]);
                mx4_to_bf16x2(ru[cc], wu[cc]);
            } else {
                wg[cc][0] = rg[cc].x; wg[cc][1] = rg[cc].y; wg[cc][2] = rg[cc].z; wg[cc][3] = rg[cc].w;
                wu[cc][0] = ru[cc].x; wu[cc][1] = ru[cc].y; wu[cc][2] = ru[cc].z; wu[cc][3] = ru[cc].w;
            }
            scg[cc] = ok[cc] ? (blocked<WDT>() ? scale_value<WDT>(hg[cc]) : 1.f) : 0.f;
            scu[cc] = ok[cc] ? (blocked<WDT>() ? scale_value<WDT>(hu[cc]) : 1.f) : 0.f;
        }
        for (int j = 0; j < n; j++) {
            const int t = routed ? s_tok[p0 + j] : j;
            const u32x4 *xr = reinterpret_cast<const u32x4 *>(s_x + (size_t)t * H);
            float g = 0.f, v = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                uint32_t xw[NW];
#pragma unroll
                for (int q4 = 0; q4 < NW / 4; q4++) {
                    const u32x4 q = xr[cl[cc] * (NW / 4) + q4];
                    xw[4 * q4] = q.x; xw[4 * q4 + 1] = q.y; xw[4 * q4 + 2] = q.z; xw[4 * q4 + 3] = q.w;
                }
                float sg = 0.f, su = 0.f;
#pragma unroll
                for (int q = 0; q < NW; q++) {
                    sg = dot2_bf16(wg[cc][q], xw[q], sg);
                    su = dot2_bf16(wu[cc][q], xw[q], su);
                }
                g = fmaf(scg[cc], sg, g);
                v = fmaf(scu[cc], su, v);
            }
            const float sc = s_sc[t];
            const float gv[2] = {g, v};
            const float sgv = wave_sum_rows<2>(gv, lane); // g in lanes 0-31, v in 32-63
            g = lane_value(sgv, 0) * sc;
            v = lane_value(sgv, 32) * sc;
            if (routed && a.limit > 0.f) { // the shared expert is not clamped
                g = clampf(g, a.limit);
                v = clampf(v, a.limit);
            }
            if (lane == 0) {
                const float h = silu_mul(g, v);
                if (routed) a.act[(size_t)(p0 + j) * a.I + irow] = h;
                else a.shared_act[(size_t)j * a.Is + irow] = h;
            }
        }
    }
}

template <int WDT>
static bool gateup_stream_dispatch(int cpl, const StreamGateUp &a, int grid, size_t lds, hipStream_t s) {
    switch (cpl) {
    case 1: launch_kernel((k_gateup_stream<WDT, 1>), dim3(grid), dim3(kStreamThreads), (uint32_t)lds, s, a); return true;
    case 2: launch_kernel((k_gateup_stream<WDT, 2>), dim3(grid), dim3(kStreamThreads), (uint32_t)lds, s, a); return true;
    case 3: launch_kernel((k_gateup_stream<WDT, 3>), dim3(grid), dim3(kStreamThreads), (uint32_t)lds, s, a); return true;
    case 4: launch_kernel((k_gateup_stream<WDT, 4>), dim3(grid), dim3(kStreamThreads), (uint32_t)lds, s, a); return true;
    default: return false;
    }
}

// The streamed kernel when it applies: bf16 x, bf16, Q8_0 or MXFP4 weights
// (the shared expert's in the same format), at most 4 chunks a lane (2 for
// MXFP4), and the batch within the LDS budget.  Returns false to leave the call to the
// per-row kernel.
// Whether the streamed gate/up kernel takes an M-token batch (with the
// selection fused into it when sel).
static bool stream_ok(const Layer &L, int M, bool shared, bool sel) {
    const int Is = shared ? L.Is : 0;
    if (L.xdt != DT_BF16 || L.edt == DT_F32 || (Is > 0 && L.sdt != L.edt) || L.E > kMaxE) return false;
    if (sel && (M > kSelMaxM || M < 1)) return false;
    if (stream_lds_bytes(L, M, sel) > kStreamLds) return false;
    const int cpl = (L.H / chunk_elems(L.edt) + kWave - 1) / kWave;
    return cpl <= (L.edt == DT_MX4 ? 2 : 4); // (MXFP4 at 3 or more would spill)
}

bool gateup_stream_selects(const Layer &L, int M, bool shared) { return stream_ok(L, M, shared, true); }

static bool launch_gateup_stream(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                                 const Mats &shared, const Routing &rt, int M, float *act, float *shared_act,
                                 hipStream_t s, const SelectSmall *sel) {
    const int Is = shared_act ? L.Is : 0;
    if (!act || !stream_ok(L, M, shared_act != nullptr, sel != nullptr)) return false;
    const size_t lds = stream_lds_bytes(L, M, sel != nullptr);
    const int cpl = (L.H / chunk_elems(L.edt) + kWave - 1) / kWave;
    StreamGateUp a;
    a.sel = sel ? *sel : SelectSmall{};
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
    a.E = L.E;
    a.I = L.I;
    a.Is = Is;
    a.limit = L.limit;
    a.act = act;
    a.shared_act = shared_act;
    const int grid = kStreamGrid;
    if (L.edt == DT_Q8) return gateup_stream_dispatch<DT_Q8>(cpl, a, grid, lds, s);
    if (L.edt == DT_MX4) return gateup_stream_dispatch<DT_MX4>(cpl, a, grid, lds, s);
    return gateup_stream_dispatch<DT_BF16>(cpl, a, grid, lds, s);
}

hipError_t launch_gateup_gemv(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                              const Mats &shared, const Routing &rt, int M, float *act,
                              float *shared_act, hipStream_t s, const SelectSmall *sel) {
    RowsGateUp a;
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
    a.max_routed = act ? (L.E < M * L.k ? L.E : M * L.k) : 0;
    a.tiles_I = (L.I + gu_rows_tile(L.edt) - 1) / gu_rows_tile(L.edt);
    a.tiles_Is = (a.Is + gu_rows_tile(L.edt) - 1) / gu_rows_tile(L.edt);
    a.limit = L.limit;
    a.act = act;
    a.shared_act = shared_act;
    if (launch_gateup_stream(L, x, tok_scale, routed, shared, rt, M, act, shared_act, s, sel)) return hipGetLastError();
    if (sel) return hipErrorInvalidValue; // the caller checked gateup_stream_selects
    const int xb = L.xdt == DT_BF16 ? 2 : 4;
    a.ncap = gemv_stage_tokens(L);
    if (a.ncap < 1) return hipErrorInvalidValue;
    // a segment holds at most M tokens (a token picks an expert at most once)
    const size_t lds = (size_t)(M < a.ncap ? M : a.ncap) * L.H * xb;
    const int grid = a.max_routed * a.tiles_I + a.tiles_Is;
    if (grid == 0) return hipSuccess;
    const int cpl = rows_cpl(L.H / chunk_elems(L.edt));
    if (L.xdt == DT_BF16) {
        if (L.edt == DT_BF16) gateup_rows_dispatch<DT_BF16, DT_BF16>(cpl, a, grid, lds, s);
        else if (L.edt == DT_Q8) gateup_rows_dispatch<DT_BF16, DT_Q8>(cpl, a, grid, lds, s);
        else if (L.edt == DT_MX4) gateup_rows_dispatch<DT_BF16, DT_MX4>(cpl, a, grid, lds, s);
        else gateup_rows_dispatch<DT_BF16, DT_F32>(cpl, a, grid, lds, s);
    } else {
        if (L.edt == DT_BF16) gateup_rows_dispatch<DT_F32, DT_BF16>(cpl, a, grid, lds, s);
        else if (L.edt == DT_Q8) gateup_rows_dispatch<DT_F32, DT_Q8>(cpl, a, grid, lds, s);
        else if (L.edt == DT_MX4) gateup_rows_dispatch<DT_F32, DT_MX4>(cpl, a, grid, lds, s);
        else gateup_rows_dispatch<DT_F32, DT_F32>(cpl, a, grid, lds, s);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ down
struct RowsDown {
    const float *act, *shared_act;
    Mats routed, shared;
    const int32_t *offsets, *active;
    int M, H, I, Is;
    int max_routed, tiles_H;
    int S, KS;      // routed experts: reduction slices over I and their width
    int Ss, KSs;    // shared expert: slices over Is
    int ncap;       // act rows one LDS stage holds
    float *y_routes, *y_shared;
    size_t slab_r, slab_s;
};

template <int WDT, int CPL, int RP>
struct DownLoads {
    u32x4 w[RP][CPL];
    uint16_t h[RP][CPL];
};

template <int WDT, int CPL, int RP>
__global__ __launch_bounds__(kThreads) void k_down_rows(RowsDown a) {
    extern __shared__ __attribute__((aligned(16))) float s_act[]; // [ncap][KS] fp32
    constexpr int N = Chunk<WDT>::N;
    constexpr int NG = dn_rows_per_wave<WDT>() / RP;
    constexpr int kTV = tokens_per_pass<CPL>();
    // act slices are staged piece-major when a chunk spans 8 pieces (MXFP4;
    // gpt-oss shape, M = 16: down 71 against 88 us).  With 2 or 4 pieces
    // (bf16, Q8_0) the scattered staging writes cost more than the strided
    // reads (DeepSeek-V2-Lite shape: 73 against 71 us), so those stay linear.
    constexpr int P = N / 4; // 16-byte pieces of act per chunk
    constexpr bool PM = P >= 8;
    using Loads = DownLoads<WDT, CPL, RP>;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int H = a.H;

    int b = blockIdx.x, width, p0 = 0, n, rt, ks, KS;
    bool shared;
    size_t mrow0;
    const float *vec;
    const int per_routed = a.S * a.tiles_H;
    if (b < a.max_routed * per_routed) {
        const int u = b / per_routed;
        if (u >= a.active[0]) return;
        const int e = a.active[1 + u];
        const int rem = b - u * per_routed;
        ks = rem / a.tiles_H;
        rt = rem - ks * a.tiles_H;
        width = a.I;
        KS = a.KS;
        p0 = a.offsets[e];
        n = a.offsets[e + 1] - p0;
        shared = false;
        mrow0 = (size_t)e * H;
        vec = a.act + (size_t)p0 * a.I;
    } else {
        const int rem = b - a.max_routed * per_routed;
        ks = rem / a.tiles_H;
        if (ks >= a.Ss) return;
        rt = rem - ks * a.tiles_H;
        width = a.Is;
        KS = a.KSs;
        n = a.M;
        shared = true;
        mrow0 = 0;
        vec = a.shared_act;
    }
    const Mats &m = shared ? a.shared : a.routed;
    const int k0 = ks * KS, klen = min(KS, width - k0);
    const size_t rbytes = row_bytes<WDT>(width);
    const char *dbase = reinterpret_cast<const char *>(m.down) + mrow0 * rbytes + row_bytes<WDT>(k0);
    const void *dsb = nullptr;
    if constexpr (blocked<WDT>()) dsb = scale_at<WDT>(m.down_s, mrow0 * (width / 32) + k0 / 32);
    float *out = shared ? a.y_shared + ks * a.slab_s : a.y_routes + ks * a.slab_r + (size_t)p0 * H;
    const int row_w = rt * kWaves * dn_rows_per_wave<WDT>() + wave * dn_rows_per_wave<WDT>();
    const int nch = klen / N;
    const int ncb = (nch + kWave * CPL - 1) / (kWave * CPL);
    const int ng = row_w < H ? min(NG, (H - row_w) / RP) : 0;
    const int nsteps = ng * ncb;
    const int cpr = klen / 4; // 16-byte pieces per staged row slice

    auto chunks = [&](int cb, int (&cl)[CPL], bool (&ok)[CPL]) {
#pragma unroll
        for (int cc = 0; cc < CPL; cc++) {
            const int c = cb * kWave * CPL + lane + kWave * cc;
            ok[cc] = c < nch;
            cl[cc] = min(c, nch - 1);
        }
    };
    auto load = [&](Loads &B, int st) {
        const int g = st / ncb, cb = st - g * ncb;
        const int h0 = row_w + g * RP;
        int cl[CPL];
        bool ok[CPL];
        chunks(cb, cl, ok);
#pragma unroll
        for (int r = 0; r < RP; r++)
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                B.w[r][cc] = load_raw(dbase + (size_t)(h0 + r) * rbytes, cl[cc]);
                if constexpr (blocked<WDT>())
                    B.h[r][cc] = scale_bits<WDT>(dsb, (size_t)(h0 + r) * (width / 32) + chunk_block<WDT>(cl[cc]));
            }
    };
    float acc[RP][kTV];
    auto dots = [&](const Loads &B, int cb, int j0, int nj) {
        int cl[CPL];
        bool ok[CPL];
        chunks(cb, cl, ok);
#pragma unroll
        for (int cc = 0; cc < CPL; cc++) {
            float wv[RP][N];
#pragma unroll
            for (int r = 0; r < RP; r++) {
                decode_chunk<WDT>(B.w[r][cc], wv[r]);
                float sc = ok[cc] ? 1.f : 0.f;
                if constexpr (blocked<WDT>()) sc *= scale_value<WDT>(B.h[r][cc]);
#pragma unroll
                for (int i = 0; i < N; i++) wv[r][i] *= sc;
            }
#pragma unroll
            for (int j = 0; j < kTV; j++) {
                if (j < nj) {
                    const f32x4 *ap = reinterpret_cast<const f32x4 *>(s_act + (size_t)(j0 + j) * KS);
                    float av[N];
#pragma unroll
                    for (int q4 = 0; q4 < N / 4; q4++) {
                        const f32x4 v = PM ? ap[piece_major(cl[cc], q4, nch, P)] : ap[cl[cc] * P + q4];
                        av[4 * q4] = v.x; av[4 * q4 + 1] = v.y; av[4 * q4 + 2] = v.z; av[4 * q4 + 3] = v.w;
                    }
#pragma unroll
                    for (int r = 0; r < RP; r++)
#pragma unroll
                        for (int i = 0; i < N; i++) acc[r][j] = fmaf(wv[r][i], av[i], acc[r][j]);
                }
            }
        }
    };
    auto compute = [&](const Loads &B, int st, int s0, int ns) {
        const int g = st / ncb, cb = st - g * ncb;
        const int h0 = row_w + g * RP;
        if constexpr (kTV == 1) {
            // rows of one chunk block: decoded and scaled once, then dotted
            // with each staged act row (chunks past the slice end get 0)
            int cl[CPL];
            bool ok[CPL];
            chunks(cb, cl, ok);
            float wv[RP][CPL][N];
#pragma unroll
            for (int cc = 0; cc < CPL; cc++)
#pragma unroll
                for (int r = 0; r < RP; r++) {
                    decode_chunk<WDT>(B.w[r][cc], wv[r][cc]);
                    float sc = ok[cc] ? 1.f : 0.f;
                    if constexpr (blocked<WDT>()) sc *= scale_value<WDT>(B.h[r][cc]);
#pragma unroll
                    for (int i = 0; i < N; i++) wv[r][cc][i] *= sc;
                }
            for (int j = 0; j < ns; j++) {
                float d[RP];
#pragma unroll
                for (int r = 0; r < RP; r++) d[r] = 0.f;
                const f32x4 *ap = reinterpret_cast<const f32x4 *>(s_act + (size_t)j * KS);
#pragma unroll
                for (int cc = 0; cc < CPL; cc++) {
                    float av[N];
#pragma unroll
                    for (int q4 = 0; q4 < N / 4; q4++) {
                        const f32x4 v = PM ? ap[piece_major(cl[cc], q4, nch, P)] : ap[cl[cc] * P + q4];
                        av[4 * q4] = v.x; av[4 * q4 + 1] = v.y; av[4 * q4 + 2] = v.z; av[4 * q4 + 3] = v.w;
                    }
#pragma unroll
                    for (int r = 0; r < RP; r++)
#pragma unroll
                        for (int i = 0; i < N; i++) d[r] = fmaf(wv[r][cc][i], av[i], d[r]);
                }
                const float v = wave_sum_rows<RP>(d, lane); // row lane / sum_lanes of the group
                if (lane % sum_lanes<RP>() == 0) out[(size_t)(s0 + j) * H + h0 + lane / sum_lanes<RP>()] = v;
            }
            return;
        }
        for (int j0 = 0; j0 < ns; j0 += kTV) {
            const int nj = min(kTV, ns - j0);
            if (cb == 0)
#pragma unroll
                for (int r = 0; r < RP; r++)
#pragma unroll
                    for (int j = 0; j < kTV; j++) acc[r][j] = 0.f;
            dots(B, cb, j0, nj);
            if (cb == ncb - 1) {
#pragma unroll
                for (int j = 0; j < kTV; j++) {
                    if (j < nj) {
                        const int jj = s0 + j0 + j;
                        float d[RP];
#pragma unroll
                        for (int r = 0; r < RP; r++) d[r] = acc[r][j];
                        const float v = wave_sum_rows<RP>(d, lane);
                        if (lane % sum_lanes<RP>() == 0) out[(size_t)jj * H + h0 + lane / sum_lanes<RP>()] = v;
                    }
                }
            }
        }
    };

    // (Issuing the first step's weight loads before the first stage's copy,
    // as the gate/up kernel does, measured slower here: gpt-oss-shaped M = 16,
    // MXFP4 down 74.7 against 71.0 us, Q8_0 65.2 against 64.2 us.)
    for (int s0 = 0; s0 < n; s0 += a.ncap) {
        const int ns = min(a.ncap, n - s0);
        __syncthreads();
        for (int q = tid; q < ns * cpr; q += kThreads) {
            const int j = q / cpr, c = q - j * cpr;
            reinterpret_cast<f32x4 *>(s_act + (size_t)j * KS)[PM ? piece_major(c / P, c % P, nch, P) : c] =
                reinterpret_cast<const f32x4 *>(vec + (size_t)(s0 + j) * width + k0)[c];
        }
        __syncthreads();
        for (int st = 0; st < nsteps; st++) {
            Loads B;
            load(B, st);
            compute(B, st, s0, ns);
        }
    }
}

// Slices of a down reduction of `width` elements: each at most 64 chunks
// (one 16-byte load per lane: 1024 Q8_0, 2048 MXFP4, 512 bf16 or 256 fp32
// elements), a multiple of 32 (whole Q8_0 and MXFP4 blocks), as even as
// that allows.  (Measured at the gpt-oss shape, M = 16: Q8_0 down 66 against
// 86 us with 2048-element slices, 90 chunks on 64 lanes; MXFP4 105 against
// 91 us with 1024-element slices, 30 chunks.)
static void down_slices(int width, int dt, int *S, int *KS) {
    if (width <= 0) {
        *S = 0;
        *KS = 0;
        return;
    }
    const int smax = kWave * chunk_elems(dt);
    *S = (width + smax - 1) / smax;
    *KS = ((width + *S - 1) / *S + 31) / 32 * 32;
    *S = (width + *KS - 1) / *KS;
}

int down_gemv_slices(int width, int dt) {
    int S, KS;
    down_slices(width, dt, &S, &KS);
    return S;
}

// (MXFP4 chunks decode to 32 values, so a group takes half the rows.)
template <int WDT>
static void down_rows_dispatch(int cpl, const RowsDown &a, int grid, size_t lds, hipStream_t s) {
    constexpr int R = WDT == DT_MX4 ? kMx4RowsDN : 4;
    switch (cpl) {
    case 1: launch_kernel((k_down_rows<WDT, 1, R>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    case 2: launch_kernel((k_down_rows<WDT, 2, R>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    case 3: launch_kernel((k_down_rows<WDT, 3, R>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    case 4: launch_kernel((k_down_rows<WDT, 4, R>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    default: launch_kernel((k_down_rows<WDT, 8, R / 2>), dim3(grid), dim3(kThreads), (uint32_t)lds, s, a); break;
    }
}

hipError_t launch_down_gemv(const Layer &L, const float *act, const float *shared_act, const Mats &routed,
                            const Mats &shared, const Routing &rt, int M, float *y_routes, float *y_shared,
                            hipStream_t s) {
    RowsDown a;
    a.act = act;
    a.shared_act = shared_act;
    a.routed = routed;
    a.shared = shared;
    a.offsets = rt.offsets;
    a.active = rt.active;
    a.M = M;
    a.H = L.H;
    a.I = L.I;
    a.Is = shared_act ? L.Is : 0;
    a.max_routed = act ? (L.E < M * L.k ? L.E : M * L.k) : 0;
    a.tiles_H = (L.H + dn_rows_tile(L.edt) - 1) / dn_rows_tile(L.edt);
    down_slices(L.I, L.edt, &a.S, &a.KS);
    down_slices(a.Is, L.sdt, &a.Ss, &a.KSs);
    const int ks_max = a.KS > a.KSs ? a.KS : a.KSs;
    a.ncap = kStageBytes / (ks_max * 4);
    if (a.ncap > kStageMax) a.ncap = kStageMax;
    a.y_routes = y_routes;
    a.y_shared = y_shared;
    a.slab_r = (size_t)M * L.k * L.H;
    a.slab_s = (size_t)M * L.H;
    const size_t lds = (size_t)(M < a.ncap ? M : a.ncap) * ks_max * 4;
    const int grid = a.max_routed * a.S * a.tiles_H + a.Ss * a.tiles_H;
    if (grid == 0) return hipSuccess;
    const int cpl = rows_cpl(ks_max / chunk_elems(L.edt));
    if (L.edt == DT_BF16) down_rows_dispatch<DT_BF16>(cpl, a, grid, lds, s);
    else if (L.edt == DT_Q8) down_rows_dispatch<DT_Q8>(cpl, a, grid, lds, s);
    else if (L.edt == DT_MX4) down_rows_dispatch<DT_MX4>(cpl, a, grid, lds, s);
    else down_rows_dispatch<DT_F32>(cpl, a, grid, lds, s);
    return hipGetLastError();
}

// ================================================================ M = 1 decode
// With one token every touched expert sees the same x, and the sorted
// position of the route to the u-th touched expert is u.
//
// gate/up: each wave holds x in registers (lane l owns chunks l, l+64, ...)
// and streams (slot, row) pairs, RP at a time and strided by the grid's
// waves, issuing all 2*RP*CPL 16-byte loads of a group before using them.
// The gate/up kernel runs the token's top-k from the router logits in its
// prologue (every wave, DPP rounds); its first wave writes the picks and their
// weights, which the down kernel reads.  (Computing the logits inside every
// gate/up workgroup instead of in a router kernel measured slower.)
struct M1Route {
    const float *logits, *bias; // logits null: one expert, no router (the pick is expert 0, weight 1)
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

// The token's top-k from its logit row (lv, bv as topk_load leaves them), as
// the slot table; the grid's first wave (`writer`) also stores the picks in
// descending key order, their weights and the per-expert counts.  Up to 64
// experts the slot table comes from the ballot of the picks (the set bits in
// ascending order); beyond, from each pick's rank among the picks.
__device__ __forceinline__ M1Slots m1_topk(const M1Route &rt, int lane, const float (&lv)[kKeysPerLane],
                                           const float (&bv)[kKeysPerLane], uint64_t *words, bool writer,
                                           int32_t *ids_out, float *w_out, int32_t *counts_out) {
    M1Slots s{0, 0, 0, 0, 0, 0, 0, 0};
    if (!rt.logits) {
        // one expert and no router: the pick is expert 0 with weight 1
        if (writer && lane == 0) {
            ids_out[0] = 0;
            w_out[0] = 1.0f;
            if (counts_out) counts_out[0] = 1;
        }
        return s;
    }
    if (rt.E <= kWave) {
        const LanePick p = topk_lane_small(lv[0], bv[0], rt.E, rt.k, rt.select, rt.bias_mode, lane, words);
        uint64_t m = __ballot(p.pick); // exactly k bits: the ranks are a permutation of 0..E-1
        for (int j = 0; j < rt.k; j++) {
            s.set(j, __builtin_ctzll(m));
            m &= m - 1;
        }
        if (writer) {
            if (p.pick) {
                ids_out[p.rank] = lane;
                w_out[p.rank] = p.w;
            }
            if (counts_out && lane < rt.E) counts_out[lane] = p.pick ? 1 : 0;
        }
        return s;
    }
    int my_id;
    float my_w;
    topk_wave_vals(lv, bv, rt.E, rt.k, rt.select, rt.bias_mode, lane, &my_id, &my_w);
    const int my_rank = pick_rank(my_id, rt.k, lane);
    for (int j = 0; j < rt.k; j++)
        s.set(__builtin_amdgcn_readlane(my_rank, j), __builtin_amdgcn_readlane(my_id, j));
    if (writer) {
        if (lane < rt.k) {
            ids_out[lane] = my_id;
            w_out[lane] = my_w;
        }
        if (counts_out)
            for (int e = lane; e < rt.E; e += kWave) {
                int c = 0;
                for (int u = 0; u < rt.k; u++) c += s.expert(u) == e;
                counts_out[e] = c;
            }
    }
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
    int total_pairs;
    float limit;
    float *act, *shared_act;
};

template <int XDT, int WDT, int CPL, int RP, bool PRE>
__global__ __launch_bounds__(kThreads) void k_gateup_m1(M1GateUpArgs a) {
    constexpr int N = Chunk<WDT>::N;
    __shared__ __align__(16) uint64_t s_words[kWaves][kWave];
    const int lane = threadIdx.x & 63;
    const int gw = uniform(blockIdx.x * kWaves + (threadIdx.x >> 6));
    // wave gw takes the RP pairs at gw * RP, then every nwv * RP further, so
    // that the waves in flight read neighbouring rows (measured faster than
    // a contiguous range of pairs a wave: gpt-oss-shaped Q8_0 16.1 against
    // 17.0 us, Mixtral-shaped 75.5 against 77.3 us)
    const int nwv = gridDim.x * kWaves;
    if (gw * RP >= a.total_pairs) return;
    const int p_end = a.total_pairs;
    const int H = a.H, nch = H / N;
    // the logit row first: the top-k needs it, and nothing else, before it
    // can start
    float lv[kKeysPerLane] = {}, bv[kKeysPerLane] = {};
    if (a.rt.logits) topk_load(a.rt.logits, a.rt.bias, a.rt.E, lane, lv, bv);
    const float sc = a.tok_scale ? a.tok_scale[0] : 1.0f;
    // x chunks this lane multiplies, loaded as stored and converted after
    // the top-k (which does not need them), so that the top-k does not wait
    // for them; lanes past the row end hold zeros and load (harmless)
    // duplicates of the last chunk.
    int cl[CPL];
    u32x2 xb[XDT == DT_BF16 ? CPL : 1][XDT == DT_BF16 ? N / 4 : 1];
    f32x4 xf[XDT == DT_BF16 ? 1 : CPL][XDT == DT_BF16 ? 1 : N / 4];
#pragma unroll
    for (int cc = 0; cc < CPL; cc++) {
        cl[cc] = min(lane + kWave * cc, nch - 1);
#pragma unroll
        for (int n4 = 0; n4 < N / 4; n4++) {
            if constexpr (XDT == DT_BF16)
                xb[cc][n4] = reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(a.x) + cl[cc] * N + 4 * n4)[0];
            else
                xf[cc][n4] = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.x) + cl[cc] * N + 4 * n4)[0];
        }
    }
    // pairs: the shared expert's rows first (q < Is), then the picks' rows.
    // PRE (layers with a shared expert, or one expert): a group whose rows
    // do not depend on the picks (shared rows, or the one expert 0) has its
    // loads issued before the top-k, so that they overlap it (DeepSeek-V2-
    // Lite shape, 29.3 against 30.5 us a call; its dense lead layer, 27.7
    // against 28.5 us; without PRE the registers it holds across the top-k
    // cost the other layers 0.5 us).
    const int routed_pairs = a.k * a.I, shared_pairs = p_end - routed_pairs;
    const size_t rbytes = row_bytes<WDT>(H);
    int slot[RP], irow[RP];
    u32x4 rg[RP][CPL], ru[RP][CPL];
    uint16_t hg[RP][CPL], hu[RP][CPL];
    auto issue_group = [&](int p, const M1Slots &sl) {
#pragma unroll
        for (int r = 0; r < RP; r++) {
            const int q = min(p + r, p_end - 1);
            size_t row;
            const Mats *m;
            if (q >= shared_pairs) {
                const int qr = q - shared_pairs;
                slot[r] = qr / a.I;
                irow[r] = qr - slot[r] * a.I;
                row = (size_t)sl.expert(slot[r]) * a.I + irow[r];
                m = &a.routed;
            } else {
                slot[r] = -1;
                irow[r] = q;
                row = q;
                m = &a.shared;
            }
            const char *grow = reinterpret_cast<const char *>(m->gate) + row * rbytes;
            const char *urow = reinterpret_cast<const char *>(m->up) + row * rbytes;
            const void *gsr = nullptr, *usr = nullptr;
            if constexpr (blocked<WDT>()) {
                gsr = scale_at<WDT>(m->gate_s, row * (H / 32));
                usr = scale_at<WDT>(m->up_s, row * (H / 32));
            }
            // every load of the group is issued before any is used
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                rg[r][cc] = load_raw(grow, cl[cc]);
                ru[r][cc] = load_raw(urow, cl[cc]);
                if constexpr (blocked<WDT>()) {
                    hg[r][cc] = scale_bits<WDT>(gsr, chunk_block<WDT>(cl[cc]));
                    hu[r][cc] = scale_bits<WDT>(usr, chunk_block<WDT>(cl[cc]));
                }
            }
        }
    };
    const int p_first = gw * RP;
    const bool early = PRE && (a.rt.E == 1 || min(p_first + RP, p_end) <= shared_pairs);
    if (early) issue_group(p_first, M1Slots{0, 0, 0, 0, 0, 0, 0, 0});
    const M1Slots slots = m1_topk(a.rt, lane, lv, bv, s_words[threadIdx.x >> 6], gw == 0, a.ids_out, a.w_out,
                                  a.counts_out);
    // MXFP4 codes with bf16 x: x stays as bf16 pairs and the codes, converted
    // to bf16 pairs, go through v_dot2c_f32_bf16 (the pre-norm scale then
    // multiplies the finished dots); otherwise x is held as fp32 with the
    // scale folded in.
    constexpr bool XD2 = XDT == DT_BF16 && WDT == DT_MX4;
    float xr[XD2 ? 1 : CPL][XD2 ? 1 : N];
    uint32_t xw[XD2 ? CPL : 1][XD2 ? N / 2 : 1];
    // (run once, after the first group's weight loads are issued)
    auto convert_x = [&]() {
#pragma unroll
    for (int cc = 0; cc < CPL; cc++) {
        const bool in = lane + kWave * cc < nch;
        const float m = in ? sc : 0.f;
#pragma unroll
        for (int n4 = 0; n4 < N / 4; n4++) {
            if constexpr (XD2) {
                xw[cc][2 * n4] = in ? xb[cc][n4].x : 0u;
                xw[cc][2 * n4 + 1] = in ? xb[cc][n4].y : 0u;
            } else if constexpr (XDT == DT_BF16) {
                const u32x2 q = xb[cc][n4];
                xr[cc][4 * n4] = bf16_lo(q.x) * m; xr[cc][4 * n4 + 1] = bf16_hi(q.x) * m;
                xr[cc][4 * n4 + 2] = bf16_lo(q.y) * m; xr[cc][4 * n4 + 3] = bf16_hi(q.y) * m;
            } else {
                const f32x4 q = xf[cc][n4];
                xr[cc][4 * n4] = q.x * m; xr[cc][4 * n4 + 1] = q.y * m;
                xr[cc][4 * n4 + 2] = q.z * m; xr[cc][4 * n4 + 3] = q.w * m;
            }
        }
    }
    };
    bool x_ready = false;
    for (int p = p_first; p < p_end; p += nwv * RP) {
        if (!(early && p == p_first)) issue_group(p, slots);
        if (!x_ready) {
            convert_x();
            x_ready = true;
        }
#pragma unroll
        for (int r = 0; r < RP; r++) {
            float g = 0.f, v = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPL; cc++) {
                float pg = 0.f, pu = 0.f;
                if constexpr (XD2) {
                    uint32_t wg[N / 2], wu[N / 2];
                    mx4_to_bf16x2(rg[r][cc], wg);
                    mx4_to_bf16x2(ru[r][cc], wu);
#pragma unroll
                    for (int q = 0; q < N / 2; q++) {
                        pg = dot2_bf16(wg[q], xw[cc][q], pg);
                        pu = dot2_bf16(wu[q], xw[cc][q], pu);
                    }
                } else {
                    float wg[N], wu[N];
                    decode_chunk<WDT>(rg[r][cc], wg);
                    decode_chunk<WDT>(ru[r][cc], wu);
#pragma unroll
                    for (int n = 0; n < N; n++) {
                        pg = fmaf(wg[n], xr[cc][n], pg);
                        pu = fmaf(wu[n], xr[cc][n], pu);
                    }
                }
                if constexpr (blocked<WDT>()) {
                    g = fmaf(scale_value<WDT>(hg[r][cc]), pg, g);
                    v = fmaf(scale_value<WDT>(hu[r][cc]), pu, v);
                } else {
                    g += pg;
                    v += pu;
                }
            }
            {
                const float gv[2] = {g, v};
                const float sgv = wave_sum_rows<2>(gv, lane); // g in lanes 0-31, v in 32-63
                g = lane_value(sgv, 0);
                v = lane_value(sgv, 32);
            }
            if constexpr (XD2) {
                g *= sc;
                v *= sc;
            }
            if (a.limit > 0.f && slot[r] >= 0) { // the shared expert is not clamped
                g = clampf(g, a.limit);
                v = clampf(v, a.limit);
            }
            if (lane == 0 && p + r < p_end) {
                const float h = silu_mul(g, v);
                if (slot[r] >= 0) a.act[(size_t)slot[r] * a.I + m1_act_index<N>(irow[r], a.I)] = h;
                else a.shared_act[m1_act_index<N>(irow[r], a.Is)] = h;
            }
        }
    }
}

// down (M = 1): a workgroup reads the k picks and weights the gate/up kernel
// wrote, then owns R output rows; its NT threads stride over the
// concatenated chunks of every touched expert's rows (then the shared
// expert's), UNR rounds at a time with every load of the rounds issued first.
// Each chunk's dot is scaled by its route's weight before the block
// reduction, which is done in a fixed order.  When every chunk fits one
// round of 768 threads, a workgroup takes 768 threads and one chunk a thread:
// the same loads in flight, spread over three times the waves, so that less
// work follows each wave's last load (gpt-oss-shaped Q8_0 layer, 720 chunks:
// 9.2 against 10.1 us for 256 threads and three rounds, in a standalone
// kernel), and 6 rows, so that the workgroups (two a CU) run in one wave
// (layer 28.1 against 28.9 us with 4 rows; MXFP4 27.9 against 29.7 us).
// At most 384 tasks (MXFP4 rows: 32-element chunks, 90 a row of 2880) take
// 384 threads and 6 rows, so that a workgroup's threads are not half idle
// (gpt-oss-shaped MXFP4 layer: 22.7 against 27.3 us a call; 8 rows 23.2).
// Up to 1408 tasks take 704 threads, two chunks each and 4 rows, so that the
// second round is full (DeepSeek-V2-Lite shape, 1408 chunks: 28.7 against
// 29.1 us a call with 256 threads in 2.75 rounds; its dense layer, 1368
// chunks: 25.0 against 25.6 us; 6 rows 30.2 and 26.6 us).
// Otherwise 256 threads and 4 rows take 4 rounds for Q8_0 (10.8 against
// 11.7 us with 2), else 2 (MXFP4 at 4: 14.3 against 10.5 us, from the
// register footprint of its 32-element chunks).
constexpr int kM1Rows = 4, kM1WideRows = 6;
constexpr int kM1WideThreads = 768;
constexpr int kM1NarrowThreads = 384, kM1NarrowRows = 6;
constexpr int kM1TwoThreads = 704, kM1TwoRows = 4;
template <int WDT> constexpr int m1_unroll() { return WDT == DT_Q8 ? 4 : 2; }
constexpr int kMaxSlots = 9; // top-k slots + the shared expert

struct M1DownArgs {
    const float *act, *shared_act;
    Mats routed, shared;
    const int32_t *ids; // [k] picks, written by the gate/up kernel
    const float *w;     // [k] their weights
    const float *seed;
    int H, I, Is, k;
    float *y;
};

template <int WDT, int NT, int UNR, int R>
__global__ __launch_bounds__(NT) void k_down_m1(M1DownArgs a) {
    constexpr int N = Chunk<WDT>::N;
    constexpr int NW = NT / kWave;
    __shared__ const char *s_row[kMaxSlots];
    __shared__ const void *s_sc[kMaxSlots];
    __shared__ const float *s_act[kMaxSlots];
    __shared__ float s_w[kMaxSlots];
    __shared__ int s_width[kMaxSlots];
    __shared__ float s_part[NW][R];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, h0 = blockIdx.x * R;
    const int n_routed = a.k; // with M = 1 every slot is a touched expert
    const int nch = a.I / N, nch_s = a.Is / N;
    if (wave == 0) {
        const int my_id = a.ids[min(lane, a.k - 1)];
        const float my_w = a.w[min(lane, a.k - 1)];
        const int my_rank = pick_rank(my_id, a.k, lane);
        if (lane < n_routed) {
            // slot = rank in ascending expert id, which is the act row of the pick
            const size_t row = (size_t)my_id * H + h0;
            s_row[my_rank] = reinterpret_cast<const char *>(a.routed.down) + row * row_bytes<WDT>(a.I);
            if constexpr (blocked<WDT>()) s_sc[my_rank] = scale_at<WDT>(a.routed.down_s, row * (a.I / 32));
            s_act[my_rank] = a.act + (size_t)my_rank * a.I;
            s_w[my_rank] = my_w;
            s_width[my_rank] = a.I;
        }
    }
    if (tid == n_routed && a.Is > 0) {
        s_row[tid] = reinterpret_cast<const char *>(a.shared.down) + (size_t)h0 * row_bytes<WDT>(a.Is);
        if constexpr (blocked<WDT>()) s_sc[tid] = scale_at<WDT>(a.shared.down_s, (size_t)h0 * (a.Is / 32));
        s_act[tid] = a.shared_act;
        s_w[tid] = 1.0f;
        s_width[tid] = a.Is;
    }
    __syncthreads();
    const int n_tasks = n_routed * nch + (a.Is > 0 ? nch_s : 0);
    const int last_row = min(R, H - h0) - 1;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] = 0.f;
    for (int t0 = 0; t0 < n_tasks; t0 += NT * UNR) {
        u32x4 raw[UNR][R];
        uint16_t hs[UNR][R];
        f32x4 av[UNR][N / 4];
        float wt[UNR];
#pragma unroll
        for (int u = 0; u < UNR; u++) {
            const int t = t0 + u * NT + tid;
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
            const size_t rb = row_bytes<WDT>(width);
            const char *row0 = s_row[slot];
            wt[u] = t < n_tasks ? s_w[slot] : 0.f;
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int rr = min(r, last_row);
                raw[u][r] = load_raw(row0 + rr * rb, c);
                if constexpr (blocked<WDT>())
                    hs[u][r] = scale_bits<WDT>(s_sc[slot], (size_t)rr * (width / 32) + chunk_block<WDT>(c));
            }
            // the chunk's pieces in the act layout of m1_act_index
            const f32x4 *ap = reinterpret_cast<const f32x4 *>(s_act[slot]);
#pragma unroll
            for (int n4 = 0; n4 < N / 4; n4++) av[u][n4] = ap[piece_major(c, n4, width / N, N / 4)];
        }
#pragma unroll
        for (int u = 0; u < UNR; u++) {
#pragma unroll
            for (int r = 0; r < R; r++) {
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
                if constexpr (blocked<WDT>()) d *= scale_value<WDT>(hs[u][r]);
                acc[r] = fmaf(wt[u], d, acc[r]);
            }
        }
    }
    {
        const float v = wave_sum_rows<R>(acc, lane); // row lane / sum_lanes of the group
        const int q = lane / sum_lanes<R>();
        if (lane % sum_lanes<R>() == 0 && q < R) s_part[wave][q] = v;
    }
    __syncthreads();
    if (tid <= last_row) {
        float v = a.seed ? a.seed[h0 + tid] : 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; wv++) v += s_part[wv][tid];
        a.y[h0 + tid] = v;
    }
}

template <int WDT>
static void down_m1_dispatch(int n_tasks, int H, const M1DownArgs &a, hipStream_t s) {
    if (n_tasks <= kM1NarrowThreads)
        launch_kernel((k_down_m1<WDT, kM1NarrowThreads, 1, kM1NarrowRows>),
                      dim3((H + kM1NarrowRows - 1) / kM1NarrowRows), dim3(kM1NarrowThreads), 0, s, a);
    else if (n_tasks <= kM1WideThreads)
        launch_kernel((k_down_m1<WDT, kM1WideThreads, 1, kM1WideRows>), dim3((H + kM1WideRows - 1) / kM1WideRows),
                      dim3(kM1WideThreads), 0, s, a);
    else if (n_tasks <= 2 * kM1TwoThreads)
        launch_kernel((k_down_m1<WDT, kM1TwoThreads, 2, kM1TwoRows>), dim3((H + kM1TwoRows - 1) / kM1TwoRows),
                      dim3(kM1TwoThreads), 0, s, a);
    else
        launch_kernel((k_down_m1<WDT, kThreads, m1_unroll<WDT>(), kM1Rows>), dim3((H + kM1Rows - 1) / kM1Rows),
                      dim3(kThreads), 0, s, a);
}

// Chunks per lane of a row of H elements, and the instantiated values.
static int m1_cpl(int H, int N) { return (H / N + kWave - 1) / kWave; }

template <int XDT, int WDT, int RP, bool PRE>
static bool m1_gateup_dispatch_p(int cpl, const M1GateUpArgs &a, int grid, hipStream_t s) {
#define M1_CASE(C) \
    case C: launch_kernel((k_gateup_m1<XDT, WDT, C, RP, PRE>), dim3(grid), dim3(kThreads), 0, s, a); return true;
    switch (cpl) {
        M1_CASE(1) M1_CASE(2) M1_CASE(3) M1_CASE(4) M1_CASE(5) M1_CASE(6) M1_CASE(8)
    default: return false;
    }
#undef M1_CASE
}
template <int XDT, int WDT, int RP>
static bool m1_gateup_dispatch(int cpl, const M1GateUpArgs &a, int grid, hipStream_t s) {
    return a.Is > 0 || a.rt.E == 1 ? m1_gateup_dispatch_p<XDT, WDT, RP, true>(cpl, a, grid, s)
                                   : m1_gateup_dispatch_p<XDT, WDT, RP, false>(cpl, a, grid, s);
}


bool m1_supported(const Layer &L) {
    const int N = chunk_elems(L.edt);
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
    const int N = chunk_elems(L.edt);
    const int cpl = m1_cpl(L.H, N);
    // Rows per load group: two for bf16, fp32 and (with bf16 x) MXFP4 rows
    // of at most four chunks per lane (about 16 loads of a group in flight),
    // else one.  With Q8_0 rows one row a group measured faster (gpt-oss
    // shape: 16.9 against 18.1 us; bf16 unchanged).  MXFP4 rows carry half
    // the bytes of Q8_0 ones, so they take up to 3072 waves and two rows a
    // group (gpt-oss shape, the layer call: 22.0 against 22.6 us with one
    // row, 23.2 with two rows and 2048 waves; one row and 2048 waves: 27.3
    // against 26.2 us with 3072, before the narrow down kernel).  Q8_0 rows
    // keep 2048 waves (the gpt-oss-shaped call: 28.0 against 29.4 us with
    // 2560 and 28.1 with 3072).
    const bool mx2 = L.edt == DT_MX4 && L.xdt == DT_BF16;
    const int RP = cpl <= 4 && (L.edt == DT_BF16 || L.edt == DT_F32 || mx2) ? 2 : 1;
    const int max_waves = L.edt == DT_MX4 ? 3072 : 2048;
    int ppw = (a.total_pairs + max_waves - 1) / max_waves;
    ppw = (ppw + RP - 1) / RP * RP;
    const int waves = (a.total_pairs + ppw - 1) / ppw;
    const int grid = (waves + kWaves - 1) / kWaves;
    bool ok;
    if (L.xdt == DT_BF16) {
        if (L.edt == DT_Q8) ok = m1_gateup_dispatch<DT_BF16, DT_Q8, 1>(cpl, a, grid, s);
        else if (L.edt == DT_MX4) ok = RP == 2 ? m1_gateup_dispatch<DT_BF16, DT_MX4, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_BF16, DT_MX4, 1>(cpl, a, grid, s);
        else if (L.edt == DT_BF16) ok = RP == 2 ? m1_gateup_dispatch<DT_BF16, DT_BF16, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_BF16, DT_BF16, 1>(cpl, a, grid, s);
        else ok = RP == 2 ? m1_gateup_dispatch<DT_BF16, DT_F32, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_BF16, DT_F32, 1>(cpl, a, grid, s);
    } else {
        if (L.edt == DT_Q8) ok = m1_gateup_dispatch<DT_F32, DT_Q8, 1>(cpl, a, grid, s);
        else if (L.edt == DT_MX4) ok = m1_gateup_dispatch<DT_F32, DT_MX4, 1>(cpl, a, grid, s);
        else if (L.edt == DT_BF16) ok = RP == 2 ? m1_gateup_dispatch<DT_F32, DT_BF16, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_F32, DT_BF16, 1>(cpl, a, grid, s);
        else ok = RP == 2 ? m1_gateup_dispatch<DT_F32, DT_F32, 2>(cpl, a, grid, s) : m1_gateup_dispatch<DT_F32, DT_F32, 1>(cpl, a, grid, s);
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_down_m1(const Layer &L, const float *act, const float *shared_act, const Mats &routed,
                          const Mats &shared, const int32_t *ids, const float *w, const float *seed,
                          float *y, hipStream_t s) {
    M1DownArgs a;
    a.act = act;
    a.shared_act = shared_act;
    a.routed = routed;
    a.shared = shared;
    a.ids = ids;
    a.w = w;
    a.seed = seed;
    a.H = L.H;
    a.I = L.I;
    a.Is = shared_act ? L.Is : 0;
    a.k = L.k;
    a.y = y;
    const int N = chunk_elems(L.edt);
    const int n_tasks = L.k * (L.I / N) + a.Is / N;
    if (L.edt == DT_BF16) down_m1_dispatch<DT_BF16>(n_tasks, L.H, a, s);
    else if (L.edt == DT_Q8) down_m1_dispatch<DT_Q8>(n_tasks, L.H, a, s);
    else if (L.edt == DT_MX4) down_m1_dispatch<DT_MX4>(n_tasks, L.H, a, s);
    else down_m1_dispatch<DT_F32>(n_tasks, L.H, a, s);
    return hipGetLastError();
}

// -------------------------------------------------------------------- combine
constexpr int kCombineSlots = 8; // top-k slots a token (the plan's limit)
// One thread per (token, 4 consecutive h): seed, then the shared expert's
// slices in order, then slots j = 0..k-1, each slot's slices (partial sums of
// a split reduction) summed in slice order before its weight is applied.
// SU: later reduction slices loaded together.  With SU > 1 every slot's
// loads of SU slices go out before any is added; each slot's slices are
// still added in slice order, so the sums are the same bits as one slice at
// a time.  Taken below 512 workgroups, where the chains of dependent loads
// set the time (one-expert layer, M = 16, 16 slices: 7.0 against 8.9 us;
// DeepSeek-V2-Lite shape, M = 16: 5.0 against 7.6 us; 256 experts, M = 16:
// 4.4 against 7.7 us).  Above that the registers it holds cost more waves
// than it saves (one-expert layer, M = 512, 1024 workgroups: 19.1 against
// 13.2 us).
template <int SU>
__global__ __launch_bounds__(256) void k_combine(const float *y_routes, const float *y_shared,
                                                 const int32_t *route_pos, const float *w,
                                                 const float *seed, int M, int H, int k, int S,
                                                 size_t slab, int Ss, size_t slab_s, float *y) {
    const int H4 = H / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)M * H4) return;
    const int t = (int)(idx / H4), c = (int)(idx % H4);
    f32x4 acc = seed ? reinterpret_cast<const f32x4 *>(seed + (size_t)t * H)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    if (y_shared) {
        const float *row = y_shared + (size_t)t * H;
        f32x4 v = reinterpret_cast<const f32x4 *>(row)[c];
        for (int sl = 1; sl < Ss; sl += SU) {
            f32x4 q[SU];
#pragma unroll
            for (int u = 0; u < SU; u++)
                if (sl + u < Ss) q[u] = reinterpret_cast<const f32x4 *>(row + (sl + u) * slab_s)[c];
#pragma unroll
            for (int u = 0; u < SU; u++)
                if (sl + u < Ss) v += q[u];
        }
        acc += v;
    }
    // the slots' positions and weights, then (up to 8 slots) every slot's
    // first slice, are loaded before any is used: two dependent round trips
    // a thread instead of two a slot (Qwen3-shaped M = 2048, 134 MB of
    // per-route rows: 28.1 against 30.8 us; Mixtral-shaped M = 512, 14.9
    // against 15.2 us)
    int rp[kCombineSlots];
    float wt[kCombineSlots];
#pragma unroll
    for (int j = 0; j < kCombineSlots; j++)
        if (j < k) {
            rp[j] = route_pos[t * k + j];
            wt[j] = w[t * k + j];
        }
    f32x4 v[kCombineSlots];
#pragma unroll
    for (int j = 0; j < kCombineSlots; j++)
        if (j < k) v[j] = reinterpret_cast<const f32x4 *>(y_routes + (size_t)rp[j] * H)[c];
    if constexpr (SU > 1) {
        for (int sl = 1; sl < S; sl += SU) {
            f32x4 q[kCombineSlots][SU];
#pragma unroll
            for (int j = 0; j < kCombineSlots; j++)
#pragma unroll
                for (int u = 0; u < SU; u++)
                    if (j < k && sl + u < S)
                        q[j][u] = reinterpret_cast<const f32x4 *>(y_routes + (size_t)rp[j] * H + (sl + u) * slab)[c];
#pragma unroll
            for (int j = 0; j < kCombineSlots; j++)
#pragma unroll
                for (int u = 0; u < SU; u++)
                    if (j < k && sl + u < S) v[j] += q[j][u];
        }
    }
#pragma unroll
    for (int j = 0; j < kCombineSlots; j++)
        if (j < k) {
            if constexpr (SU == 1) {
                const float *row = y_routes + (size_t)rp[j] * H;
                for (int sl = 1; sl < S; sl++) v[j] += reinterpret_cast<const f32x4 *>(row + sl * slab)[c];
            }
            acc.x = fmaf(wt[j], v[j].x, acc.x);
            acc.y = fmaf(wt[j], v[j].y, acc.y);
            acc.z = fmaf(wt[j], v[j].z, acc.z);
            acc.w = fmaf(wt[j], v[j].w, acc.w);
        }
    reinterpret_cast<f32x4 *>(y + (size_t)t * H)[c] = acc;
}

hipError_t launch_combine(const Layer &L, const float *y_routes, const float *y_shared,
                          const int32_t *route_pos, const float *w, const float *seed, int M,
                          float *y, hipStream_t s, int slices, int shared_slices) {
    const size_t n = (size_t)M * (L.H / 4);
    const unsigned grid = (unsigned)((n + 255) / 256);
    const auto kern = (slices > 1 || shared_slices > 1) && grid < 512 ? k_combine<4> : k_combine<1>;
    launch_kernel(kern, dim3(grid), dim3(256), 0, s, y_routes, y_shared,
                  route_pos, w, seed, M, L.H, L.k, slices, (size_t)M * L.k * L.H, shared_slices,
                  (size_t)M * L.H, y);
    return hipGetLastError();
}

} // namespace moe
