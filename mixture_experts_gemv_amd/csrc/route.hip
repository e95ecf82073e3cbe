// Routing kernels: RMS pre-norm scale, router GEMV, wave top-k + softmax, and
// the expert histogram / scan / stable scatter of the routes.
//
// For small batches a router kernel with one workgroup per (expert, 4 tokens)
// is followed by one workgroup that runs every token's top-k and the
// permutation.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace moe {


// ------------------------------------------------------------------ pre-norm
// scale[t] = 1 / sqrt(mean_i x[t][i]^2 + eps); one wave per token.
template <int XDT>
__global__ __launch_bounds__(256) void k_rms_scale(const void *x, int M, int H, float eps, float *scale) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= M) return;
    const char *row = reinterpret_cast<const char *>(x) + (size_t)t * H * dt_bytes<XDT>();
    float s = 0.f;
    for (int c = lane; c < H / 8; c += kWave) {
        float v[8];
        load8<XDT>(row, c, v);
#pragma unroll
        for (int i = 0; i < 8; i++) s += v[i] * v[i];
    }
    s = wave_sum(s);
    if (lane == 0) scale[t] = 1.0f / sqrtf(s / (float)H + eps);
}

hipError_t launch_rms_scale(const Layer &L, const void *x, int M, float *scale, hipStream_t s) {
    dim3 grid((M + 3) / 4);
    if (L.xdt == DT_BF16)
        launch_kernel(k_rms_scale<DT_BF16>, grid, dim3(256), 0, s, x, M, L.H, L.eps, scale);
    else
        launch_kernel(k_rms_scale<DT_F32>, grid, dim3(256), 0, s, x, M, L.H, L.eps, scale);
    return hipGetLastError();
}

// The normed rows of the fused layer: xn[t][i] = x[t][i] * scale[t] * gamma[i]
// (gamma stored like x; null = unit gain) as fp32 rows; when xs is given, as
// the split bf16 rows the grouped-GEMM router reads (per 8 elements: their 8
// hi values bf16(v), then their 8 lo values bf16(v - hi)); when xh is given,
// as the fp16 rows (saturated to +-65504) the grouped GEMM's experts read.  One thread per
// 8 elements of a row.
template <int XDT>
__global__ __launch_bounds__(256) void k_norm_apply(const void *x, const void *gamma, const float *scale, int H,
                                                    float *xn, uint16_t *xs, uint16_t *xh) {
    const int t = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= H / 8) return;
    float v[8], g[8];
    load8<XDT>(reinterpret_cast<const char *>(x) + (size_t)t * H * dt_bytes<XDT>(), c, v);
    if (gamma) {
        load8<XDT>(gamma, c, g);
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) g[i] = 1.f;
    }
    const float sc = scale[t];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = v[i] * sc * g[i];
    f32x4 *o = reinterpret_cast<f32x4 *>(xn + (size_t)t * H + (size_t)c * 8);
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
    if (xs) {
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            hi[i] = f32_to_bf16_rne(v[i]);
            lo[i] = f32_to_bf16_rne(v[i] - __uint_as_float(hi[i] << 16));
        }
        u32x4 *q = reinterpret_cast<u32x4 *>(xs + (size_t)t * H * 2 + (size_t)c * 16);
        q[0] = u32x4{hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16, hi[6] | hi[7] << 16};
        q[1] = u32x4{lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16, lo[6] | lo[7] << 16};
    }
    if (xh) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; i++) h[i] = f32_to_f16_sat(v[i]);
        *reinterpret_cast<u32x4 *>(xh + (size_t)t * H + (size_t)c * 8) =
            u32x4{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
    }
}

hipError_t launch_norm_apply(const Layer &L, const void *x, const void *gamma, const float *scale, int M,
                             float *xn, uint16_t *xs, uint16_t *xh, hipStream_t s) {
    const dim3 grid((L.H / 8 + 255) / 256, M);
    if (L.xdt == DT_BF16)
        launch_kernel(k_norm_apply<DT_BF16>, grid, dim3(256), 0, s, x, gamma, scale, L.H, xn, xs, xh);
    else
        launch_kernel(k_norm_apply<DT_F32>, grid, dim3(256), 0, s, x, gamma, scale, L.H, xn, xs, xh);
    return hipGetLastError();
}

// ---------------------------------------------------------------- router dots
// One wave: logits of expert row `wrow` for tokens t0..t0+nt-1 (nt <= TM).
// Lanes stride the row in 8-element pieces, CB pieces per lane per block.
// Every load of a block (the router pieces and the pieces of all TM tokens)
// is issued unconditionally before any is used: indices past the row end or
// past the last token are clamped, and their products masked.  Each token's
// sum is wave-reduced.
// Q8_0 router rows (the INT8 router): piece p is 8 int8 values of the int8
// plane and block p / 4's fp16 scale.  xs (bf16 [H], or null) is the router's
// per-element input scale; it multiplies the router piece (x * s * w is
// computed as x * (w * s)).
template <int XDT, int RDT, int TM, int CB>
__device__ __forceinline__ void router_dots(const void *x, const void *wrow, const void *wsrow,
                                            const uint16_t *xs, int H, int t0, int nt,
                                            int lane, float (&acc)[TM], int cb = 0, int ce = -1) {
    const size_t xrow = (size_t)H * dt_bytes<XDT>();
    const char *xb = reinterpret_cast<const char *>(x) + (size_t)t0 * xrow;
    const int nch = ce < 0 ? H / 8 : ce;  // this wave covers 8-element pieces cb..nch-1
#pragma unroll
    for (int i = 0; i < TM; i++) acc[i] = 0.f;
    for (int c0 = cb; c0 < nch; c0 += kWave * CB) {
        float w[CB][8];
        int cc[CB];
#pragma unroll
        for (int j = 0; j < CB; j++) {
            const int c = c0 + lane + kWave * j;
            cc[j] = min(c, nch - 1);
            if constexpr (RDT == DT_Q8) {
                const u32x2 q = reinterpret_cast<const u32x2 *>(wrow)[cc[j]];
                const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(wsrow)[cc[j] >> 2]);
                w[j][0] = i8_to_f32<0>(q.x) * d; w[j][1] = i8_to_f32<1>(q.x) * d;
                w[j][2] = i8_to_f32<2>(q.x) * d; w[j][3] = i8_to_f32<3>(q.x) * d;
                w[j][4] = i8_to_f32<0>(q.y) * d; w[j][5] = i8_to_f32<1>(q.y) * d;
                w[j][6] = i8_to_f32<2>(q.y) * d; w[j][7] = i8_to_f32<3>(q.y) * d;
            } else {
                load8<RDT>(wrow, cc[j], w[j]);
            }
            if (xs) {
                float g[8];
                load8<DT_BF16>(xs, cc[j], g);
#pragma unroll
                for (int i = 0; i < 8; i++) w[j][i] *= g[i];
            }
        }
        float xv[TM][CB][8];
#pragma unroll
        for (int tm = 0; tm < TM; tm++) {
            const int tc = min(tm, nt - 1);
#pragma unroll
            for (int j = 0; j < CB; j++) load8<XDT>(xb + tc * xrow, cc[j], xv[tm][j]);
        }
#pragma unroll
        for (int j = 0; j < CB; j++) {
            const float mk = c0 + lane + kWave * j < nch ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) w[j][i] *= mk;
        }
#pragma unroll
        for (int tm = 0; tm < TM; tm++)
#pragma unroll
            for (int j = 0; j < CB; j++)
#pragma unroll
                for (int i = 0; i < 8; i++) acc[tm] = fmaf(w[j][i], xv[tm][j][i], acc[tm]);
    }
#pragma unroll
    for (int tm = 0; tm < TM; tm++) acc[tm] = tm < nt ? wave_sum(acc[tm]) : 0.f;
}

// Start of expert e's router row and of its Q8_0 scale row.
template <int RDT>
__device__ __forceinline__ const char *router_row(const RouterW &rw, int e, int H) {
    return reinterpret_cast<const char *>(rw.w) + (size_t)e * row_bytes<RDT>(H);
}
__device__ __forceinline__ const void *router_srow(const RouterW &rw, int e, int H) {
    return rw.w_s ? reinterpret_cast<const char *>(rw.w_s) + (size_t)e * (H / 32) * 2 : nullptr;
}

// logits[t][e] = scale[t] * sum_i x[t][i] * s[i] * router[e][i].  One wave per
// (expert, group of TM tokens).
constexpr int kRouterTM = 4;

template <int XDT, int RDT>
__global__ __launch_bounds__(64) void k_router_gemv(const void *x, RouterW rw,
                                                    const float *tok_scale, int M, int H, int E,
                                                    float *logits) {
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * kRouterTM;
    const int lane = threadIdx.x;
    const int nt = min(kRouterTM, M - t0);
    float acc[kRouterTM];
    router_dots<XDT, RDT, kRouterTM, 2>(x, router_row<RDT>(rw, e, H), router_srow(rw, e, H), rw.xs, H, t0, nt,
                                        lane, acc);
#pragma unroll
    for (int tm = 0; tm < kRouterTM; tm++) {
        if (tm < nt && lane == 0) {
            float v = acc[tm];
            if (tok_scale) v *= tok_scale[t0 + tm];
            logits[(size_t)(t0 + tm) * E + e] = v;
        }
    }
}

template <int XDT>
static void router_gemv_rdt(const Layer &L, const void *x, const RouterW &rw, const float *tok_scale, int M,
                            float *logits, hipStream_t s) {
    const dim3 grid(L.E, (M + kRouterTM - 1) / kRouterTM);
    if (L.rdt == DT_BF16)
        launch_kernel((k_router_gemv<XDT, DT_BF16>), grid, dim3(64), 0, s, x, rw, tok_scale, M, L.H, L.E, logits);
    else if (L.rdt == DT_Q8)
        launch_kernel((k_router_gemv<XDT, DT_Q8>), grid, dim3(64), 0, s, x, rw, tok_scale, M, L.H, L.E, logits);
    else
        launch_kernel((k_router_gemv<XDT, DT_F32>), grid, dim3(64), 0, s, x, rw, tok_scale, M, L.H, L.E, logits);
}

hipError_t launch_router(const Layer &L, const void *x, const RouterW &rw, const float *tok_scale,
                         int M, float *logits, hipStream_t s) {
    if (L.xdt == DT_BF16) router_gemv_rdt<DT_BF16>(L, x, rw, tok_scale, M, logits, s);
    else router_gemv_rdt<DT_F32>(L, x, rw, tok_scale, M, logits, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------- wave top-k
__global__ __launch_bounds__(256) void k_topk(const float *logits, const float *bias, int M, int E,
                                              int k, int select, int bias_mode, int32_t *ids,
                                              float *w) {
    __shared__ __align__(16) uint64_t s_words[4][kWave];
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    const int lane = threadIdx.x & 63;
    if (t >= M) return;
    topk_wave(logits + (size_t)t * E, bias, E, k, select, bias_mode, lane, ids + (size_t)t * k,
              w + (size_t)t * k, s_words[wave]);
}

hipError_t launch_topk(const Layer &L, const float *logits, const float *bias, int M, int32_t *ids,
                       float *w, hipStream_t s) {
    launch_kernel(k_topk, dim3((M + 3) / 4), dim3(256), 0, s, logits, L.bias_mode ? bias : nullptr,
                       M, L.E, L.k, L.select, L.bias_mode, ids, w);
    return hipGetLastError();
}

// ------------------------------------------- top-k with counts, then scatter
// The routing of the layer call beyond the small-batch route.  k_topk_hist:
// one wave per token, kTkWaves tokens a workgroup.  A token's logits are the
// sum of S slices of partial logits (slice order), times its token scale
// when there is one (S = 1 and no scale after the GEMV router); the picks go
// to ids and w as in k_topk, and the workgroup's expert counts (LDS atomics,
// then one row of `hist` [G][E]) feed the scatter.  k_scatter: each
// workgroup takes the routes of as many consecutive top-k workgroups as fit
// 1024 threads, one route a thread.  From `hist` it forms each expert's
// total and its routes before the workgroup's first route; offsets are the
// exclusive scan of the totals.  Lanes holding the same expert find each
// other with 8 ballots, the waves' counts are scanned in LDS, and the routes
// keep their order within an expert.  Workgroup 0 writes the counts,
// offsets, the active-expert list and the tile list.  (Against k_topk and
// the single-workgroup k_permute, which the stage-wise entry points keep:
// Qwen3-shaped M = 2048, 8.5 + 7.6 against 5.4 + 18.9 us; Mixtral-shaped
// M = 512, 5.1 + 6.6 against 4.8 + 7.0 us.)
constexpr int kTkWaves = 16;

// The lane's logits (expert lane + 64 c, c < NC) as sums of the S slices
// p[0], p[slab], .. in slice order.  Each group of 8 slices is loaded for
// every c before any is added (indexes clamped, extra values unused).
template <int NC>
__device__ inline void sum_slices(const float *row, size_t slab, int S, int E, int lane, float (&v)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; c++) v[c] = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float q[NC][8];
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int e = min(lane + kWave * c, E - 1);
#pragma unroll
            for (int u = 0; u < 8; u++) q[c][u] = row[(size_t)min(s0 + u, S - 1) * slab + e];
        }
#pragma unroll
        for (int c = 0; c < NC; c++)
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (s0 + u < S) v[c] = (s0 + u == 0) ? q[c][u] : v[c] + q[c][u];
    }
}

__global__ __launch_bounds__(kTkWaves * kWave) void k_topk_hist(const float *part, int S, const float *tok_scale,
                                                                const float *bias, int M, int E, int k, int select,
                                                                int bias_mode, int32_t *ids, float *w,
                                                                int32_t *hist, const float *sqp, int H, float eps,
                                                                float *scale_out) {
    __shared__ __align__(16) uint64_t s_words[kTkWaves][kWave];
    __shared__ int s_hist[kMaxE];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTkWaves + wave;
    for (int e = threadIdx.x; e < E; e += kTkWaves * kWave) s_hist[e] = 0;
    __syncthreads();
    if (t < M) {
        const size_t slab = (size_t)M * E;
        const float *lrow = part + (size_t)t * E;
        const bool scaled = tok_scale || sqp;
        float sc = tok_scale ? tok_scale[t] : 1.0f;
        if (sqp) {
            // the pre-norm's scale from the router's per-slice sums of
            // squares: lane s loads slice s (slices past 64 added in turn),
            // then a wave sum
            float ss = 0.f;
            for (int s2 = lane; s2 < S; s2 += kWave) ss += sqp[(size_t)s2 * M + t];
            ss = wave_sum(ss);
            sc = 1.0f / sqrtf(ss / (float)H + eps);
            if (lane == 0) scale_out[t] = sc;
        }
        int32_t *ids_row = ids + (size_t)t * k;
        float *w_row = w + (size_t)t * k;
        if (E <= kWave) {
            const int e = min(lane, E - 1);
            float lv1[1];
            sum_slices<1>(lrow, slab, S, E, lane, lv1);
            const float lv = scaled ? lv1[0] * sc : lv1[0];
            const float bv = bias ? bias[e] : 0.f;
            const LanePick p = topk_lane_small(lv, bv, E, k, select, bias_mode, lane, s_words[wave]);
            if (p.pick) {
                ids_row[p.rank] = lane;
                w_row[p.rank] = p.w;
                atomicAdd(&s_hist[lane], 1);
            }
        } else {
            float lv[kKeysPerLane], bv[kKeysPerLane];
            if (E <= 2 * kWave) {
                float l2[2];
                sum_slices<2>(lrow, slab, S, E, lane, l2);
                lv[0] = l2[0];
                lv[1] = l2[1];
                lv[2] = lv[3] = 0.f;
            } else {
                sum_slices<kKeysPerLane>(lrow, slab, S, E, lane, lv);
            }
#pragma unroll
            for (int c = 0; c < kKeysPerLane; c++) {
                const int e = min(lane + kWave * c, E - 1);
                if (scaled) lv[c] *= sc;
                bv[c] = bias && kWave * c < E ? bias[e] : 0.f;
            }
            int id;
            float wt;
            topk_wave_vals(lv, bv, E, k, select, bias_mode, lane, &id, &wt);
            if (lane < k) {
                ids_row[lane] = id;
                w_row[lane] = wt;
                atomicAdd(&s_hist[id], 1);
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kTkWaves * kWave) hist[(size_t)blockIdx.x * E + e] = s_hist[e];
}

hipError_t launch_topk_hist(const Layer &L, const float *part, int S, const float *tok_scale, const float *bias,
                            int M, int32_t *ids, float *w, int32_t *hist, hipStream_t s, const float *sqp,
                            float *scale_out) {
    if (sqp && !scale_out) return hipErrorInvalidValue;
    launch_kernel(k_topk_hist, dim3((M + kTkWaves - 1) / kTkWaves), dim3(kTkWaves * kWave), 0, s, part, S,
                  tok_scale, L.bias_mode ? bias : nullptr, M, L.E, L.k, L.select, L.bias_mode, ids, w, hist, sqp,
                  L.H, L.eps, scale_out);
    return hipGetLastError();
}

int topk_hist_groups(int M) { return (M + kTkWaves - 1) / kTkWaves; }

// ---------------------------------------------------------------- permutation
// One workgroup of NW waves.  Wave w owns a contiguous slice of routes.
//  1. per-wave expert histogram in LDS;
//  2. per expert, the exclusive sum over waves (so slices keep their order)
//     and the total; an exclusive scan over experts gives offsets;
//  3. each wave walks its slice 64 routes at a time; lanes holding the same
//     expert find each other with 8 ballots (one per bit of the id) and take
//     consecutive places in lane order, which keeps the scatter stable;
//  4. the touched-expert list and the GEMM tile list come from the counts.
// ids outside 0..E-1 get no place, so every write stays in bounds whatever
// the caller passes.
struct PermuteOut {
    int32_t *counts, *offsets, *sorted, *route_pos, *active, *tiles;
    int tile_rows;
};

template <int NW>
struct PermuteSmem {
    int hist[NW][kMaxE];
    int cnt[kMaxE];
    int off[kMaxE + 1];
    int scan[kMaxE + 1];
};


// Touched-expert list and GEMM tile list.  Tile list layout (E experts):
//   tiles[0]           number of tiles T
//   tiles[1 + e]       first tile of expert e (e = 0..E; tiles[1 + E] = T)
//   tiles[2 + E + 2i]  expert of tile i;  tiles[3 + E + 2i]  its first sorted row
// An expert's tiles are consecutive, tile_rows rows each (the last ragged).
__device__ void write_plan(int E, int tile_rows, const int *cnt, const int *off, int *scan_lds,
                           int32_t *active, int32_t *tiles) {
    const int tid = threadIdx.x;
    const int c = tid < E ? cnt[tid] : 0;
    int n_active;
    const int ai = block_scan_256(c > 0 ? 1 : 0, scan_lds, &n_active);
    if (tid < E && c > 0) active[1 + ai] = tid;
    if (tid == 0) active[0] = n_active;
    if (tiles) {
        int n_tiles;
        const int nt = (c + tile_rows - 1) / tile_rows;
        const int ti = block_scan_256(nt, scan_lds, &n_tiles);
        int32_t *pairs = tiles + 2 + E;
        if (tid < E) {
            tiles[1 + tid] = ti;
            for (int j = 0; j < nt; j++) {
                pairs[2 * (ti + j)] = tid;
                pairs[2 * (ti + j) + 1] = off[tid] + j * tile_rows;
            }
        }
        if (tid == 0) {
            tiles[0] = n_tiles;
            tiles[1 + E] = n_tiles;
        }
    }
}

constexpr int kPermChunk = 16; // route ids per lane loaded together

template <int NW>
__device__ void permute_block(const int32_t *ids, int R, int E, const PermuteOut &o, PermuteSmem<NW> &sm) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63;
    for (int i = tid; i < NW * kMaxE; i += NW * kWave) (&sm.hist[0][0])[i] = 0;
    __syncthreads();
    const int per = (((R + NW - 1) / NW) + 63) / 64 * 64;
    const int r0 = min(R, wv * per), r1 = min(R, r0 + per);
    // ids of routes base + 64 j + lane, j < kPermChunk, all loads issued first
    // (index clamped into the wave's range; -1 past its end)
    auto load_chunk = [&](int base, int (&ev)[kPermChunk]) {
#pragma unroll
        for (int j = 0; j < kPermChunk; j++) ev[j] = ids[min(base + j * kWave + lane, r1 - 1)];
#pragma unroll
        for (int j = 0; j < kPermChunk; j++)
            if (base + j * kWave + lane >= r1) ev[j] = -1;
    };
    // a wave whose routes fit one chunk keeps its ids in registers for the
    // scatter below
    const bool one_chunk = per <= kWave * kPermChunk;
    int ev[kPermChunk];
    for (int base = r0; base < r1; base += kWave * kPermChunk) {
        load_chunk(base, ev);
#pragma unroll
        for (int j = 0; j < kPermChunk; j++)
            if (ev[j] >= 0 && ev[j] < E) atomicAdd(&sm.hist[wv][ev[j]], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += NW * kWave) {
        int sacc = 0;
        for (int w = 0; w < NW; w++) {
            const int c = sm.hist[w][e];
            sm.hist[w][e] = sacc;
            sacc += c;
        }
        sm.cnt[e] = sacc;
    }
    __syncthreads();
    int total;
    const int ex = block_scan_256(tid < E ? sm.cnt[tid] : 0, sm.scan, &total);
    if (tid < E) {
        sm.off[tid] = ex;
        o.counts[tid] = sm.cnt[tid];
        o.offsets[tid] = ex;
    }
    if (tid == 0) {
        sm.off[E] = total;
        o.offsets[E] = total;
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int cb = r0; cb < r1; cb += kWave * kPermChunk) {
        if (!one_chunk) load_chunk(cb, ev);
#pragma unroll
        for (int j = 0; j < kPermChunk; j++) {
            if (cb + j * kWave >= r1) break; // wave-uniform: the rest of the chunk is past the range
            const int r = cb + j * kWave + lane;
            int e = ev[j];
            const bool valid = e >= 0 && e < E;
            if (!valid) e = 0;
            uint64_t peers = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; b++) {
                const uint64_t m = __ballot(valid && ((e >> b) & 1));
                peers &= ((e >> b) & 1) ? m : ~m;
            }
            const int rank = __popcll(peers & lt_mask);
            if (valid) {
                const int pos = sm.off[e] + sm.hist[wv][e] + rank;
                o.sorted[pos] = r;
                o.route_pos[r] = pos;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) sm.hist[wv][e] += __popcll(peers);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    write_plan(E, o.tile_rows, sm.cnt, sm.off, sm.scan, o.active, o.tiles);
}

constexpr int kPermWaves = 16;

__global__ __launch_bounds__(kPermWaves * kWave) void k_permute(const int32_t *ids, int R, int E, PermuteOut o) {
    __shared__ PermuteSmem<kPermWaves> sm;
    permute_block<kPermWaves>(ids, R, E, o, sm);
}

__global__ __launch_bounds__(256) void k_plan_from_offsets(int E, int tile_rows, const int32_t *offsets,
                                                          int32_t *active, int32_t *tiles) {
    __shared__ int cnt[kMaxE];
    __shared__ int off[kMaxE + 1];
    __shared__ int scan[kMaxE + 1];
    const int tid = threadIdx.x;
    if (tid < E) {
        off[tid] = offsets[tid];
        cnt[tid] = offsets[tid + 1] - offsets[tid];
    }
    __syncthreads();
    write_plan(E, tile_rows, cnt, off, scan, active, tiles);
}

hipError_t launch_permute(int E, int R, int tile_rows, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *sorted, int32_t *route_pos, int32_t *active,
                          int32_t *tiles, hipStream_t s) {
    PermuteOut o{counts, offsets, sorted, route_pos, active, tiles, tile_rows};
    launch_kernel(k_permute, dim3(1), dim3(kPermWaves * kWave), 0, s, ids, R, E, o);
    return hipGetLastError();
}

hipError_t launch_plan_from_offsets(int E, int tile_rows, const int32_t *offsets, int32_t *active,
                                    int32_t *tiles, hipStream_t s) {
    launch_kernel(k_plan_from_offsets, dim3(1), dim3(256), 0, s, E, tile_rows, offsets, active,
                       tiles);
    return hipGetLastError();
}

constexpr int kScThreads = 1024;

__global__ __launch_bounds__(kScThreads) void k_scatter(const int32_t *ids, const int32_t *hist, int G, int R,
                                                         int E, int k, PermuteOut o) {
    __shared__ int s_tot[kMaxE], s_bef[kMaxE], s_off[kMaxE + 1], s_scan[kMaxE + 1];
    __shared__ int s_wc[kScThreads / kWave][kMaxE];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rc = kTkWaves * k;                  // routes of one top-k workgroup
    const int ct = max(1, kScThreads / rc);       // top-k workgroups a scatter workgroup
    const int g0 = blockIdx.x * ct;
    for (int i = tid; i < kMaxE; i += kScThreads) s_tot[i] = s_bef[i] = 0;
    for (int i = tid; i < (kScThreads / kWave) * kMaxE; i += kScThreads) (&s_wc[0][0])[i] = 0;
    __syncthreads();
    // totals and counts before this workgroup: thread q E + e (q < P) sums
    // rows q, q + P, .. of expert e's column of hist, 8 loads at a time
    {
        const int P = max(1, min(kScThreads / E, G));
        if (tid < P * E) {
            const int q = tid / E, e = tid - q * E;
            int tot = 0, bef = 0;
            for (int g = q; g < G; g += 8 * P) {
                int c[8];
#pragma unroll
                for (int u = 0; u < 8; u++) c[u] = g + u * P < G ? hist[(size_t)(g + u * P) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    tot += c[u];
                    if (g + u * P < g0) bef += c[u];
                }
            }
            atomicAdd(&s_tot[e], tot);
            atomicAdd(&s_bef[e], bef);
        }
    }
    __syncthreads();
    int total;
    const int ex = block_scan_256(tid < E ? s_tot[tid] : 0, s_scan, &total);
    if (tid < E) s_off[tid] = ex;
    if (tid == 0) s_off[E] = total;
    // this thread's route, and its rank among the wave's lanes of the same expert
    const int r = g0 * rc + tid;
    const bool have = tid < ct * rc && r < R;
    int e = have ? ids[r] : -1;
    const bool valid = have && e >= 0 && e < E;
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const uint64_t m = __ballot(valid && ((e >> b) & 1));
        peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) s_wc[wv][e] = __popcll(peers);
    __syncthreads();
    if (tid < E) {
        int acc = s_off[tid] + s_bef[tid];
        for (int w2 = 0; w2 < kScThreads / kWave; w2++) {
            const int c = s_wc[w2][tid];
            s_wc[w2][tid] = acc;
            acc += c;
        }
    }
    __syncthreads();
    if (valid) {
        const int pos = s_wc[wv][e] + rank;
        o.sorted[pos] = r;
        o.route_pos[r] = pos;
    }
    if (blockIdx.x == 0) {
        if (tid < E) {
            o.counts[tid] = s_tot[tid];
            o.offsets[tid] = s_off[tid];
        }
        if (tid == 0) o.offsets[E] = s_off[E];
        write_plan(E, o.tile_rows, s_tot, s_off, s_scan, o.active, o.tiles);
    }
}

hipError_t launch_scatter(int E, int M, int k, int tile_rows, const int32_t *ids, const int32_t *hist,
                          int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *route_pos, int32_t *active,
                          int32_t *tiles, hipStream_t s) {
    PermuteOut o{counts, offsets, sorted, route_pos, active, tiles, tile_rows};
    const int G = topk_hist_groups(M), ct = std::max(1, kScThreads / (kTkWaves * k));
    launch_kernel(k_scatter, dim3((G + ct - 1) / ct), dim3(kScThreads), 0, s, ids, hist, G, M * k, E, k, o);
    return hipGetLastError();
}

// ----------------------------------------------------- small-batch route
// Two launches for M <= kSmallM tokens.  The router kernel: workgroup (e, g)
// computes expert e's logits for tokens 4g..4g+3 (its waves split the row;
// partial dots meet in LDS).  Then one workgroup loads every logit into LDS
// with one round of loads, runs each token's top-k (one wave per token) and
// the permutation.  (Handing over inside one kernel instead, the last
// workgroup to take a ticket after a device-scope release doing the select,
// measured about 6 us slower with 128 workgroups than the second launch.)
constexpr int kSmallM = 16;

struct RouteSmallArgs {
    const void *x;
    RouterW rw;
    const float *bias, *tok_scale;
    int M, H, E, k, select, bias_mode;
    float *logits;
    int32_t *ids;
    float *w;
    PermuteOut o;
};

constexpr int kRouteWaves = 4;
constexpr int kRouteTM = 4;    // tokens per workgroup
constexpr int kSmallRoutes = kSmallM * 8; // routes of a small batch (top_k <= 8)

template <int XDT, int RDT>
__global__ __launch_bounds__(kRouteWaves * kWave) void k_router_small(RouteSmallArgs a) {
    __shared__ float s_part[kRouteWaves][kRouteTM];
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int e = blockIdx.x, t0 = blockIdx.y * kRouteTM;
    const int nt = min(kRouteTM, a.M - t0);
    const int nch = a.H / 8;
    const int cb = wave * nch / kRouteWaves, ce = (wave + 1) * nch / kRouteWaves;
    float acc[kRouteTM];
    router_dots<XDT, RDT, kRouteTM, 2>(a.x, router_row<RDT>(a.rw, e, a.H), router_srow(a.rw, e, a.H), a.rw.xs, a.H,
                                       t0, nt, lane, acc, cb, ce);
    if (lane == 0)
#pragma unroll
        for (int tm = 0; tm < kRouteTM; tm++) s_part[wave][tm] = acc[tm];
    __syncthreads();
    if (threadIdx.x < nt) {
        const int t = t0 + threadIdx.x;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kRouteWaves; w++) v += s_part[w][threadIdx.x];
        if (a.tok_scale) v *= a.tok_scale[t];
        a.logits[(size_t)t * a.E + e] = v;
    }
}

// The selection as one workgroup of kSmallM waves (select_small; the
// streamed gate/up kernel runs the same selection in its prologue instead,
// when it takes the batch).  (The per-expert bit masks replaced a pass over
// all routes per route and per expert: gpt-oss-shaped M = 16, 6.2 us with
// those passes.)
constexpr int kSelWaves = kSmallM;
static_assert(kSmallM <= kSelMaxM, "select_small takes at most kSelMaxM tokens");

__global__ __launch_bounds__(kSelWaves * kWave) void k_select_small(RouteSmallArgs a) {
    __shared__ int s_ids[kSmallRoutes];
    __shared__ float s_logit[kSmallM * kMaxE];
    __shared__ float s_bias[kMaxE];
    __shared__ uint32_t s_mask[kMaxE];
    __shared__ int s_off[kMaxE + 1], s_act[kMaxE + 1];
    __shared__ int s_scan[4];
    __shared__ __align__(16) uint64_t s_words[kSelWaves][kWave];
    const SelectSmall sel{a.logits, a.bias, a.M, a.E, a.k, a.select, a.bias_mode, a.ids, a.w,
                          a.o.counts, a.o.offsets, a.o.sorted, a.o.route_pos, a.o.active};
    select_small(sel, true, s_logit, s_bias, s_mask, s_ids, s_scan, &s_words[0][0], s_off, s_act, nullptr);
}

// One expert (a dense layer, k = 1): every route is expert 0 with weight 1
// whatever its logit (a softmax over one logit, or one sigmoid score
// normalised by itself), so the forward call runs no router.  The plan is
// the identity order, one count, one touched expert and ceil(M / tile_rows)
// tiles (pairs at tiles + 2 + E, E = 1).
__global__ __launch_bounds__(256) void k_route_one(int M, int tile_rows, int32_t *ids, float *w, int32_t *counts,
                                                   int32_t *offsets, int32_t *sorted, int32_t *route_pos,
                                                   int32_t *active, int32_t *tiles) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < M) {
        ids[t] = 0;
        w[t] = 1.0f;
        sorted[t] = t;
        route_pos[t] = t;
    }
    const int T = tiles ? (M + tile_rows - 1) / tile_rows : 0;
    if (t < T) {
        tiles[3 + 2 * t] = 0;
        tiles[4 + 2 * t] = t * tile_rows;
    }
    if (t == 0) {
        counts[0] = M;
        offsets[0] = 0;
        offsets[1] = M;
        active[0] = 1;
        active[1] = 0;
        if (tiles) {
            tiles[0] = T;
            tiles[1] = 0;
            tiles[2] = T;
        }
    }
}

hipError_t launch_route_one(int M, int tile_rows, int32_t *ids, float *w, int32_t *counts, int32_t *offsets,
                            int32_t *sorted, int32_t *route_pos, int32_t *active, int32_t *tiles, hipStream_t s) {
    if (M <= 0 || tile_rows <= 0) return hipErrorInvalidValue;
    launch_kernel(k_route_one, dim3((M + 255) / 256), dim3(256), 0, s, M, tile_rows, ids, w, counts, offsets, sorted,
                  route_pos, active, tiles);
    return hipGetLastError();
}

int route_small_max_tokens() { return kSmallM; }

template <int XDT>
static void router_small_rdt(const Layer &L, const RouteSmallArgs &a, hipStream_t s) {
    const dim3 grid(L.E, (a.M + kRouteTM - 1) / kRouteTM), block(kRouteWaves * kWave);
    if (L.rdt == DT_BF16) launch_kernel((k_router_small<XDT, DT_BF16>), grid, block, 0, s, a);
    else if (L.rdt == DT_Q8) launch_kernel((k_router_small<XDT, DT_Q8>), grid, block, 0, s, a);
    else launch_kernel((k_router_small<XDT, DT_F32>), grid, block, 0, s, a);
}

static void router_small_dispatch(const Layer &L, const RouteSmallArgs &a, hipStream_t s) {
    if (L.xdt == DT_BF16) router_small_rdt<DT_BF16>(L, a, s);
    else router_small_rdt<DT_F32>(L, a, s);
}

hipError_t launch_route_small(const Layer &L, const void *x, const RouterW &rw, const float *bias,
                              const float *tok_scale, int M, float *logits, int32_t *ids, float *w,
                              int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *route_pos,
                              int32_t *active, hipStream_t s) {
    if (M > kSmallM || M * L.k > kSmallRoutes) return hipErrorInvalidValue;
    const RouteSmallArgs a{x, rw, L.bias_mode ? bias : nullptr, tok_scale, M, L.H, L.E, L.k, L.select,
                           L.bias_mode, logits, ids, w,
                           PermuteOut{counts, offsets, sorted, route_pos, active, nullptr, 1}};
    router_small_dispatch(L, a, s);
    launch_kernel(k_select_small, dim3(1), dim3(kSelWaves * kWave), 0, s, a);
    return hipGetLastError();
}


hipError_t launch_router_small(const Layer &L, const void *x, const RouterW &rw, const float *tok_scale,
                               int M, float *logits, hipStream_t s) {
    if (M > kSmallM) return hipErrorInvalidValue;
    const RouteSmallArgs a{x, rw, nullptr, tok_scale, M, L.H, L.E, L.k, L.select, L.bias_mode, logits,
                           nullptr, nullptr, PermuteOut{}};
    router_small_dispatch(L, a, s);
    return hipGetLastError();
}

} // namespace moe
