// Routing kernels: RMS pre-norm scale, router GEMV, wave top-k + softmax, and
// the expert histogram / scan / stable scatter of the routes.
#include "common.h"
#include "launch.h"

namespace moe {

// 8 consecutive elements of a row stored as fp32 or bf16, as floats.
template <int DT>
__device__ __forceinline__ void load8(const void *row, int c8, float *v) {
    if constexpr (DT == DT_BF16) {
        u32x4 q = reinterpret_cast<const u32x4 *>(row)[c8];
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(row) + 2 * c8;
        f32x4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// ------------------------------------------------------------------ pre-norm
// scale[t] = 1 / sqrt(mean_i x[t][i]^2 + eps); one wave per token.
template <int XDT>
__global__ __launch_bounds__(256) void k_rms_scale(const void *x, int M, int H, float eps, float *scale) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= M) return;
    const char *row = reinterpret_cast<const char *>(x) + (size_t)t * H * (XDT == DT_BF16 ? 2 : 4);
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
        hipLaunchKernelGGL(k_rms_scale<DT_BF16>, grid, dim3(256), 0, s, x, M, L.H, L.eps, scale);
    else
        hipLaunchKernelGGL(k_rms_scale<DT_F32>, grid, dim3(256), 0, s, x, M, L.H, L.eps, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------- router GEMV
// logits[t][e] = scale[t] * sum_i x[t][i] * router[e][i].  One wave per
// (expert, group of TM tokens); lanes stride the row in 8-element pieces.
constexpr int kRouterTM = 8;

template <int XDT, int RDT>
__global__ __launch_bounds__(64) void k_router_gemv(const void *x, const void *router,
                                                    const float *tok_scale, int M, int H, int E,
                                                    float *logits) {
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * kRouterTM;
    const int lane = threadIdx.x;
    const int nt = min(kRouterTM, M - t0);
    const size_t xrow_bytes = (size_t)H * (XDT == DT_BF16 ? 2 : 4);
    const char *wrow = reinterpret_cast<const char *>(router) + (size_t)e * H * (RDT == DT_BF16 ? 2 : 4);
    const char *xbase = reinterpret_cast<const char *>(x) + (size_t)t0 * xrow_bytes;
    float acc[kRouterTM];
#pragma unroll
    for (int i = 0; i < kRouterTM; i++) acc[i] = 0.f;
    for (int c = lane; c < H / 8; c += kWave) {
        float w[8];
        load8<RDT>(wrow, c, w);
#pragma unroll
        for (int tm = 0; tm < kRouterTM; tm++) {
            if (tm < nt) {
                float xv[8];
                load8<XDT>(xbase + tm * xrow_bytes, c, xv);
#pragma unroll
                for (int i = 0; i < 8; i++) acc[tm] = fmaf(w[i], xv[i], acc[tm]);
            }
        }
    }
#pragma unroll
    for (int tm = 0; tm < kRouterTM; tm++) {
        if (tm < nt) {
            float v = wave_sum(acc[tm]);
            if (tok_scale) v *= tok_scale[t0 + tm];
            if (lane == 0) logits[(size_t)(t0 + tm) * E + e] = v;
        }
    }
}

hipError_t launch_router(const Layer &L, const void *x, const void *router, const float *tok_scale,
                         int M, float *logits, hipStream_t s) {
    dim3 grid(L.E, (M + kRouterTM - 1) / kRouterTM);
    if (L.xdt == DT_BF16 && L.rdt == DT_BF16)
        hipLaunchKernelGGL((k_router_gemv<DT_BF16, DT_BF16>), grid, dim3(64), 0, s, x, router, tok_scale, M, L.H, L.E, logits);
    else if (L.xdt == DT_BF16)
        hipLaunchKernelGGL((k_router_gemv<DT_BF16, DT_F32>), grid, dim3(64), 0, s, x, router, tok_scale, M, L.H, L.E, logits);
    else if (L.rdt == DT_BF16)
        hipLaunchKernelGGL((k_router_gemv<DT_F32, DT_BF16>), grid, dim3(64), 0, s, x, router, tok_scale, M, L.H, L.E, logits);
    else
        hipLaunchKernelGGL((k_router_gemv<DT_F32, DT_F32>), grid, dim3(64), 0, s, x, router, tok_scale, M, L.H, L.E, logits);
    return hipGetLastError();
}

// ---------------------------------------------------------------- wave top-k
// One wave per token; lane l holds experts l, l+64, l+128, l+192.
// Selection key s = logit (+ bias for LOGIT and SELECT_ONLY); softmax input
// u = logit (+ bias for LOGIT).  k rounds of a wave argmax on the
// order-preserving key, ties to the lower expert id.
constexpr int kMaxE = 256;
constexpr int kKeysPerLane = kMaxE / kWave;

__global__ __launch_bounds__(256) void k_topk(const float *logits, const float *bias, int M, int E,
                                              int k, int select, int bias_mode, int32_t *ids,
                                              float *w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= M) return;
    const float *lrow = logits + (size_t)t * E;
    uint32_t key[kKeysPerLane];
    float u[kKeysPerLane];
#pragma unroll
    for (int c = 0; c < kKeysPerLane; c++) {
        const int e = lane + kWave * c;
        if (e < E) {
            const float l = lrow[e];
            const float b = bias ? bias[e] : 0.f;
            const float sk = bias_mode != 0 ? l + b : l;
            u[c] = bias_mode == 1 ? l + b : l;
            key[c] = order_key(sk);
        } else {
            u[c] = -INFINITY;
            key[c] = 0u;
        }
    }
    uint32_t taken = 0u;
    int my_id = 0;          // lane j keeps the id chosen in round j
    float my_u = -INFINITY; // and its softmax input
    for (int j = 0; j < k; j++) {
        uint32_t bk = 0u;
        int bid = 0x7fffffff;
        float bu = 0.f;
#pragma unroll
        for (int c = 0; c < kKeysPerLane; c++) {
            const int e = lane + kWave * c;
            const bool cand = e < E && !((taken >> c) & 1u);
            if (cand && (bid == 0x7fffffff || key[c] > bk)) { bk = key[c]; bid = e; bu = u[c]; }
        }
        const uint32_t mk = wave_max_u32(bid == 0x7fffffff ? 0u : bk);
        const int win = wave_min_i32((bid != 0x7fffffff && bk == mk) ? bid : 0x7fffffff);
        if ((win & 63) == lane) taken |= 1u << (win >> 6);
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bid == win ? bu : 0.f), win & 63));
        if (lane == j) { my_id = win; my_u = wu; }
    }
    float wj;
    if (select == 0) {
        const float m = wave_max(lane < k ? my_u : -INFINITY);
        const float ex = lane < k ? expf(my_u - m) : 0.f;
        const float z = wave_sum(ex);
        wj = ex / z;
    } else {
        float m = -INFINITY;
#pragma unroll
        for (int c = 0; c < kKeysPerLane; c++) m = fmaxf(m, u[c]);
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int c = 0; c < kKeysPerLane; c++)
            if (lane + kWave * c < E) z += expf(u[c] - m);
        z = wave_sum(z);
        wj = expf(my_u - m) / z;
    }
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        w[(size_t)t * k + lane] = wj;
    }
}

hipError_t launch_topk(const Layer &L, const float *logits, const float *bias, int M, int32_t *ids,
                       float *w, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3((M + 3) / 4), dim3(256), 0, s, logits, L.bias_mode ? bias : nullptr,
                       M, L.E, L.k, L.select, L.bias_mode, ids, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------- permutation
// One workgroup of 16 waves.  Wave w owns a contiguous slice of routes.
//  1. per-wave expert histogram in LDS;
//  2. per expert, the exclusive sum over waves (so slices keep their order)
//     and the total; an exclusive scan over experts gives offsets;
//  3. each wave walks its slice 64 routes at a time; lanes holding the same
//     expert find each other with 8 ballots (one per bit of the id) and take
//     consecutive places in lane order, which keeps the scatter stable;
//  4. the touched-expert list and the GEMM tile list come from the counts.
constexpr int kPermWaves = 16;
constexpr int kPermThreads = kPermWaves * kWave;

// Exclusive scan of v over threads 0..255 (others pass 0); returns the
// thread's exclusive prefix and the total in *total.  All threads call it.
__device__ int block_scan_256(int v, int *lds /*[256+1]*/, int *total) {
    const int tid = threadIdx.x;
    if (tid < 256) lds[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        int add = 0;
        if (tid < 256 && tid >= off) add = lds[tid - off];
        __syncthreads();
        if (tid < 256) lds[tid] += add;
        __syncthreads();
    }
    const int incl = tid < 256 ? lds[tid] : 0;
    *total = lds[255];
    __syncthreads();
    return incl - v;
}

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
        if (tid < E)
            for (int j = 0; j < nt; j++) {
                tiles[1 + 2 * (ti + j)] = tid;
                tiles[2 + 2 * (ti + j)] = off[tid] + j * tile_rows;
            }
        if (tid == 0) tiles[0] = n_tiles;
    }
}

__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t *ids, int R, int E, int tile_rows,
                                                         int32_t *counts, int32_t *offsets,
                                                         int32_t *sorted, int32_t *route_pos,
                                                         int32_t *active, int32_t *tiles) {
    __shared__ int hist[kPermWaves][kMaxE];
    __shared__ int cnt[kMaxE];
    __shared__ int off[kMaxE + 1];
    __shared__ int scan[kMaxE + 1];
    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63;
    for (int i = tid; i < kPermWaves * kMaxE; i += kPermThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const int per = (((R + kPermWaves - 1) / kPermWaves) + 63) / 64 * 64;
    const int r0 = min(R, wv * per), r1 = min(R, r0 + per);
    // ids outside 0..E-1 are skipped (they get no place), which keeps every
    // write in bounds whatever the caller passes.
    for (int r = r0 + lane; r < r1; r += kWave) {
        const int e = ids[r];
        if (e >= 0 && e < E) atomicAdd(&hist[wv][e], 1);
    }
    __syncthreads();
    if (tid < E) {
        int sacc = 0;
        for (int w = 0; w < kPermWaves; w++) {
            const int c = hist[w][tid];
            hist[w][tid] = sacc;
            sacc += c;
        }
        cnt[tid] = sacc;
    }
    __syncthreads();
    int total;
    const int ex = block_scan_256(tid < E ? cnt[tid] : 0, scan, &total);
    if (tid < E) {
        off[tid] = ex;
        counts[tid] = cnt[tid];
        offsets[tid] = ex;
    }
    if (tid == 0) {
        off[E] = total;
        offsets[E] = total;
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = r0; base < r1; base += kWave) {
        const int r = base + lane;
        int e = r < r1 ? ids[r] : -1;
        const bool valid = e >= 0 && e < E;
        if (!valid) e = 0;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const uint64_t m = __ballot(valid && ((e >> b) & 1));
            peers &= ((e >> b) & 1) ? m : ~m;
        }
        const int rank = __popcll(peers & lt_mask);
        int pos = 0;
        if (valid) {
            pos = off[e] + hist[wv][e] + rank;
            sorted[pos] = r;
            route_pos[r] = pos;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == 0) hist[wv][e] += __popcll(peers);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    write_plan(E, tile_rows, cnt, off, scan, active, tiles);
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
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), 0, s, ids, R, E, tile_rows, counts,
                       offsets, sorted, route_pos, active, tiles);
    return hipGetLastError();
}

hipError_t launch_plan_from_offsets(int E, int tile_rows, const int32_t *offsets, int32_t *active,
                                    int32_t *tiles, hipStream_t s) {
    hipLaunchKernelGGL(k_plan_from_offsets, dim3(1), dim3(256), 0, s, E, tile_rows, offsets, active,
                       tiles);
    return hipGetLastError();
}

} // namespace moe
