// Wave-level top-k with softmax weights (device code shared by the routing
// and the single-token expert kernels).
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxE = 256;
constexpr int kKeysPerLane = kMaxE / kWave;

// One wave selects the top-k experts of one token from its logit row.
// Lane l holds experts l, l+64, l+128, l+192.  Selection key
// s = logit (+ bias for LOGIT and SELECT_ONLY); softmax input u = logit
// (+ bias for LOGIT).  k rounds of a wave argmax on the order-preserving key,
// ties to the lower expert id.  On return lane j < k holds the j-th pick
// (descending key) in *id and its weight in *wt: softmax over the k picks
// (select 0), the all-expert softmax read at the pick (select 1), or, with
// sigmoid scores (select 2), the pick's score sigmoid(logit) divided by the
// sum of the picks' scores; there the bias (any bias mode) is added to the
// score for the selection only.
// (topk_wave_vals takes the lane's logits and biases already loaded: lv[c]
// and bv[c] for expert lane + 64 c, any value past E.)
__device__ inline void topk_wave_vals(const float (&lv)[kKeysPerLane], const float (&bv)[kKeysPerLane], int E,
                                      int k, int select, int bias_mode, int lane, int *id, float *wt) {
    uint32_t key[kKeysPerLane];
    float u[kKeysPerLane];
#pragma unroll
    for (int c = 0; c < kKeysPerLane; c++) {
        const int e = lane + kWave * c;
        if (e < E) {
            if (select == 2) {
                u[c] = 1.0f / (1.0f + expf(-lv[c]));
                key[c] = order_key(bias_mode != 0 ? u[c] + bv[c] : u[c]);
            } else {
                const float sk = bias_mode != 0 ? lv[c] + bv[c] : lv[c];
                u[c] = bias_mode == 1 ? lv[c] + bv[c] : lv[c];
                key[c] = order_key(sk);
            }
        } else {
            u[c] = -INFINITY;
            key[c] = 0u;
        }
    }
    uint32_t taken = 0u;
    int my_id = 0;
    float my_u = -INFINITY;
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
    if (select == 2) {
        const float z = wave_sum(lane < k ? my_u : 0.f);
        wj = my_u / z;
    } else if (select == 0) {
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
    *id = my_id;
    *wt = wj;
}

// The lane's logits and biases for topk_wave_vals (lv[c], bv[c]: expert
// lane + 64 c).  All loads are issued together (clamped index, masked in the
// selection); groups of 64 past E load nothing (every wave of a grid may run
// this on the same row, so each load is a hot cache line).
__device__ inline void topk_load(const float *lrow, const float *bias, int E, int lane,
                                 float (&lv)[kKeysPerLane], float (&bv)[kKeysPerLane]) {
#pragma unroll
    for (int c = 0; c < kKeysPerLane; c++) {
        lv[c] = bv[c] = 0.f;
        if (kWave * c < E) {
            const int e = min(lane + kWave * c, E - 1);
            lv[c] = lrow[e];
            bv[c] = bias ? bias[e] : 0.f;
        }
    }
}

__device__ inline void topk_wave_core(const float *lrow, const float *bias, int E, int k, int select,
                                      int bias_mode, int lane, int *id, float *wt) {
    float lv[kKeysPerLane], bv[kKeysPerLane];
    topk_load(lrow, bias, E, lane, lv, bv);
    topk_wave_vals(lv, bv, E, k, select, bias_mode, lane, id, wt);
}

// Top-k of at most 64 experts, one a lane (lane l holds expert l's logit lv
// and bias bv; lanes past E hold nothing).  Keys, softmax inputs and the
// three weight rules are those of topk_wave_vals.  Each lane writes one
// 64-bit word to `words` (the wave's own 64 entries in LDS, 16-byte aligned):
// its key in the high half and 64 - l in the low half, so that a larger word
// comes earlier in the selection order (descending key, ties to the lower id)
// and every valid expert's word is nonzero.  A lane's rank is the number of
// words larger than its own, and the picks are the valid lanes of rank < k:
// one pass over E words instead of k rounds of wave reductions.  Every lane
// must be active.  Returns, per lane, whether it is a pick, its rank (the
// pick's place in descending key order) and, for a pick, its weight.
struct LanePick {
    bool pick;
    int rank;
    float w;
};

__device__ inline LanePick topk_lane_small(float lv, float bv, int E, int k, int select, int bias_mode,
                                           int lane, uint64_t *words) {
    const bool valid = lane < E;
    float u, sk;
    if (select == 2) {
        u = 1.0f / (1.0f + expf(-lv));
        sk = bias_mode != 0 ? u + bv : u;
    } else {
        sk = bias_mode != 0 ? lv + bv : lv;
        u = bias_mode == 1 ? lv + bv : lv;
    }
    const uint64_t mine = valid ? ((uint64_t)order_key(sk) << 32) | (uint64_t)(kWave - lane) : 0ull;
    words[lane] = mine;
    // LDS accesses of one wave complete in issue order; the fences keep the
    // compiler from moving the reads above the write
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
    const u64x2 *w2 = reinterpret_cast<const u64x2 *>(words);
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < (E + 1) >> 1; j++) { // words past E are zero
        const u64x2 q = w2[j];
        rank += q.x > mine;
        rank += q.y > mine;
    }
    const bool pick = valid && rank < k;
    float w;
    if (select == 2) {
        w = u / wave_sum(pick ? u : 0.f);
    } else {
        const bool in = select == 0 ? pick : valid; // softmax over the picks, or over all experts
        const float m = wave_max(in ? u : -INFINITY);
        const float ex = in ? expf(u - m) : 0.f;
        w = ex / wave_sum(ex);
    }
    return LanePick{pick, rank, w};
}

// Rank of lane j's pick among the k picks in ascending expert id (lanes < k):
// the order in which a one-token batch lists its touched experts.
__device__ inline int pick_rank(int my_id, int k, int lane) {
    int rank = 0;
    for (int j = 0; j < k; j++) {
        const int other = __builtin_amdgcn_readlane(my_id, j);
        rank += other < my_id;
    }
    return lane < k ? rank : 0;
}

// Exclusive scan of v over threads 0..255 (others pass 0); returns the
// thread's exclusive prefix and the total in *total.  All threads of the
// block call it; the block has at least 256 threads.  Waves 0-3 scan their
// 64 values with shuffles, then add the totals of the waves before them.
__device__ inline int block_scan_256(int v, int *lds /*[>= 4]*/, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int x = tid < 256 ? v : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (wave < 4 && lane == kWave - 1) lds[wave] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) before += (w < wave) ? lds[w] : 0;
    *total = lds[0] + lds[1] + lds[2] + lds[3];
    __syncthreads();
    return tid < 256 ? x + before - v : 0;
}


// One wave per token.  Selection key s = logit (+ bias for LOGIT and
// SELECT_ONLY); softmax input u = logit (+ bias for LOGIT); descending key,
// ties to the lower expert id.  Up to 64 experts: one expert a lane and a
// rank count over the wave's words in LDS (`words`, 64 entries); more: lane
// l holds experts l, l+64, l+128, l+192 and k rounds of a wave argmax pick
// them.  Pick j (descending key) goes to ids_row[j] and w_row[j] (both skipped
// when ids_row is null) and to lds_ids[j] when given.
__device__ inline void topk_wave(const float *lrow, const float *bias, int E, int k, int select,
                          int bias_mode, int lane, int32_t *ids_row, float *w_row, uint64_t *words,
                          int *lds_ids = nullptr) {
    if (E <= kWave) {
        const int e = min(lane, E - 1);
        const float lv = lrow[e];
        const float bv = bias ? bias[e] : 0.f;
        const LanePick p = topk_lane_small(lv, bv, E, k, select, bias_mode, lane, words);
        if (p.pick) {
            if (ids_row) {
                ids_row[p.rank] = lane;
                w_row[p.rank] = p.w;
            }
            if (lds_ids) lds_ids[p.rank] = lane;
        }
        return;
    }
    int id;
    float wt;
    topk_wave_core(lrow, bias, E, k, select, bias_mode, lane, &id, &wt);
    if (lane < k) {
        if (ids_row) {
            ids_row[lane] = id;
            w_row[lane] = wt;
        }
        if (lds_ids) lds_ids[lane] = id;
    }
}


// The selection of a batch of M <= 16 tokens in one workgroup (at least
// max(M, 4) waves).  One wave per token for the top-k.  A token picks an
// expert at most once, so each expert's set of tokens is a bit mask (bit t:
// token t picked it), built with LDS atomic ORs: its population count is the
// expert's count, and a route (t, expert e) takes sorted place offsets[e]
// plus the number of earlier tokens in e's mask (routes grouped by expert,
// tokens ascending: a stable counting sort).  Offsets and the touched-expert
// list are block scans of the counts.  The workgroup's own copy of the
// result goes to LDS (s_off [E + 1], s_act [1 + E], s_tok [M * k]: the token
// of each sorted place, when given); with `writer` it is also written to
// global memory (ids, w [M][k]; counts [E]; offsets [E + 1]; sorted and
// route_pos [M * k]; active [1 + E]).  LDS scratch: s_logit [M * E], s_bias
// [E], s_mask [E], s_ids [M * k], s_scan [4], s_words [waves][64] (16-byte
// aligned).  Every thread of the workgroup calls it; it ends on a barrier.
constexpr int kSelMaxM = 16;
static_assert(kSelMaxM <= 32, "a token set is a 32-bit mask");
struct SelectSmall {
    const float *logits, *bias; // logits [M][E] fp32; bias [E] or null
    int M, E, k, select, bias_mode;
    int32_t *ids;
    float *w;
    int32_t *counts, *offsets, *sorted, *route_pos, *active;
};
__device__ inline void select_small(const SelectSmall &a, bool writer, float *s_logit, float *s_bias,
                                    uint32_t *s_mask, int *s_ids, int *s_scan, uint64_t *s_words, int *s_off,
                                    int *s_act, int *s_tok) {
    const int tid = threadIdx.x, nthr = blockDim.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6),
              lane = tid & 63;
    const int R = a.M * a.k;
    for (int i = tid; i < a.M * a.E; i += nthr) s_logit[i] = a.logits[i];
    if (a.bias)
        for (int i = tid; i < a.E; i += nthr) s_bias[i] = a.bias[i];
    for (int i = tid; i < a.E; i += nthr) s_mask[i] = 0u;
    __syncthreads();
    if (wave < a.M)
        topk_wave(s_logit + wave * a.E, a.bias ? s_bias : nullptr, a.E, a.k, a.select, a.bias_mode, lane,
                  writer ? a.ids + (size_t)wave * a.k : nullptr, writer ? a.w + (size_t)wave * a.k : nullptr,
                  s_words + (size_t)wave * kWave, s_ids + wave * a.k);
    __syncthreads();
    if (tid < R) atomicOr(&s_mask[s_ids[tid]], 1u << (tid / a.k));
    __syncthreads();
    const int cnt = tid < a.E ? __popc(s_mask[tid]) : 0;
    int tot, atot;
    const int off = block_scan_256(cnt, s_scan, &tot);
    const int aoff = block_scan_256(cnt > 0 ? 1 : 0, s_scan, &atot);
    if (tid < a.E) {
        s_off[tid] = off;
        if (cnt > 0) s_act[1 + aoff] = tid;
        if (writer) {
            a.counts[tid] = cnt;
            a.offsets[tid] = off;
            if (cnt > 0) a.active[1 + aoff] = tid;
        }
    }
    if (tid == 0) {
        s_off[a.E] = tot;
        s_act[0] = atot;
        if (writer) {
            a.offsets[a.E] = tot;
            a.active[0] = atot;
        }
    }
    __syncthreads();
    if (tid < R) {
        const int e = s_ids[tid], t = tid / a.k;
        const int pos = s_off[e] + __popc(s_mask[e] & ((1u << t) - 1u));
        if (s_tok) s_tok[pos] = t;
        if (writer) {
            a.sorted[pos] = tid;
            a.route_pos[tid] = pos;
        }
    }
    __syncthreads();
}

} // namespace moe
