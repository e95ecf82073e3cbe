// Internal device helpers shared by the HIP kernels of the routed MoE layer.
// Target: CDNA4 (gfx950), wave64.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- launches
// Optional timing of the kernels one stage of the layer launches.  While
// `stop` is set, every launch goes through hipExtLaunchKernel: the first one
// records `start` when it begins and each one records `stop` when it ends, so
// the pair spans exactly the stage's kernels, as a profiler's kernel trace
// does, without the dispatch gap in front of them.
struct StageTimer {
    hipEvent_t start = nullptr, stop = nullptr;
    int launches = 0;
};
StageTimer &stage_timer(); // per host thread

template <typename... P, typename... A>
inline void launch_kernel(void (*k)(P...), dim3 grid, dim3 block, uint32_t shm, hipStream_t s, A... args) {
    StageTimer &t = stage_timer();
    if (t.stop) {
        hipExtLaunchKernelGGL(k, grid, block, shm, s, t.launches == 0 ? t.start : nullptr, t.stop, 0,
                              static_cast<P>(args)...);
        t.launches++;
    } else {
        hipLaunchKernelGGL(k, grid, block, shm, s, static_cast<P>(args)...);
    }
}

enum Dtype : int { DT_F32 = 0, DT_BF16 = 1, DT_Q8 = 2, DT_MX4 = 3 };

// Weight formats that carry one scale per 32-element block along the
// reduction (Q8_0: fp16 scale and int8 values; MXFP4: E8M0 scale and FP4
// E2M1 codes, two per byte).
template <int DT> __host__ __device__ constexpr bool blocked() { return DT == DT_Q8 || DT == DT_MX4; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 to fp16 bits, round to nearest even, saturated to +-65504.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)fminf(fmaxf(v, -65504.f), 65504.f));
}

// An E8M0 scale byte as the float 2^(e - 127); 0 gives 2^-127 (a float
// subnormal), 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0x7fc00000u : e << 23));
}

// Sign-extended byte b of a 32-bit word, as float.
template <int B>
__device__ __forceinline__ float i8_to_f32(uint32_t w) {
    return (float)(int32_t)((int32_t)(w << (24 - 8 * B)) >> 24);
}

// ---------------------------------------------------------- wave reductions
// DPP controls: quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror,
// row_mirror.  Each step pairs every lane with exactly one partner in its
// 16-lane row, so after the four steps every lane of a row holds that row's
// result; the four rows' results are then read from lanes 0, 16, 32 and 48
// and combined as (r0 op r1) op (r2 op r3), so every lane ends with the same,
// order-fixed value.  (Reading the rows out with readlane replaces a
// ds_swizzle step, which goes through the LDS unit.)
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_hmirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); }

struct OpSum { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// All-reduce of a float over the 64 lanes; requires all lanes active.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = op(v, __int_as_float(dpp_xor1(__float_as_int(v))));
    v = op(v, __int_as_float(dpp_xor2(__float_as_int(v))));
    v = op(v, __int_as_float(dpp_hmirror(__float_as_int(v))));
    v = op(v, __int_as_float(dpp_mirror(__float_as_int(v))));
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpSum()); }

// Sums over the 64 lanes of K values at once (K = 2, 4 or 8; all lanes
// active): afterwards every lane of group q = lane / (64 / K) holds the sum
// of v[q].  Each exchange halves the values a lane carries: with partner
// lane ^ b (b = 32, 16, ..), lanes with bit b clear keep the first half of
// their values and add the partner's first half, the others the second half.
// The groups of 64 / K lanes then all-reduce their one value with the DPP
// steps of wave_reduce.  log2(K) exchanges and one group reduction replace K
// full reductions; the order of the additions is fixed.  (In the per-row and
// streamed kernels, against one wave_sum a value: gpt-oss-shaped Q8_0 M = 16,
// 162.3 against 168.2 us a call; DeepSeek-V2-Lite-shaped, 180.7 against
// 191.7 us; MXFP4, 159.6 against 167.0 us.  With ds_bpermute exchanges in
// place of the lane swaps it gained little and slowed the one-token down
// kernel.)
// The value of lane ^ 32 (b = 32) or lane ^ 16 (b = 16), or, within a
// 16-lane row, lane ^ 8 (b = 8), with the gfx950 lane-swap instructions and
// DPP (VALU only).  The swaps return the two operands after the exchange; with
// both operands v, a lane in the upper half (odd row) finds its partner's
// value in the first, a lane in the lower half (even row) in the second.
template <int B>
__device__ __forceinline__ float lane_xor(float v, int lane) {
    const uint32_t u = __float_as_uint(v);
    if constexpr (B == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float((lane & 32) ? r[0] : r[1]);
    } else if constexpr (B == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    } else {
        static_assert(B == 8, "lane_xor: 8, 16 or 32");
        return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false)); // row_ror:8
    }
}

template <int K>
__device__ __forceinline__ float wave_sum_split(const float (&v)[K], int lane) {
    static_assert(K == 2 || K == 4 || K == 8, "K must be 2, 4 or 8");
    float w[K];
#pragma unroll
    for (int i = 0; i < K; i++) w[i] = v[i];
    // exchanges with lane ^ 32, then ^ 16, then ^ 8 while values remain
    auto exchange = [&](auto bconst, int n) {
        constexpr int b = decltype(bconst)::value;
        const bool up = (lane & b) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; i++) {
            const float keep = up ? w[n / 2 + i] : w[i];
            const float send = up ? w[i] : w[n / 2 + i];
            w[i] = keep + lane_xor<b>(send, lane);
        }
    };
    exchange(std::integral_constant<int, 32>{}, K);
    if constexpr (K >= 4) exchange(std::integral_constant<int, 16>{}, K / 2);
    if constexpr (K >= 8) exchange(std::integral_constant<int, 8>{}, K / 4);
    float x = w[0];
    if constexpr (K == 2) x += lane_xor<16>(x, lane);
    x += __int_as_float(dpp_xor1(__float_as_int(x)));
    x += __int_as_float(dpp_xor2(__float_as_int(x)));
    x += __int_as_float(dpp_hmirror(__float_as_int(x)));
    if (K <= 4) x += __int_as_float(dpp_mirror(__float_as_int(x)));
    return x;
}

// R values (1 <= R <= 8) summed over the wave as by wave_sum_split, padded
// with zeros to a power of two KP: lane l holds the sum of v[l / sum_lanes<R>()]
// (for that index below R).  R = 1 is wave_sum.
template <int R> constexpr int sum_ways() { return R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : 8; }
template <int R> constexpr int sum_lanes() { return 64 / sum_ways<R>(); }
template <int R>
__device__ __forceinline__ float wave_sum_rows(const float (&v)[R], int lane) {
    static_assert(R >= 1 && R <= 8, "1 to 8 values");
    constexpr int KP = sum_ways<R>();
    if constexpr (KP == 1) {
        return wave_sum(v[0]);
    } else {
        float w[KP];
#pragma unroll
        for (int i = 0; i < KP; i++) w[i] = i < R ? v[i] : 0.f;
        return wave_sum_split<KP>(w, lane);
    }
}
// The value lane `src` holds, in every lane.
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMaxF()); }

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = umax32(v, (uint32_t)dpp_xor1((int)v));
    v = umax32(v, (uint32_t)dpp_xor2((int)v));
    v = umax32(v, (uint32_t)dpp_hmirror((int)v));
    v = umax32(v, (uint32_t)dpp_mirror((int)v));
    return umax32(umax32((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
                  umax32((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, dpp_xor1(v));
    v = min(v, dpp_xor2(v));
    v = min(v, dpp_hmirror(v));
    v = min(v, dpp_mirror(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// fp32 -> uint32 whose unsigned order is the float order (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float silu_mul(float g, float v) {
    return g / (1.0f + __expf(-g)) * v;
}

__device__ __forceinline__ float clampf(float v, float lim) {
    return fminf(fmaxf(v, -lim), lim);
}

// ---------------------------------------------------------- 16-byte chunk loads
// A "chunk" is the elements one lane takes per 16-byte weight load:
// 4 fp32, 8 bf16, 16 Q8_0 int8 values (half a Q8_0 block) or 32 MXFP4 codes
// (one MXFP4 block).
template <int DT> struct Chunk;
template <> struct Chunk<DT_F32> { static constexpr int N = 4; };
template <> struct Chunk<DT_BF16> { static constexpr int N = 8; };
template <> struct Chunk<DT_Q8> { static constexpr int N = 16; };
template <> struct Chunk<DT_MX4> { static constexpr int N = 32; };

// Load chunk c of a weight row into floats (Q8_0: the raw q values; the
// caller applies the block scale).
template <int DT>
__device__ __forceinline__ void load_chunk(const void *row, int c, float *w);

template <>
__device__ __forceinline__ void load_chunk<DT_F32>(const void *row, int c, float *w) {
    f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row) + c);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}
template <>
__device__ __forceinline__ void load_chunk<DT_BF16>(const void *row, int c, float *w) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + c);
    w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void load_chunk<DT_Q8>(const void *row, int c, float *w) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + c);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        w[4 * i + 0] = i8_to_f32<0>(d[i]);
        w[4 * i + 1] = i8_to_f32<1>(d[i]);
        w[4 * i + 2] = i8_to_f32<2>(d[i]);
        w[4 * i + 3] = i8_to_f32<3>(d[i]);
    }
}

// Raw 16-byte chunk load (no conversion) and its decoding, so that a group of
// loads can be issued before any of them is used.
__device__ __forceinline__ u32x4 load_raw(const void *row, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + c);
}

template <int DT>
__device__ __forceinline__ void decode_chunk(u32x4 v, float *w) {
    if constexpr (DT == DT_F32) {
        w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y);
        w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
    } else if constexpr (DT == DT_BF16) {
        w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
        w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
    } else if constexpr (DT == DT_Q8) {
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            w[4 * i + 0] = i8_to_f32<0>(d[i]);
            w[4 * i + 1] = i8_to_f32<1>(d[i]);
            w[4 * i + 2] = i8_to_f32<2>(d[i]);
            w[4 * i + 3] = i8_to_f32<3>(d[i]);
        }
    } else {
        // MXFP4 codes, element 2j in the low nibble of byte j: the hardware
        // converter takes one byte (two codes) at a time, exactly (scale 1;
        // the block scale is applied to the chunk's dot).
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 0);
            const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 1);
            const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 2);
            const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 3);
            w[8 * i + 0] = p0.x; w[8 * i + 1] = p0.y; w[8 * i + 2] = p1.x; w[8 * i + 3] = p1.y;
            w[8 * i + 4] = p2.x; w[8 * i + 5] = p2.y; w[8 * i + 6] = p3.x; w[8 * i + 7] = p3.y;
        }
    }
}

// The 32 codes of an MXFP4 chunk as 16 words of bf16 pairs (exact: every
// E2M1 value is a bf16 value).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void mx4_to_bf16x2(u32x4 v, uint32_t (&o)[16]) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        o[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 0));
        o[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 1));
        o[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 2));
        o[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 3));
    }
}

// Block scales: the stored bits of block i of a scale plane (fp16 for Q8_0,
// an E8M0 byte for MXFP4), and their value.
template <int DT>
__device__ __forceinline__ uint16_t scale_bits(const void *plane, size_t i) {
    if constexpr (DT == DT_MX4) return reinterpret_cast<const uint8_t *>(plane)[i];
    else return reinterpret_cast<const uint16_t *>(plane)[i];
}
template <int DT>
__device__ __forceinline__ float scale_value(uint16_t bits) {
    if constexpr (DT == DT_MX4) return e8m0_to_f32(bits);
    else return f16_bits_to_f32(bits);
}
// Block (index along a row) that chunk c falls in.
template <int DT> __host__ __device__ constexpr int chunk_block(int c) { return c * Chunk<DT>::N / 32; }
// A scale plane advanced by i blocks.
template <int DT>
__host__ __device__ inline const void *scale_at(const void *plane, size_t i) {
    return reinterpret_cast<const char *>(plane) + i * (DT == DT_MX4 ? 1 : 2);
}

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

template <int DT> constexpr int dt_bytes() { return DT == DT_BF16 ? 2 : 4; }

// Wave-uniform copy of a value the compiler cannot prove uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Bytes of n stored elements of a row (Q8_0: the int8 plane only; MXFP4: the
// code plane only, two codes per byte; n even).
template <int DT> __host__ __device__ constexpr size_t row_bytes(size_t n) {
    return DT == DT_F32 ? n * 4 : (DT == DT_BF16 ? n * 2 : (DT == DT_Q8 ? n : n / 2));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// Where a row's vector pieces sit when the row is stored piece-major: the row
// is cut into chunks of P 16-byte pieces (one lane's share of a load) and the
// chunks into blocks of 64; a block holds piece 0 of each of its chunks, then
// piece 1, and so on.  A wave reading piece q of 64 consecutive chunks, one
// chunk a lane, then reads contiguous memory (no LDS bank conflicts, fewest
// cache lines) instead of P * 16 bytes apart.  Returns the piece index.
__device__ __forceinline__ int piece_major(int c, int q, int nch, int P) {
    const int blk = c >> 6, bw = min(64, nch - (blk << 6));
    return blk * 64 * P + q * bw + (c & 63);
}

// Where element i of a one-token act row of `width` elements is stored.  The
// row is cut into chunks of N elements (one down-kernel lane's share) and the
// chunks into blocks of 64; a block is stored piece-major: the first four
// floats of each of its chunks, then the next four, and so on.  A wave of the
// down kernel, one chunk a lane, then reads each 16-byte piece of its chunks
// from contiguous memory instead of 64 bytes apart.
template <int N>
__device__ __forceinline__ int m1_act_index(int i, int width) {
    const int c = i / N, j = i - c * N;
    return piece_major(c, j >> 2, width / N, N / 4) * 4 + (j & 3);
}

} // namespace moe
