// MFMA grouped-GEMM path of the routed MoE layer (bf16 or fp16 operands,
// fp32 accumulate), for batches in which the touched experts see several tokens
// each: the per-expert products are then dense contractions.
//
// Uses:
//   gate/up  A = gathered token rows of x (bf16; in the fused call the normed
//            rows as fp16, with B converted to fp16 as in down), B = gate and
//            up rows of the tile's expert, epilogue silu(clamp(g)) * clamp(v)
//            -> act, written as fp32 or, inside the layer, as fp16 (the
//            precision the pages keep act in);
//   down     A = fp16 act rows, B = down rows converted to fp16 in registers,
//            fp16 MFMAs -> per-route outputs;
//   shared   the same two with identity rows (all tokens), for a shared expert.
// B is bf16, Q8_0 (int8 plus fp16 scales per 32 reduction elements) or
// MXFP4 (E2M1 codes plus E8M0 scales), converted exactly to bf16 (fp16 with
// fp16 A) in registers; each block's products are scaled once.  (The
// router's reduction-sliced kernel is at the end of this file.)
//
// Tiles: 32, 64, 96, 128 or 160 rows (tokens or routes of one expert), by
// the routes an expert is expected to hold (mfma_tile_rows below), so that
// most experts' tokens share one pass over the weights without running
// tiles that are mostly empty rows, x 128
// (gate/up: 32 columns of gate and of up per wave) or 256 (down: 64 columns
// per wave) output columns.  Four waves each own all rows of their columns
// and issue v_mfma_f32_32x32x16_bf16.
//
// Two kernels:
//   k_gemm_lds  both operands go global -> LDS with asynchronous copies
//     (global_load_lds_dwordx4) in a 3-stage pipeline, XOR-swizzled rows;
//     64 reduction elements a stage (128 for Q8_0 and MXFP4 B with 32-row
//     tiles);
//   k_gemm_reg (fp32 A handed in by a caller of the stage-wise entry points,
//     bf16 B) A is staged through registers into LDS (double buffered, split
//     into hi/lo once as it is written), B fragments are loaded straight into
//     registers, one step ahead.
// (act as fp16 against act carried as two bf16 numbers, hi and lo, for
// about 16 bits: the down GEMM's A bytes and MFMAs halve; Qwen3-shaped Zipf
// M = 2048, 467 against 529 us a call, Mixtral-shaped M = 512, 634 against
// 737 us.  A single bf16 would cost about 1.6e-3 relative L2 of the output.)
#include <algorithm>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A operand formats of the grouped GEMM: bf16 rows (x), fp16 rows (act of the
// down GEMM, and the fused layer's normed x; B is then converted to fp16 in
// registers).
enum AFormat { AF_BF16 = 0, AF_F16 = 1 };

constexpr int kMB = 4;              // 32-row blocks per wave
constexpr int kBM = 32 * kMB;       // rows per tile
constexpr int kMBWide = 5;          // the layer call's wide tiles (bf16 weights)
constexpr int kBMWide = 32 * kMBWide;
constexpr int kBK = 64;            // reduction granularity of K (both kernels need K % 64 == 0)
constexpr int kLdsRow = kBK + 8;   // bf16 elements per padded LDS row of the register-staged kernel
constexpr int kGW = 4;
constexpr int kGThreads = kGW * kWave;

// Rows of the grouped GEMM's tiles for a batch of M tokens, by the routes
// an expert can be expected to hold (the mean, plus one standard deviation of
// a random spread when the layer has several experts): 32 up to 32 routes,
// then 64 and 96 up to 64 and 96.  An expert just over 32 routes would
// otherwise run a second 32-row tile, and one of 33 to 96 routes a 128-row
// tile a quarter or more empty (gpt-oss-shaped Q8_0 M = 256, 378 against
// 398 us a call, M = 512, 466 against 582 us; MXFP4 M = 384, 375 against
// 660 us; Mixtral-shaped M = 128, 557 against 613 us, M = 256, 626 against
// 680 us; Qwen3-shaped M = 512, 291 against 321 us).  MXFP4 keeps 32 rows
// while the mean is at most 64 (gpt-oss shape, M = 256: 357 against 363 us
// with 64-row tiles, from the down GEMM; since 32-row tiles take 128-element
// stages, M = 512: 385 against 440 us) and otherwise always takes 64-row
// tiles, several an expert if need be (M = 1024: 586 against 631 us with
// 32-row tiles; before those stages, M = 512: 499 against 579 us with
// 96-row tiles; M = 768, 611 against 837 us, and M = 1024, 684 against
// 996 us with 128- and 160-row tiles; Q8_0 at M = 512 the other way round:
// 530 against 469 us, so bf16 and Q8_0 keep 96).  Beyond 96 routes bf16
// and Q8_0 take the height of least estimated cost among 96, 128 and (bf16)
// 160 rows: tiles times their MFMA-weighted size, which picks the 96-row
// tile when it needs no more tiles than 128 rows (gpt-oss-shaped Q8_0
// M = 1024: 861 against 981 us; M = 768, one 128-row tile: 661 against
// 748 us) and 160 over 128 when it saves a tile.  An expert a few routes
// over a multiple of 128 otherwise runs an extra, nearly empty tile that
// streams its weights and the whole reduction again (Mixtral-shaped,
// 128 routes an expert on average at M = 512: 811 against 922 us a call;
// M = 1024: 1396 against 1461 us; Qwen3-shaped M = 4096: 1019 against
// 1031 us; a dense layer at M = 512, exactly four 128-row tiles, keeps 128).
// Q8_0 weights keep 128 rows: 160-row tiles measured no faster (gpt-oss
// shape, M = 1024: 760 against 748 us; M = 2048: 1266 against 1177 us).
// The stage-wise entry points always use kBM.
int mfma_tile_rows(const Layer &L, int M) {
    const long R = (long)M * L.k;
    const double c = (double)R / L.E, hi = c + (L.E > 1 ? std::sqrt(c) : 0.0);
    if (L.edt == DT_MX4 ? R <= 64L * L.E : hi <= 32) return 32;
    if (hi <= 64 || L.edt == DT_MX4) return 64;
    if (hi <= 96) return 96;
    // the height of least estimated cost: tiles times (1 + 0.316 rows / 128),
    // a tile's weight stream plus MFMA work growing with its rows (0.316
    // puts a 160-row tile at 1.06 times a 128-row one)
    int best = kBM;
    double best_cost = 1e300;
    for (const int bm : {96, kBM, kBMWide}) {
        if (bm == kBMWide && L.edt != DT_BF16) continue;
        const double cost = std::ceil(hi / bm) * (1.0 + 0.316 * bm / kBM);
        if (cost < best_cost) {
            best_cost = cost;
            best = bm;
        }
    }
    return best;
}
int mfma_tile_rows() { return kBM; }

enum GemmKind { GK_GATEUP = 0, GK_PLAIN = 1 };

struct GemmArgs {
    const void *a;           // x: bf16 [rows][K]; act: fp32 [rows][K] (rows = sorted positions)
    const int32_t *sorted;   // x rows of routed tiles: token = sorted[p] / k_route; null: row = p
    int k_route;
    const int32_t *tiles;    // tile list (layout in the permutation); null: identity tiles
    const int32_t *offsets;  // expert row ranges (routed tiles)
    int E;                   // experts (tile list layout)
    int M;                   // identity tiles: number of rows
    int max_tiles;           // tile slots in the grid
    int ksplit;              // reduction split: slice ks writes out + ks * slab
    size_t slab;
    const uint16_t *b0, *b1; // bf16 [experts][N][K], or Q8_0 int8 planes; b1 only for gate/up
    size_t b_stride;         // elements between experts' matrices
    const uint16_t *s0, *s1; // Q8_0: fp16 block scales [experts][N][K/32] of b0, b1
    size_t s_stride;         // Q8_0: scales between experts' matrices
    int N, K;
    const float *tok_scale;  // per-token scale of the products (pre-norm), or null
    float limit;             // gate/up clamp (0 = off)
    float *out;              // fp32 [rows][ldo]; gate/up with out_fmt ACT_F16: fp16 rows
    int ldo;
    int out_fmt;             // gate/up act rows: ACT_F32 or ACT_F16
    int tile_rows;           // rows per tile of the LDS kernel (32, 64, 96, 128 or 160; the tile list's)
    int n_ntiles;            // column tiles
    int units;               // LDS kernel: workgroups per token tile (n_ntiles * ksplit)
};

template <int KIND>
struct GemmShape {
    static constexpr int NB = 2;                                  // 32-column B blocks per wave
    static constexpr int WCOLS = KIND == GK_GATEUP ? 32 : 64;     // output columns per wave
    static constexpr int COLS = kGW * WCOLS;                      // output columns per tile
};

// Reduction elements per pipeline stage (bf16 or fp16 A; half that for split
// A with bf16 B) and number of LDS stages of the asynchronous-copy kernel.  A
// stage holds 128 bytes of each A row (20 KB for 160 rows) and of each of the
// 256 B columns (32 KB of bf16 B; less for Q8_0 and MXFP4).
constexpr int kStageK = 64;
constexpr int kStages = 3;

typedef __attribute__((address_space(3))) void *lds_ptr;

// 16-byte LDS read issued as inline assembly: the compiler cannot see that it
// reads LDS, so it does not wait for every outstanding global->LDS copy
// before it (it cannot tell which stage a copy writes).  The caller waits for
// the results with lds_wait.
__device__ __forceinline__ u32x4 lds_load16(const unsigned char *p) {
    u32x4 r;
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char *)p;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}

// Wait for this lane's LDS reads; the values pass through the statements so
// that nothing using them is scheduled before the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&v)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)");
#pragma unroll
    for (int i = 0; i < N; i++) asm volatile("" : "+v"(v[i]));
}

// Asynchronous 16-byte copy global -> LDS for each lane: lane i writes LDS
// bytes l + 16*i (l wave-uniform).  Completion is tracked by vmcnt.
__device__ __forceinline__ void copy16_lds(const void *g, unsigned char *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)l, 16, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding) that waits for at most n outstanding
// vector memory operations and for nothing else.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }


// XOR swizzle of a 16-byte chunk within an LDS row of CH chunks: rows of 8
// or more chunks (128 B) xor with (row ^ row / 8) % 8, so that 8 consecutive
// rows land on 8 different 16-byte bank groups of 128 bytes, and 16
// consecutive rows on 16 different groups of 256 bytes (consecutive even
// rows, and odd rows, take distinct values; measured against row % 8:
// Mixtral-shaped M = 512 down GEMM 379 against 391 us, Qwen3-shaped M = 2048
// layer 600 against 608 us).  Rows of 4 chunks (64 B, two rows per 128
// bytes of banks) xor with (row / 2) % 4.  Rows of 2 chunks (MXFP4 columns,
// read 4 bytes at a time) xor with (row / 8) % 2, which halves the conflicts
// of rows 8 apart.
template <int CH>
__device__ __forceinline__ int swz(int row) {
    return CH >= 8 ? ((row ^ (row >> 3)) & 7) : (CH == 4 ? ((row >> 1) & 3) : ((row >> 3) & 1));
}

// 8- and 4-byte LDS reads, issued like lds_load16 (the caller waits).
__device__ __forceinline__ u32x2 lds_load8(const unsigned char *p) {
    u32x2 r;
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char *)p;
    asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
__device__ __forceinline__ uint32_t lds_load4(const unsigned char *p) {
    uint32_t r;
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char *)p;
    asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
template <typename T>
__device__ __forceinline__ void lds_keep(T &v) { asm volatile("" : "+v"(v)); }

// 4-byte asynchronous copy global -> LDS: lane i writes LDS bytes l + 4*i.
__device__ __forceinline__ void copy4_lds(const void *g, unsigned char *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)l, 4, 0, 0);
}

// 8 Q8_0 int8 values (two words) as 8 bf16 (exact: |q| <= 127).
__device__ __forceinline__ u32x4 q8x8_to_bf16(u32x2 w) {
    u32x4 o;
    const uint32_t f0 = __float_as_uint(i8_to_f32<0>(w.x)), f1 = __float_as_uint(i8_to_f32<1>(w.x));
    const uint32_t f2 = __float_as_uint(i8_to_f32<2>(w.x)), f3 = __float_as_uint(i8_to_f32<3>(w.x));
    const uint32_t f4 = __float_as_uint(i8_to_f32<0>(w.y)), f5 = __float_as_uint(i8_to_f32<1>(w.y));
    const uint32_t f6 = __float_as_uint(i8_to_f32<2>(w.y)), f7 = __float_as_uint(i8_to_f32<3>(w.y));
    o.x = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
    o.y = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    o.z = __builtin_amdgcn_perm(f5, f4, 0x07060302u);
    o.w = __builtin_amdgcn_perm(f7, f6, 0x07060302u);
    return o;
}

// 8 Q8_0 int8 values as 8 fp16 (exact: |q| <= 127).
__device__ __forceinline__ u32x4 q8x8_to_f16(u32x2 w) {
    u32x4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(i8_to_f32<0>(w.x), i8_to_f32<1>(w.x)));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(i8_to_f32<2>(w.x), i8_to_f32<3>(w.x)));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(i8_to_f32<0>(w.y), i8_to_f32<1>(w.y)));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(i8_to_f32<2>(w.y), i8_to_f32<3>(w.y)));
    return o;
}

// 8 bf16 values as 8 fp16: exact wherever the value is a normal fp16
// (6.1e-5 <= |v| <= 65504); smaller magnitudes lose low bits to the fp16
// subnormal range (an absolute error below 2^-24), larger ones saturate.
// (The conversion rounds toward zero, so finite values beyond the fp16
// range come out as +-65504.)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)));
}
__device__ __forceinline__ u32x4 bf16x8_to_f16(u32x4 v) {
    return u32x4{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
}

// One 32x32x16 MFMA on bf16 (H false) or fp16 (H true) operands.
template <bool H>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (H)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// silu(g) * v with the hardware reciprocal (v_rcp_f32, 1 ulp) in place of
// the IEEE division: the grouped GEMM's epilogue runs on one wave a SIMD,
// where the division's ten dependent instructions per element show.
__device__ __forceinline__ float silu_mul_rcp(float g, float v) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * v;
}

// BF (B format): 0 = bf16; 1 = Q8_0 (int8 plane plus fp16 scales per 32
// reduction elements); 2 = MXFP4 (E2M1 codes, two a byte, plus an E8M0 scale
// per 32 reduction elements).  Block-scaled stages span 64 reduction elements
// (two scale blocks; int8 columns take half the LDS of bf16 ones, MXFP4
// columns a quarter).  Q8_0: a 4-byte copy per lane brings each column's two
// scales along.  MXFP4: each lane loads its columns' two scale bytes into
// registers with the stage's copies (their rows are only 2-byte aligned).
// Each block's products are accumulated by the MFMAs separately and added to
// the accumulator times the column's scale.  (Stages of 128 elements with
// 32-row tiles measured no faster for Q8_0.)
template <int KIND, int AF, int MB, int BF>
__global__ __launch_bounds__(kGThreads, 1) void k_gemm_lds(GemmArgs a) {
    constexpr bool AH = AF == AF_F16;              // fp16 A (and B converted to fp16)
    constexpr bool BQ = BF == 1;                   // Q8_0 B
    constexpr bool BX = BF == 2;                   // MXFP4 B
    constexpr bool BS = BQ || BX;                  // block-scaled B
    constexpr int BM = 32 * MB;                    // rows per tile
    constexpr int NB = GemmShape<KIND>::NB;
    constexpr int WCOLS = GemmShape<KIND>::WCOLS;
    constexpr int EB = BQ ? 1 : 2;                 // bytes per B element (bf16, Q8_0)
    // reduction elements per stage: 128 for block-scaled B with 32-row tiles
    // (a Q8_0 column then takes a whole 128-byte line a stage, an MXFP4 one
    // half a line, and a stage moves enough bytes to cover the copies'
    // latency: Q8_0 at H = I = 2944, M = 64, 241 against 266 us a call;
    // MXFP4, 205 against 298 us; at the gpt-oss shape, H = I = 2880 and so a
    // half last stage, Q8_0 M = 64 272 against 283 us, MXFP4 M = 64 236
    // against 292 us and M = 256 301 against 330 us; with 64-row tiles it
    // measured slower), else 64.  K need only be
    // a multiple of 64: a last stage of 64 elements reads its missing half
    // from the 64 elements before it and skips those blocks.
    constexpr int BK = (BS && MB == 1) ? 2 * kStageK : kStageK;
    constexpr bool RAGGED = BK > 64;               // K may end half way into a stage
    constexpr int NBLK = BK / 32;                  // scale blocks per stage
    constexpr int SCP = BQ ? NBLK / 2 : 0;         // 4-byte scale copies per lane per stage
    constexpr int SRG = BX ? NB * (NBLK / 2) : 0;  // MXFP4 2-byte scale loads per lane per stage
    constexpr int NST = kStages;                   // LDS stages
    constexpr int ARB = BK * 2;                    // A bytes per row per stage
    constexpr int BRB = BX ? BK / 2 : BK * EB;     // B bytes per column per stage
    constexpr int ACH = ARB / 16;                  // 16-byte chunks per A row per stage
    constexpr int BCH = BRB / 16;                  // 16-byte chunks per B column per stage
    constexpr int WBC = 64;                        // B columns per wave (gate/up: 32 gate + 32 up)
    constexpr int A_BYTES = BM * ARB;
    constexpr int WB_BYTES = WBC * BRB;            // one wave's B per stage
    constexpr int WS_BYTES = BQ ? WBC * 2 * NBLK : 0; // one wave's scales per stage
    constexpr int ST_BYTES = A_BYTES + kGW * WB_BYTES + kGW * WS_BYTES;
    constexpr int A_DMA = BM * ARB / (kWave * 16) / kGW; // A copies per wave per stage (each 1 KB)
    constexpr int B_DMA = WB_BYTES / (kWave * 16);        // B copies per wave per stage
    constexpr int LPS = A_DMA + B_DMA + SCP + SRG; // vector memory operations per lane per stage
    static_assert(!BQ || NBLK % 2 == 0, "Q8_0 scales are copied in pairs of blocks");
    static_assert(!BX || NBLK == 2 || NBLK == 4, "MXFP4 stages hold 2 or 4 scale blocks (one 32-bit word)");
    // one LDS array per stage, named explicitly in an NST-way unrolled loop
    // (measured faster than one array indexed by kt % NST)
    __shared__ __attribute__((aligned(16))) unsigned char sm0[ST_BYTES], sm1[ST_BYTES], sm2[ST_BYTES];
    __shared__ const char *s_src[BM];
    __shared__ float s_scl[BM]; // the rows' token scales (pre-norm), or 1
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uniform(tid >> 6);

    // ---- which tile, column block and reduction slice.  The workgroups of
    // one expert cover its column units c = (slice, column block) for every
    // token tile tl, per_tile units a tile: per_tile * Te (unit, tile) pairs,
    // taken in unit-major order.  Workgroups are dispatched to the 8 XCDs in
    // turn, so the expert's local workgroup l runs on XCD offset l & 7; XCD
    // offset s takes the s-th contiguous run of about a eighth of the pairs
    // (its (l >> 3)-th pair).  A unit's token tiles so run on one XCD, or two
    // where a run ends inside the unit: its weights come from HBM about once
    // an XCD and the L2 serves the other tiles, and the XCD's units share one
    // reduction slice of the A rows.  (Qwen3-shaped Zipf M = 2048, 6 gate/up
    // units a tile: 1.05 against 1.26 GB fetched with the flat tile-major
    // order, at the same time; 8 units take the same order as before.)
    const int g = blockIdx.x;
    const int per_tile = a.units;
    int e = 0, ts, Te, p0, nrows;
    if (a.tiles) {
        const int q = g / per_tile;
        if (q >= a.tiles[0]) return;
        const int32_t *pairs = a.tiles + 2 + a.E;
        e = pairs[2 * q];
        ts = a.tiles[1 + e];
        Te = a.tiles[2 + e] - ts;
    } else {
        ts = 0;
        Te = (a.M + BM - 1) / BM;
        if (g >= Te * per_tile) return;
    }
    const int local = g - ts * per_tile;
    int tl, cu;
    {
        const int total = per_tile * Te, s8 = local & 7;
        int before = 0; // pairs on the XCD offsets before s8
        for (int j = 0; j < s8; j++) before += (total - j + 7) >> 3;
        const int pr = before + (local >> 3);
        cu = pr / Te;
        tl = pr - cu * Te;
    }
    const int ks = cu / a.n_ntiles, nt = cu - ks * a.n_ntiles;
    if (a.tiles) {
        p0 = a.tiles[2 + a.E + 2 * (ts + tl) + 1];
        nrows = min(BM, a.offsets[e + 1] - p0);
    } else {
        p0 = tl * BM;
        nrows = min(BM, a.M - p0);
    }
    if (tid < BM) {
        const int p = p0 + min(tid, nrows - 1);
        const int t = a.sorted ? a.sorted[p] / a.k_route : p;
        s_src[tid] = reinterpret_cast<const char *>(a.a) + (size_t)t * a.K * 2;
        s_scl[tid] = a.tok_scale ? a.tok_scale[t] : 1.0f;
    }
    __syncthreads();

    const int K = a.K, N = a.N, NKS = (K + BK - 1) / BK;
    const int kb = ks * NKS / a.ksplit, nk = (ks + 1) * NKS / a.ksplit - kb; // this slice's stages
    const int colw = nt * GemmShape<KIND>::COLS + wave * WCOLS;
    const bool wave_on = colw < N;

    // ---- copy sources.  A copy of 1 KB fills 64 / ACH A rows or 64 / BCH B
    // columns of one stage; lane i writes LDS bytes i*16..i*16+15, which hold
    // logical 16-byte chunk (slot ^ row) of its row: an XOR swizzle that keeps
    // the MFMA operand reads below free of most bank conflicts.
    // (RAGGED: whether the copy's chunk lies in the second half of a stage)
    const char *asrc[A_DMA];
    bool ahi[A_DMA];
#pragma unroll
    for (int q = 0; q < A_DMA; q++) {
        const int r = (wave * A_DMA + q) * (kWave / ACH) + lane / ACH, c = (lane % ACH) ^ swz<ACH>(r);
        asrc[q] = s_src[r] + c * 16;
        ahi[q] = 2 * c >= ACH;
    }
    const char *bsrc[B_DMA];
    bool bhi[B_DMA];
#pragma unroll
    for (int q = 0; q < B_DMA; q++) {
        const int cl = q * (kWave / BCH) + lane / BCH, c = (lane % BCH) ^ swz<BCH>(cl);
        bhi[q] = 2 * c >= BCH;
        const uint16_t *mat = (KIND == GK_GATEUP && cl >= 32) ? a.b1 : a.b0;
        const int col = KIND == GK_GATEUP ? colw + (cl & 31) : colw + cl;
        const size_t el = (size_t)e * a.b_stride + (size_t)min(col, N - 1) * K; // first element of the column
        bsrc[q] = reinterpret_cast<const char *>(mat) + (BX ? el / 2 : el * EB) + c * 16;
    }
    // Q8_0: lane i copies the two scales of column i of the wave's 64
    const char *ssrc = nullptr;
    if constexpr (BQ) {
        const uint16_t *sm = (KIND == GK_GATEUP && lane >= 32) ? a.s1 : a.s0;
        const int col = KIND == GK_GATEUP ? colw + (lane & 31) : colw + lane;
        ssrc = reinterpret_cast<const char *>(sm + a.s_stride * e + (size_t)min(col, N - 1) * (K / 32));
    }
    // MXFP4: the scale bytes of the lane's column in each 32-column block nb
    const uint8_t *xsrc[NB > 0 ? NB : 1];
    if constexpr (BX) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const uint8_t *sm = reinterpret_cast<const uint8_t *>((KIND == GK_GATEUP && nb == 1) ? a.s1 : a.s0);
            const int col = KIND == GK_GATEUP ? colw + (lane & 31) : colw + nb * 32 + (lane & 31);
            xsrc[nb] = sm + a.s_stride * e + (size_t)min(col, N - 1) * (K / 32);
        }
    }
    // part `part` of nparts of stage kt's copies (copy c of the wave's A, B
    // and Q8_0 scale copies goes with part c % nparts; MXFP4 scale loads with
    // the last part), so that a compute step can spread the next stage's
    // copies over its MFMA substeps
    auto issue_part = [&](int kt, unsigned char *st, uint32_t (&xs)[NB], int part, int nparts) {
        const int k0 = (kb + kt) * BK; // first reduction element of stage kt
        const size_t ka = (size_t)k0 * 2, kbb = BX ? (size_t)k0 / 2 : (size_t)k0 * EB;
        // a last stage of BK / 2 elements: second-half chunks read the first
        // half's sources again (the blocks are skipped by the compute)
        const bool tail = RAGGED && k0 + BK > K;
        constexpr size_t HA = BK / 2 * 2, HB = BX ? BK / 4 : BK / 2 * EB; // bytes of half a stage
#pragma unroll
        for (int q = 0; q < A_DMA; q++)
            if (q % nparts == part) copy16_lds(asrc[q] + ka - (tail && ahi[q] ? HA : 0), st + (wave * A_DMA + q) * 1024);
#pragma unroll
        for (int q = 0; q < B_DMA; q++)
            if ((A_DMA + q) % nparts == part)
                copy16_lds(bsrc[q] + kbb - (tail && bhi[q] ? HB : 0), st + A_BYTES + wave * WB_BYTES + q * 1024);
        if constexpr (BQ)
#pragma unroll
            for (int j = 0; j < SCP; j++)
                if ((A_DMA + B_DMA + j) % nparts == part)
                    copy4_lds(ssrc + (size_t)(k0 / 32) * 2 + 4 * (tail && 2 * j >= SCP ? j - SCP / 2 : j),
                              st + A_BYTES + kGW * WB_BYTES + wave * WS_BYTES + j * (kWave * 4));
        if constexpr (BX)
            if (part == nparts - 1)
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    uint32_t w = *reinterpret_cast<const uint16_t *>(xsrc[nb] + k0 / 32);
                    if constexpr (NBLK == 4)
                        w |= (uint32_t)*reinterpret_cast<const uint16_t *>(xsrc[nb] + k0 / 32 + (tail ? 0 : 2)) << 16;
                    xs[nb] = w;
                }
    };
    auto issue = [&](int kt, unsigned char *st, uint32_t (&xs)[NB]) { issue_part(kt, st, xs, 0, 1); };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[mb][nb][r] = 0.f;

    // kn >= 0: the copies of stage kn into `nxt` (and MXFP4 scale registers
    // xn) go out a part per substep, between that substep's LDS reads and
    // its MFMAs
    // nvb: the stage's scale blocks that lie inside K (block-scaled B)
    auto compute = [&](const unsigned char *st, uint32_t (&xs)[NB], int kn, unsigned char *nxt,
                       uint32_t (&xn)[NB], int nvb) {
        const unsigned char *bw = st + A_BYTES + wave * WB_BYTES;
        if constexpr (BX) {
            // column bytes of substep s: chunk s/2, bytes 8 (s%2) + 4 (l/32) .. +3
            // (the codes of elements 16s + 8 (l/32) .. +7); A as below
#pragma unroll
            for (int bl = 0; bl < NBLK; bl++) {
                if (RAGGED && bl >= nvb) break;
                f32x16 blk[MB][NB];
#pragma unroll
                for (int s = 2 * bl; s < 2 * bl + 2; s++) {
                    const int g8 = 2 * s + (lane >> 5);
                    uint32_t q[NB];
                    u32x4 v[MB];
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const int cl = nb * 32 + (lane & 31);
                        q[nb] = lds_load4(bw + cl * BRB + (((s >> 1) ^ swz<BCH>(cl)) * 16) + 8 * (s & 1) +
                                          4 * (lane >> 5));
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; mb++) {
                        const int r = mb * 32 + (lane & 31);
                        v[mb] = lds_load16(st + r * ARB + ((g8 ^ swz<ACH>(r)) * 16));
                    }
                    if (kn >= 0) issue_part(kn, nxt, xn, s, BK / 16);
                    asm volatile("s_waitcnt lgkmcnt(0)");
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) lds_keep(q[nb]);
#pragma unroll
                    for (int i = 0; i < MB; i++) lds_keep(v[i]);
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        u32x4 bv;
                        if constexpr (AH) {
                            bv.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[nb], 1.0f, 0));
                            bv.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[nb], 1.0f, 1));
                            bv.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[nb], 1.0f, 2));
                            bv.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[nb], 1.0f, 3));
                        } else {
                            bv.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[nb], 1.0f, 0));
                            bv.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[nb], 1.0f, 1));
                            bv.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[nb], 1.0f, 2));
                            bv.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[nb], 1.0f, 3));
                        }
#pragma unroll
                        for (int mb = 0; mb < MB; mb++)
                            blk[mb][nb] = mfma32<AH>(v[mb], bv, s == 2 * bl ? f32x16{} : blk[mb][nb]);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const float sc = e8m0_to_f32((xs[nb] >> (8 * bl)) & 255u);
#pragma unroll
                    for (int mb = 0; mb < MB; mb++)
#pragma unroll
                        for (int r = 0; r < 16; r++) acc[mb][nb][r] = fmaf(sc, blk[mb][nb][r], acc[mb][nb][r]);
                }
            }
        } else if constexpr (!BQ) {
#pragma unroll
            for (int s = 0; s < BK / 16; s++) {
                // every read of the substep first, one wait, then the MFMAs.
                // Lane l takes the 8 reduction elements g = 2s + l/32 of its
                // row or column.
                const int g8 = 2 * s + (lane >> 5);
                u32x4 v[NB + MB];
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const int cl = nb * 32 + (lane & 31);
                    v[nb] = lds_load16(bw + cl * BRB + ((g8 ^ swz<BCH>(cl)) * 16));
                }
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    const int r = mb * 32 + (lane & 31);
                    v[NB + mb] = lds_load16(st + r * ARB + ((g8 ^ swz<ACH>(r)) * 16));
                }
                if (kn >= 0) issue_part(kn, nxt, xn, s, BK / 16);
                lds_wait(v);
                if constexpr (AH)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) v[nb] = bf16x8_to_f16(v[nb]);
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) acc[mb][nb] = mfma32<AH>(v[NB + mb], v[nb], acc[mb][nb]);
            }
        } else {
            // this lane's columns' scales of the stage: fp16 pairs (blocks 2j, 2j+1)
            uint32_t sw[NB][SCP];
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
#pragma unroll
                for (int j = 0; j < SCP; j++)
                    sw[nb][j] = lds_load4(st + A_BYTES + kGW * WB_BYTES + wave * WS_BYTES + j * (kWave * 4) +
                                          (nb * 32 + (lane & 31)) * 4);
#pragma unroll
            for (int bl = 0; bl < NBLK; bl++) {
                if (RAGGED && bl >= nvb) break;
                f32x16 blk[MB][NB];
#pragma unroll
                for (int s = 2 * bl; s < 2 * bl + 2; s++) {
                    // column bytes 16s + 8 (l/32) .. +7 of chunk s; A as above
                    const int g8 = 2 * s + (lane >> 5);
                    u32x2 q[NB];
                    u32x4 v[MB];
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const int cl = nb * 32 + (lane & 31);
                        q[nb] = lds_load8(bw + cl * BRB + ((s ^ swz<BCH>(cl)) * 16) + 8 * (lane >> 5));
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; mb++) {
                        const int r = mb * 32 + (lane & 31);
                        v[mb] = lds_load16(st + r * ARB + ((g8 ^ swz<ACH>(r)) * 16));
                    }
                    if (kn >= 0) issue_part(kn, nxt, xn, s, BK / 16);
                    asm volatile("s_waitcnt lgkmcnt(0)");
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) lds_keep(q[nb]);
#pragma unroll
                    for (int i = 0; i < MB; i++) lds_keep(v[i]);
                    if (s == 2 * bl) {
#pragma unroll
                        for (int nb = 0; nb < NB; nb++)
#pragma unroll
                            for (int j = 0; j < SCP; j++) lds_keep(sw[nb][j]);
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const u32x4 bv = AH ? q8x8_to_f16(q[nb]) : q8x8_to_bf16(q[nb]);
#pragma unroll
                        for (int mb = 0; mb < MB; mb++)
                            blk[mb][nb] = mfma32<AH>(v[mb], bv, s == 2 * bl ? f32x16{} : blk[mb][nb]);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const uint32_t pair = sw[nb][bl >> 1];
                    const float sc = f16_bits_to_f32((uint16_t)((bl & 1) ? pair >> 16 : pair));
#pragma unroll
                    for (int mb = 0; mb < MB; mb++)
#pragma unroll
                        for (int r = 0; r < 16; r++) acc[mb][nb][r] = fmaf(sc, blk[mb][nb][r], acc[mb][nb][r]);
                }
            }
        }
    };

    // ---- NST-stage pipeline: stage kt is computed while stages kt+1 ..
    // kt+NST-1 are in flight.  The copies write LDS asynchronously: each lane
    // waits (vmcnt) until its copies of stage kt have landed, then the
    // workgroup barrier makes every lane's copies visible.
    // stage kt lives in buffer kt % NST
    // (MXFP4: the scale registers of stage kt are xr[kt % NST], loaded by its
    // issue and covered by the same vmcnt wait as its copies)
    uint32_t xr0[NB], xr1[NB], xr2[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) xr0[nb] = xr1[nb] = xr2[nb] = 0u;
    auto step = [&](int kt, const unsigned char *cur, unsigned char *nxt, uint32_t (&xc)[NB],
                    uint32_t (&xn)[NB]) {
        const int ahead = min(nk, kt + NST - 1) - (kt + 1); // stages issued after kt
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        // bf16 B: the next stage's copies interleave with this stage's MFMAs
        // (issued as one burst before them, they held the MFMAs back:
        // Mixtral-shaped M = 512, 734 against 769 us a call; Qwen3-shaped
        // M = 2048, 527 against 552 us).  Q8_0 and MXFP4 B keep the burst
        // (interleaved: gpt-oss-shaped Q8_0 M = 64, 296 against 286 us;
        // MXFP4 M = 512, 493 against 478 us).
        const int kn = kt + NST - 1 < nk ? kt + NST - 1 : -1;
        if constexpr (!BQ && !BX) {
            if (wave_on) compute(cur, xc, kn, nxt, xn, NBLK);
            else if (kn >= 0) issue(kn, nxt, xn);
        } else {
            if (kn >= 0) issue(kn, nxt, xn);
            if (wave_on) compute(cur, xc, -1, nxt, xn, min(NBLK, (K - (kb + kt) * BK) / 32));
        }
    };
    if (nk > 0) issue(0, sm0, xr0);
    if (nk > 1) issue(1, sm1, xr1);
    static_assert(NST == 3, "the unrolled loop below names three stage buffers");
    for (int k0 = 0; k0 < nk; k0 += 3) {
        step(k0, sm0, sm2, xr0, xr2);
        if (k0 + 1 < nk) step(k0 + 1, sm1, sm0, xr1, xr0);
        if (k0 + 2 < nk) step(k0 + 2, sm2, sm1, xr2, xr1);
    }
    if (!wave_on) return;

    // ---- epilogue: straight-line code (rows past the tile's end and
    // columns past N only skip their stores, so that the scheduler can
    // interleave the rows), token scales from LDS, and non-temporal stores
    // (the outputs are not read again by this kernel; L2 keeps the A rows).
    // (Measured against a per-row early exit, per-row token-scale loads and
    // cached stores: Mixtral-shaped M = 512 gate/up and down, Qwen3-shaped
    // M = 2048 down, 33-40 us each from the stores alone.)
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); // < BM
            const bool in = m < nrows;
            const float sc = s_scl[m];
            if constexpr (KIND == GK_GATEUP) {
                const int i = colw + (lane & 31);
                float gv = acc[mb][0][r] * sc, uv = acc[mb][1][r] * sc;
                if (a.limit > 0.f) {
                    gv = clampf(gv, a.limit);
                    uv = clampf(uv, a.limit);
                }
                const float h = silu_mul_rcp(gv, uv);
                if (in && i < N) {
                    if (a.out_fmt == ACT_F16) {
                        uint16_t *hrow = reinterpret_cast<uint16_t *>(a.out) + (size_t)(p0 + m) * a.ldo;
                        __builtin_nontemporal_store(f32_to_f16_sat(h), hrow + i);
                    } else {
                        __builtin_nontemporal_store(h, a.out + ks * a.slab + (size_t)(p0 + m) * a.ldo + i);
                    }
                }
            } else {
                float *orow = a.out + ks * a.slab + (size_t)(p0 + m) * a.ldo;
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const int n = colw + nb * 32 + (lane & 31);
                    const float v = acc[mb][nb][r] * sc;
                    if (in && n < N) __builtin_nontemporal_store(v, orow + n);
                }
            }
        }
    }
}

template <int KIND, bool A_F32>
__global__ __launch_bounds__(kGThreads, 2) void k_gemm_reg(GemmArgs a) {
    constexpr int NS = A_F32 ? 2 : 1;      // bf16 planes of A (hi, lo)
    constexpr int NB = GemmShape<KIND>::NB;
    constexpr int WCOLS = GemmShape<KIND>::WCOLS;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][NS][kBM * kLdsRow];
    __shared__ const char *s_src[kBM];
    __shared__ int s_tok[kBM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uniform(tid >> 6);

    // ---- which tile, column block and reduction slice.  g runs over an
    // expert's (slice, column block, token tile) with the token tile fastest.
    // Consecutive workgroups land on different XCDs, so the column blocks of
    // one expert spread over all eight L2s and HBM channels at once; the
    // token tiles of a column block follow one another in launch order.
    // (Renumbering so that each XCD takes a contiguous run, or putting the
    // tile index fastest across experts, measured 10-30% slower.)
    const int g = blockIdx.x;
    const int per_tile = a.n_ntiles * a.ksplit; // workgroups per token tile
    int e = 0, ts, Te, p0, nrows;
    if (a.tiles) {
        const int q = g / per_tile;
        if (q >= a.tiles[0]) return;
        const int32_t *pairs = a.tiles + 2 + a.E;
        e = pairs[2 * q];
        ts = a.tiles[1 + e];
        Te = a.tiles[2 + e] - ts;
    } else {
        ts = 0;
        Te = (a.M + kBM - 1) / kBM;
        if (g >= Te * per_tile) return;
    }
    const int local = g - ts * per_tile;
    const int ks = local / (Te * a.n_ntiles);
    const int rem = local - ks * Te * a.n_ntiles;
    const int nt = rem / Te, tl = rem - nt * Te;
    if (a.tiles) {
        p0 = a.tiles[2 + a.E + 2 * (ts + tl) + 1];
        nrows = min(kBM, a.offsets[e + 1] - p0);
    } else {
        p0 = tl * kBM;
        nrows = min(kBM, a.M - p0);
    }
    if (tid < kBM) {
        const int p = p0 + min(tid, nrows - 1);
        const int t = a.sorted ? a.sorted[p] / a.k_route : p;
        s_src[tid] = A_F32 ? reinterpret_cast<const char *>(a.a) + (size_t)p * a.K * 4
                           : reinterpret_cast<const char *>(a.a) + (size_t)t * a.K * 2;
        s_tok[tid] = t;
    }

    const int K = a.K, N = a.N, NK = K / kBK;
    const int kb = ks * NK / a.ksplit, nk = (ks + 1) * NK / a.ksplit - kb; // this slice's K steps
    const int colw = nt * GemmShape<KIND>::COLS + wave * WCOLS;
    const bool wave_on = colw < N;
    // B row of this lane for each column block (gate/up: block 0 gate, 1 up)
    const uint16_t *brow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const uint16_t *mat = (KIND == GK_GATEUP && nb == 1) ? a.b1 : a.b0;
        const int col = KIND == GK_GATEUP ? colw + (lane & 31) : colw + nb * 32 + (lane & 31);
        brow[nb] = mat + (size_t)e * a.b_stride + (size_t)min(col, N - 1) * K + 8 * (lane >> 5);
    }
    __syncthreads();

    // ---- A staging: global -> registers -> LDS
    constexpr int CPR = A_F32 ? 16 : 8;               // 16-byte chunks per row per K step
    constexpr int A_CHUNKS = kBM * CPR / kGThreads;   // per thread
    auto load_a = [&](int k0, u32x4 (&r)[A_CHUNKS]) {
#pragma unroll
        for (int j = 0; j < A_CHUNKS; j++) {
            const int c = tid + kGThreads * j;
            const int row = c / CPR, col = c % CPR;
            r[j] = *reinterpret_cast<const u32x4 *>(s_src[row] + (size_t)k0 * (A_F32 ? 4 : 2) + col * 16);
        }
    };
    auto store_a = [&](int buf, const u32x4 (&r)[A_CHUNKS]) {
#pragma unroll
        for (int j = 0; j < A_CHUNKS; j++) {
            const int c = tid + kGThreads * j;
            const int row = c / CPR, col = c % CPR;
            if constexpr (A_F32) {
                const float f[4] = {__uint_as_float(r[j].x), __uint_as_float(r[j].y),
                                    __uint_as_float(r[j].z), __uint_as_float(r[j].w)};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    hi[q] = f32_to_bf16_rne(f[q]);
                    lo[q] = f32_to_bf16_rne(f[q] - __uint_as_float(hi[q] << 16));
                }
                const u32x2 vh = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
                const u32x2 vl = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
                *reinterpret_cast<u32x2 *>(&sA[buf][0][row * kLdsRow + col * 4]) = vh;
                if constexpr (NS == 2) *reinterpret_cast<u32x2 *>(&sA[buf][NS - 1][row * kLdsRow + col * 4]) = vl;
            } else {
                *reinterpret_cast<u32x4 *>(&sA[buf][0][row * kLdsRow + col * 8]) = r[j];
            }
        }
    };
    // ---- B fragments for one K step: [substep][column block]
    auto load_b = [&](int k0, u32x4 (&bq)[4][NB]) {
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
                bq[s][nb] = *reinterpret_cast<const u32x4 *>(brow[nb] + k0 + 16 * s);
    };

    f32x16 acc[kMB][NB];
#pragma unroll
    for (int mb = 0; mb < kMB; mb++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[mb][nb][r] = 0.f;

    auto compute = [&](int buf, const u32x4 (&bq)[4][NB]) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
#pragma unroll
            for (int mb = 0; mb < kMB; mb++) {
                const int off = (mb * 32 + (lane & 31)) * kLdsRow + 16 * s + 8 * (lane >> 5);
#pragma unroll
                for (int h = 0; h < NS; h++) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8 *>(&sA[buf][h][off]);
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const bf16x8 bf = __builtin_bit_cast(bf16x8, bq[s][nb]);
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[mb][nb], 0, 0, 0);
                    }
                }
            }
        }
    };

    u32x4 bq0[4][NB], bq1[4][NB];
    {
        u32x4 ar[A_CHUNKS];
        load_a(kb * kBK, ar);
        if (wave_on) load_b(kb * kBK, bq0);
        store_a(0, ar);
    }
    __syncthreads();
    auto step = [&](int kt, const u32x4 (&cur)[4][NB], u32x4 (&nxt)[4][NB]) {
        const bool more = kt + 1 < nk;
        u32x4 ar[A_CHUNKS];
        if (more) {
            load_a((kb + kt + 1) * kBK, ar);
            if (wave_on) load_b((kb + kt + 1) * kBK, nxt);
        }
        if (wave_on) compute(kt & 1, cur);
        if (more) store_a((kt + 1) & 1, ar);
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, bq0, bq1);
        if (kt + 1 < nk) step(kt + 1, bq1, bq0);
    }
    if (!wave_on) return;

    // ---- epilogue
#pragma unroll
    for (int mb = 0; mb < kMB; mb++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m >= nrows) continue;
            const float sc = a.tok_scale ? a.tok_scale[s_tok[m]] : 1.0f;
            float *orow = a.out + ks * a.slab + (size_t)(p0 + m) * a.ldo;
            if constexpr (KIND == GK_GATEUP) {
                const int i = colw + (lane & 31);
                if (i < N) {
                    float gv = acc[mb][0][r] * sc, uv = acc[mb][1][r] * sc;
                    if (a.limit > 0.f) {
                        gv = clampf(gv, a.limit);
                        uv = clampf(uv, a.limit);
                    }
                    orow[i] = silu_mul(gv, uv);
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; nb++) {
                    const int n = colw + nb * 32 + (lane & 31);
                    if (n < N) orow[n] = acc[mb][nb][r] * sc;
                }
            }
        }
    }
}

// a_mode: 0 = bf16 A rows (gate/up), 2 = fp32 A rows (down), 3 = fp16 A rows (act of down),
// 4 = fp16 A rows (gate/up: the fused layer's normed x).  bq: B format (0 bf16, 1 Q8_0,
// 2 MXFP4; a.s0 / a.s1 hold the block scales); fp32 A takes bf16 B only.
template <int KIND, int AF, int MB>
static void launch_lds_b(const GemmArgs &a, int bf, unsigned grid, hipStream_t s) {
    if (bf == 1) {
        // (run_gemm refuses wide tiles with Q8_0 weights)
        if constexpr (MB != kMBWide) launch_kernel((k_gemm_lds<KIND, AF, MB, 1>), dim3(grid), dim3(kGThreads), 0, s, a);
    }
    else if (bf == 2) launch_kernel((k_gemm_lds<KIND, AF, MB, 2>), dim3(grid), dim3(kGThreads), 0, s, a);
    else launch_kernel((k_gemm_lds<KIND, AF, MB, 0>), dim3(grid), dim3(kGThreads), 0, s, a);
}

template <int KIND, int AF>
static void launch_lds(const GemmArgs &a, int bf, unsigned grid, hipStream_t s) {
    if (a.tile_rows == 32) launch_lds_b<KIND, AF, 1>(a, bf, grid, s);
    else if (a.tile_rows == 64) launch_lds_b<KIND, AF, 2>(a, bf, grid, s);
    else if (a.tile_rows == 96) launch_lds_b<KIND, AF, 3>(a, bf, grid, s);
    else if (a.tile_rows == kBMWide) launch_lds_b<KIND, AF, kMBWide>(a, bf, grid, s);
    else launch_lds_b<KIND, AF, kMB>(a, bf, grid, s);
}

// B format of a weight dtype: 0 bf16, 1 Q8_0, 2 MXFP4.
static int b_format(int dt) { return dt == DT_Q8 ? 1 : (dt == DT_MX4 ? 2 : 0); }

static hipError_t run_gemm(int kind, int a_mode, int bq, GemmArgs &a, hipStream_t s) {
    const int cols = kind == GK_GATEUP ? GemmShape<GK_GATEUP>::COLS : GemmShape<GK_PLAIN>::COLS;
    a.n_ntiles = (a.N + cols - 1) / cols;
    if (a.ksplit < 1) a.ksplit = 1;
    const int per_tile = a.n_ntiles * a.ksplit;
    if ((long)a.max_tiles * per_tile == 0) return hipSuccess;
    if (a_mode == 2) {
        // fp32 A (act handed in by a caller): register-staged kernel, A split
        // into bf16 hi/lo once per workgroup as it is written to LDS
        if (a.tile_rows != kBM || bq) return hipErrorInvalidValue;
        const unsigned grid = (unsigned)(((long)a.max_tiles * per_tile + 7) / 8 * 8);
        launch_kernel((k_gemm_reg<GK_PLAIN, true>), dim3(grid), dim3(kGThreads), 0, s, a);
    } else {
        a.units = per_tile;
        const unsigned grid = (unsigned)((long)a.max_tiles * a.units);
        if (a.tile_rows != 32 && a.tile_rows != 64 && a.tile_rows != 96 && a.tile_rows != kBM && !(a.tile_rows == kBMWide && bq != 1))
            return hipErrorInvalidValue;
        if (kind == GK_GATEUP && a_mode == 0) launch_lds<GK_GATEUP, AF_BF16>(a, bq, grid, s);
        else if (kind == GK_GATEUP && a_mode == 4) launch_lds<GK_GATEUP, AF_F16>(a, bq, grid, s);
        else if (kind == GK_PLAIN && a_mode == 3) launch_lds<GK_PLAIN, AF_F16>(a, bq, grid, s);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool mfma_supported(const Layer &L) {
    const auto ok = [](int dt) { return dt == DT_BF16 || dt == DT_Q8 || dt == DT_MX4; };
    return L.xdt == DT_BF16 && ok(L.edt) && (L.Is == 0 || ok(L.sdt)) && L.H % kBK == 0 && L.I % kBK == 0 &&
           L.Is % kBK == 0;
}

// Reduction slices of the routed down projection: enough workgroups to fill
// the chip (about 512) when an M-token batch has few token tiles (up to 16
// slices, for one-expert layers), keeping at least 4 K steps per slice.  The slices' outputs are summed, in slice order,
// by the combine.  Token tiles are estimated as at least one per expert the
// routes can touch.
int down_ksplit(const Layer &L, int M, int tile_rows) {
    const long R = (long)M * L.k;
    const long tiles = std::max(std::min(R, (long)L.E), (R + tile_rows - 1) / tile_rows);
    const long ntiles = (L.H + GemmShape<GK_PLAIN>::COLS - 1) / GemmShape<GK_PLAIN>::COLS;
    const int nk = L.I / kBK;
    int S = 1;
    while (tiles * ntiles * S < 512 && S < 16 && nk / (2 * S) >= 4) S *= 2;
    return S;
}

hipError_t launch_gateup_mfma(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                              const Mats &shared, const Routing &rt, int M, int max_tiles, int tile_rows,
                              float *act, float *shared_act, int act_fmt, hipStream_t s, bool x_half) {
    const int a_mode = x_half ? 4 : 0;
    if (act) {
        GemmArgs a{};
        a.tile_rows = tile_rows;
        a.a = x;
        a.sorted = rt.sorted;
        a.k_route = L.k;
        a.tiles = rt.tiles;
        a.offsets = rt.offsets;
        a.E = L.E;
        a.max_tiles = max_tiles;
        a.b0 = static_cast<const uint16_t *>(routed.gate);
        a.b1 = static_cast<const uint16_t *>(routed.up);
        a.b_stride = (size_t)L.I * L.H;
        a.s0 = static_cast<const uint16_t *>(routed.gate_s);
        a.s1 = static_cast<const uint16_t *>(routed.up_s);
        a.s_stride = (size_t)L.I * (L.H / 32);
        a.N = L.I;
        a.K = L.H;
        a.tok_scale = tok_scale;
        a.limit = L.limit;
        a.out = act;
        a.ldo = L.I;
        a.out_fmt = act_fmt;
        hipError_t err = run_gemm(GK_GATEUP, a_mode, b_format(L.edt), a, s);
        if (err != hipSuccess) return err;
    }
    if (shared_act && L.Is > 0) {
        GemmArgs a{};
        a.a = x;
        a.M = M;
        a.tile_rows = M <= 32 ? 32 : kBM;
        a.max_tiles = (M + a.tile_rows - 1) / a.tile_rows;
        a.b0 = static_cast<const uint16_t *>(shared.gate);
        a.b1 = static_cast<const uint16_t *>(shared.up);
        a.s0 = static_cast<const uint16_t *>(shared.gate_s);
        a.s1 = static_cast<const uint16_t *>(shared.up_s);
        a.N = L.Is;
        a.K = L.H;
        a.tok_scale = tok_scale;
        a.limit = 0.f; // the shared expert is not clamped
        a.out = shared_act;
        a.ldo = L.Is;
        a.out_fmt = act_fmt;
        return run_gemm(GK_GATEUP, a_mode, b_format(L.sdt), a, s);
    }
    return hipSuccess;
}

hipError_t launch_down_mfma(const Layer &L, const float *act, const float *shared_act,
                            const Mats &routed, const Mats &shared, const Routing &rt, int M,
                            int max_tiles, int tile_rows, float *y_routes, float *y_shared, int act_fmt,
                            hipStream_t s) {
    const int a_mode = act_fmt == ACT_F16 ? 3 : 2;
    if (act) {
        GemmArgs a{};
        a.a = act;
        a.tiles = rt.tiles;
        a.offsets = rt.offsets;
        a.E = L.E;
        a.max_tiles = max_tiles;
        a.tile_rows = tile_rows;
        a.ksplit = down_ksplit(L, M, tile_rows);
        a.slab = (size_t)M * L.k * L.H;
        a.b0 = static_cast<const uint16_t *>(routed.down);
        a.b_stride = (size_t)L.H * L.I;
        a.s0 = static_cast<const uint16_t *>(routed.down_s);
        a.s_stride = (size_t)L.H * (L.I / 32);
        a.N = L.H;
        a.K = L.I;
        a.out = y_routes;
        a.ldo = L.H;
        hipError_t err = run_gemm(GK_PLAIN, a_mode, b_format(L.edt), a, s);
        if (err != hipSuccess) return err;
    }
    if (shared_act && L.Is > 0) {
        GemmArgs a{};
        a.a = shared_act;
        a.M = M;
        a.tile_rows = act_fmt != ACT_F32 && M <= 32 ? 32 : kBM;
        a.max_tiles = (M + a.tile_rows - 1) / a.tile_rows;
        a.b0 = static_cast<const uint16_t *>(shared.down);
        a.s0 = static_cast<const uint16_t *>(shared.down_s);
        a.N = L.H;
        a.K = L.Is;
        a.out = y_shared;
        a.ldo = L.H;
        return run_gemm(GK_PLAIN, a_mode, b_format(L.sdt), a, s);
    }
    return hipSuccess;
}

// ------------------------------------------------------------------ router
// Router logits of the grouped-GEMM path, in reduction slices: workgroup
// (tile, s) computes part[s][t][e] = x[t] . router[e] over slice s of the
// reduction (32-element steps [s NS / S, (s+1) NS / S), at most
// kRpMaxSteps) for the 64 tokens of its tile and every expert, with
// v_mfma_f32_16x16x32_bf16.  The top-k kernel adds the S slices in slice
// order and applies the token scale.  x is read once: the tile's rows of the
// slice are staged in LDS, padded so that a row starts 64 bytes past a
// multiple of 512 (the 16-byte fragment reads of 16 rows and 4 k-groups then
// fall on 32 distinct bank groups); the router fragments go straight into
// registers, all issued before the staging.  Waves own expert tiles (16
// experts) w, w + 4, .. with all 4 token tiles when there are at least 4
// expert tiles, else token tile w with every expert tile (NJ: expert tiles a
// wave).  Workgroup b takes slice b % S.  (It replaced a kernel of one
// workgroup per 16 tokens x 16 experts over the whole reduction, whose
// workgroups each re-read x and the router rows: Qwen3-shaped M = 2048,
// 134 MB of L2 reads for 8.9 MB of operands.)  XS: x rows are split bf16
// hi/lo pairs (the fused layer's normed rows), one MFMA per half.  sqp (or
// null; bf16 rows only): each token's sum of squares over the slice,
// sqp[s][t], from the staged rows, for the pre-norm's scale, which the top-k
// then forms (no separate pass over x).
typedef float f32x4m __attribute__((ext_vector_type(4)));
constexpr int kRpTok = 64;
constexpr int kRpMaxSteps = 8;

int router_slices(const Layer &L, int M) {
    const int NS = L.H / 32, tiles = (M + kRpTok - 1) / kRpTok;
    int S = (NS + kRpMaxSteps - 1) / kRpMaxSteps;
    while (S < 16 && (long)tiles * S < 256 && 2 * S <= NS) S *= 2;
    return std::min(std::max(S, (NS + kRpMaxSteps - 1) / kRpMaxSteps), NS);
}

template <bool XS, int NJ, bool BYE>
__global__ __launch_bounds__(256) void k_router_part(const uint16_t *x, const uint16_t *router, int M, int E, int K,
                                                     int S, float *part, float *sqp) {
    constexpr int AP = XS ? 2 : 1;
    constexpr int MT = BYE ? 4 : 1; // token tiles a wave
    __shared__ __align__(16) unsigned char s_x[kRpTok * (kRpMaxSteps * 64 * AP + 64)];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int s = blockIdx.x % S, t0 = (blockIdx.x / S) * kRpTok;
    const int NS = K / 32, st0 = s * NS / S, nst = (s + 1) * NS / S - st0; // 1 <= nst <= kRpMaxSteps
    const int rowb = (nst * 64 * AP + 511) / 512 * 512 + 64;
    // router fragments: expert tile n_j, 8 reduction elements (lane / 16) of
    // each step (steps past the slice repeat its last; they are not used)
    u32x4 bf[NJ][kRpMaxSteps];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int n = BYE ? wave + 4 * j : j;
        const int e = min(n * 16 + (lane & 15), E - 1);
        const uint16_t *row = router + (size_t)e * K + st0 * 32 + (lane >> 4) * 8;
#pragma unroll
        for (int st = 0; st < kRpMaxSteps; st++)
            bf[j][st] = *reinterpret_cast<const u32x4 *>(row + min(st, nst - 1) * 32);
    }
    // stage the tile's x rows of the slice (16-byte chunks; rows past M repeat
    // row M - 1, chunks past the slice repeat its last)
    {
        const int cpr = nst * 4 * AP;
        constexpr int CPR = kRpMaxSteps * 4 * AP, U = kRpTok * CPR / 256;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = u * 256 + tid, r = i / CPR, c = min(i % CPR, cpr - 1), t = min(t0 + r, M - 1);
            v[u] = *reinterpret_cast<const u32x4 *>(x + ((size_t)t * K + st0 * 32) * AP + c * 8);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = u * 256 + tid, r = i / CPR, c = i % CPR;
            if (c < cpr) *reinterpret_cast<u32x4 *>(s_x + r * rowb + c * 16) = v[u];
        }
    }
    __syncthreads();
    if (!XS && sqp) {
        // four threads a token, each every fourth 16-byte chunk in order,
        // then a fixed-order sum of the four
        const int r = tid >> 2, q = tid & 3, cpr = nst * 4;
        float ss = 0.f;
        for (int c = q; c < cpr; c += 4) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(s_x + r * rowb + c * 16);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xffff0000u);
                ss = fmaf(lo, lo, ss);
                ss = fmaf(hi, hi, ss);
            }
        }
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        if (q == 0 && t0 + r < M) sqp[(size_t)s * M + t0 + r] = ss;
    }
    f32x4m acc[MT][NJ];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int j = 0; j < NJ; j++) acc[mt][j] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kRpMaxSteps; st++) {
        if (st < nst) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const int r = (BYE ? mt : wave) * 16 + (lane & 15);
                const unsigned char *ap = s_x + r * rowb + (st * 4 + (lane >> 4)) * 16 * AP;
                const u32x4 ah = *reinterpret_cast<const u32x4 *>(ap);
                u32x4 al;
                if constexpr (XS) al = *reinterpret_cast<const u32x4 *>(ap + 16);
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah),
                                                                         __builtin_bit_cast(bf16x8, bf[j][st]),
                                                                         acc[mt][j], 0, 0, 0);
                    if constexpr (XS)
                        acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al),
                                                                             __builtin_bit_cast(bf16x8, bf[j][st]),
                                                                             acc[mt][j], 0, 0, 0);
                }
            }
        }
    }
    // D rows are tokens (4 (lane / 16) + r), columns experts (lane % 16)
    float *ps = part + (size_t)s * M * E;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int n = BYE ? wave + 4 * j : j;
            const int e = n * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int t = t0 + (BYE ? mt : wave) * 16 + 4 * (lane >> 4) + r;
                if (t < M && e < E) ps[(size_t)t * E + e] = acc[mt][j][r];
            }
        }
    }
}

template <bool XS>
static void launch_router_part(const uint16_t *x, const uint16_t *router, int M, int E, int K, int S, float *part,
                               float *sqp, hipStream_t s) {
    const int NT = (E + 15) / 16;
    const dim3 grid((unsigned)(((M + kRpTok - 1) / kRpTok) * S));
#define RP_LAUNCH(NJ, BYE) \
    launch_kernel((k_router_part<XS, NJ, BYE>), grid, dim3(256), 0, s, x, router, M, E, K, S, part, sqp)
    if (NT == 1) RP_LAUNCH(1, false);
    else if (NT == 2) RP_LAUNCH(2, false);
    else if (NT == 3) RP_LAUNCH(3, false);
    else if (NT <= 4) RP_LAUNCH(1, true);
    else if (NT <= 8) RP_LAUNCH(2, true);
    else if (NT <= 12) RP_LAUNCH(3, true);
    else RP_LAUNCH(4, true);
#undef RP_LAUNCH
}

hipError_t launch_router_mfma(const Layer &L, const void *x, const void *router, int M, float *part, int S,
                              float *sqp, hipStream_t s, bool x_split) {
    if (x_split && sqp) return hipErrorInvalidValue;
    if (L.H % 32 || L.E > 256 || S < 1 || (L.H / 32 + S - 1) / S > kRpMaxSteps) return hipErrorInvalidValue;
    if (x_split)
        launch_router_part<true>(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(router), M, L.E,
                                 L.H, S, part, nullptr, s);
    else
        launch_router_part<false>(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(router), M, L.E,
                                  L.H, S, part, sqp, s);
    return hipGetLastError();
}

} // namespace moe
