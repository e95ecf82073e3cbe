// Internal launchers of the routed MoE kernels (host side).  Each returns the
// HIP error of its launch.  All pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct Layer {
    int H, E, k, I, Is;
    int select, bias_mode;
    float limit, eps;
    int xdt, rdt, edt, sdt; // DT_F32 / DT_BF16 / DT_Q8 / DT_MX4 (experts only)
};

// Weights of a set of SwiGLU experts: gate/up [n][W][H], down [n][H][W].
struct Mats {
    const void *gate, *up, *down;
    const void *gate_s, *up_s, *down_s; // block scale planes (Q8_0 fp16, MXFP4 E8M0) or null
};

// Router weights: rows [E][H] (fp32, bf16, or the int8 plane of Q8_0 rows),
// their Q8_0 fp16 block scales [E][H/32] (or null), and the router's
// per-element input scale (bf16 [H], or null for ones).
struct RouterW {
    const void *w, *w_s;
    const uint16_t *xs;
};

// Routing state produced by the permutation.
struct Routing {
    const int32_t *offsets;       // [E+1]
    const int32_t *sorted;        // [R]
    const int32_t *route_pos;     // [R]
    const int32_t *active;        // [1+E]: count, then touched experts ascending
    const int32_t *tiles;         // MFMA tile list: [0] count T, [1+e] first tile of expert e
                                  // (e = 0..E), then T pairs (expert, first sorted row)
};

hipError_t launch_rms_scale(const Layer &L, const void *x, int M, float *scale, hipStream_t s);
// xn = x * scale[t] * gamma (fp32 rows); xs (or null): the same rows split
// into bf16 hi/lo pairs (the grouped-GEMM router's input); xh (or null): the
// same rows as fp16 (the grouped GEMM's A).
hipError_t launch_norm_apply(const Layer &L, const void *x, const void *gamma, const float *scale, int M,
                             float *xn, uint16_t *xs, uint16_t *xh, hipStream_t s);
hipError_t launch_router(const Layer &L, const void *x, const RouterW &rw, const float *tok_scale,
                         int M, float *logits, hipStream_t s);
hipError_t launch_topk(const Layer &L, const float *logits, const float *bias, int M, int32_t *ids,
                       float *w, hipStream_t s);
hipError_t launch_permute(int E, int R, int tile_rows, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *sorted, int32_t *route_pos, int32_t *active,
                          int32_t *tiles, hipStream_t s);
// Top-k from S slices of partial logits part [S][M][E] (summed in slice
// order, times tok_scale[t] when given), writing also the expert counts of
// each group of tokens, hist [topk_hist_groups(M)][E]; then the stable
// scatter of the routes from ids and hist (several workgroups), with the
// outputs of launch_permute.
int topk_hist_groups(int M);
// With sqp (the router's partial sums of squares [S][M]) the token scale
// 1 / sqrt(sum / H + eps) is formed here, written to scale_out [M] and
// applied to the logits (tok_scale is then ignored).
hipError_t launch_topk_hist(const Layer &L, const float *part, int S, const float *tok_scale, const float *bias,
                            int M, int32_t *ids, float *w, int32_t *hist, hipStream_t s,
                            const float *sqp = nullptr, float *scale_out = nullptr);
hipError_t launch_scatter(int E, int M, int k, int tile_rows, const int32_t *ids, const int32_t *hist,
                          int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *route_pos, int32_t *active,
                          int32_t *tiles, hipStream_t s);
// Router + top-k + permutation for M <= route_small_max_tokens() (two launches).
int route_small_max_tokens();
hipError_t launch_route_small(const Layer &L, const void *x, const RouterW &rw, const float *bias,
                              const float *tok_scale, int M, float *logits, int32_t *ids, float *w,
                              int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *route_pos,
                              int32_t *active, hipStream_t s);
// The routing of a one-expert layer (k = 1), which needs no router: ids 0,
// weights 1, the identity order, counts, offsets, the touched list and (tiles
// non-null) the tile list of tile_rows-row tiles.  One launch.
hipError_t launch_route_one(int M, int tile_rows, int32_t *ids, float *w, int32_t *counts, int32_t *offsets,
                            int32_t *sorted, int32_t *route_pos, int32_t *active, int32_t *tiles, hipStream_t s);
// Derive the active-expert list and the tile list from offsets alone.
hipError_t launch_plan_from_offsets(int E, int tile_rows, const int32_t *offsets, int32_t *active,
                                    int32_t *tiles, hipStream_t s);

// GEMV path (any M; the expert's vectors are staged in LDS).
// Tokens one LDS stage of the gate/up kernel holds (0: hidden too large).
int gemv_stage_tokens(const Layer &L);
// With sel (M <= 16 tokens, gateup_stream_selects true) the streamed kernel
// runs the batch's selection from sel->logits itself and writes it to sel's
// outputs; rt's offsets, sorted and active are then those outputs.
struct SelectSmall;
bool gateup_stream_selects(const Layer &L, int M, bool shared);
hipError_t launch_gateup_gemv(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                              const Mats &shared, const Routing &rt, int M, float *act,
                              float *shared_act, hipStream_t s, const SelectSmall *sel = nullptr);
// Per-route down products, split over the reduction:
// y_routes [down_gemv_slices(I, edt)][M*k][H], y_shared [down_gemv_slices(Is, sdt)][M][H].
hipError_t launch_down_gemv(const Layer &L, const float *act, const float *shared_act, const Mats &routed,
                            const Mats &shared, const Routing &rt, int M, float *y_routes, float *y_shared,
                            hipStream_t s);
int down_gemv_slices(int width, int dt); // dt: the weights' format
// y[t] = seed[t] + sum_s y_shared[s][t] + sum_j w[t][j] * sum_s y_routes[s][route_pos[t*k+j]]
// (slices of a split reduction, slabs M*k*H and M*H apart).
hipError_t launch_combine(const Layer &L, const float *y_routes, const float *y_shared,
                          const int32_t *route_pos, const float *w, const float *seed, int M,
                          float *y, hipStream_t s, int slices, int shared_slices);
// Reduction slices of the MFMA down projection for an M-token call.
int down_ksplit(const Layer &L, int M, int tile_rows);

// M = 1 decode kernels (x shared by every touched expert).
bool m1_supported(const Layer &L);
// Router logits only (M <= route_small_max_tokens()).
hipError_t launch_router_small(const Layer &L, const void *x, const RouterW &rw, const float *tok_scale,
                               int M, float *logits, hipStream_t s);
// Top-k from the logits and gate/up in one kernel; writes ids_out / w_out
// ([k]) and counts_out ([E], may be null).
hipError_t launch_gateup_m1(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                            const Mats &shared, const float *logits, const float *bias, int32_t *ids_out,
                            float *w_out, int32_t *counts_out, float *act, float *shared_act,
                            hipStream_t s);
// Down projection and combine from the picks and weights the gate/up kernel wrote.
hipError_t launch_down_m1(const Layer &L, const float *act, const float *shared_act, const Mats &routed,
                          const Mats &shared, const int32_t *ids, const float *w, const float *seed,
                          float *y, hipStream_t s);

// MFMA grouped-GEMM path (bf16 x and experts).
int mfma_tile_rows();                          // tiles of the stage-wise entry points
int mfma_tile_rows(const Layer &L, int M);     // tiles of the layer call for M tokens
bool mfma_supported(const Layer &L);
// Partial router logits part [S][M][E] over S = router_slices(L, M) slices
// of the reduction (bf16 router; the token scale is left to the top-k), and,
// when sqp is given (bf16 x only), the tokens' partial sums of squares
// sqp [S][M] for the pre-norm.
// x_split: x rows are split bf16 hi/lo pairs (launch_norm_apply's xs) rather than bf16.
int router_slices(const Layer &L, int M);
hipError_t launch_router_mfma(const Layer &L, const void *x, const void *router, int M, float *part, int S,
                              float *sqp, hipStream_t s, bool x_split = false);
hipError_t launch_gateup_mfma(const Layer &L, const void *x, const float *tok_scale, const Mats &routed,
                              const Mats &shared, const Routing &rt, int M, int max_tiles, int tile_rows,
                              float *act, float *shared_act, int act_fmt, hipStream_t s,
                              bool x_half = false);
// act_fmt: the rows of act / shared_act.  ACT_F32: fp32 rows; ACT_F16: fp16
// rows (values beyond +-65504 saturate), which the down GEMM multiplies on
// fp16 MFMAs.
enum ActFormat { ACT_F32 = 0, ACT_F16 = 1 };
hipError_t launch_down_mfma(const Layer &L, const float *act, const float *shared_act,
                            const Mats &routed, const Mats &shared, const Routing &rt, int M,
                            int max_tiles, int tile_rows, float *y_routes, float *y_shared, int act_fmt,
                            hipStream_t s);

hipError_t launch_q8_split(const void *blocks, int64_t rows, int cols, int8_t *qs,
                           uint16_t *scales, hipStream_t s);
hipError_t launch_mxfp4_split(const void *blocks, int64_t rows, int cols, uint8_t *codes,
                              uint8_t *scales, hipStream_t s);

} // namespace moe
