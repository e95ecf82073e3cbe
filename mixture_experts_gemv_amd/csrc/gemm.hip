// MFMA grouped-GEMM path of the routed MoE layer (bf16, large batches).
#include "common.h"
#include "launch.h"

namespace moe {

int mfma_tile_rows() { return 128; }

hipError_t launch_gateup_mfma(const Layer &, const void *, const float *, const Mats &, const Mats &,
                              const Routing &, int, int, float *, float *, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_down_mfma(const Layer &, const float *, const float *, const Mats &, const Mats &,
                            const Routing &, int, int, float *, float *, hipStream_t) {
    return hipErrorNotSupported;
}

} // namespace moe
