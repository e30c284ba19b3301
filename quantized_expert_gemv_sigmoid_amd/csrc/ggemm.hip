// Grouped MFMA GEMM path for large token counts (prefill).
#include "../../include/moe.h"
#include "common.h"

namespace moe {

bool mfma_supported(const Shape &) { return false; }

size_t mfma_extra_workspace(const Shape &) { return 0; }

hipError_t launch_mfma_experts(const Shape &, const uint16_t *, const moe_layer_desc *, int,
                               const Work &, hipStream_t, hipEvent_t const *)
{
    return hipErrorNotSupported;
}

}  // namespace moe
