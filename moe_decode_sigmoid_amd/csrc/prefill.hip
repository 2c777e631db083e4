// Prefill path of the gfx950 MoE layer (placeholder until the grouped GEMM lands).
#include "common.h"
#include "launch.h"

namespace moe {

size_t prefill_ws_bytes(int) { return 0; }

hipError_t launch_prefill(int, int, const uint16_t*, const uint16_t*, const ExpertsDev&,
                          const ExpertsDev&, uint16_t*, int32_t*, float*, uint8_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
