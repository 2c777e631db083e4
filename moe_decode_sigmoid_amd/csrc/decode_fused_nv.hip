// Instances of the single-launch decode kernels for NVFP4 weights: one layer
// per launch (k_decode_fused: every batch size and fused-neighbour
// combination).
// The kernel body is in decode_layer.h.
#define MOE_DECODE_INSTANTIATES
#include "decode_layer.h"

namespace moe {

template hipError_t launch_fused_fmt<FMT_NVFP4>(int, const uint16_t*, const uint16_t*,
                                                const ExpertsDev&, const ExpertsDev&, uint16_t*,
                                                int32_t*, float*, uint8_t*, hipStream_t,
                                                hipEvent_t, hipEvent_t, const FuseDev&);
template bool occupancy_fused_fmt<FMT_NVFP4>();

}  // namespace moe
