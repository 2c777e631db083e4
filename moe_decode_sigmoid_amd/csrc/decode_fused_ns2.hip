// Instances of the single-launch decode kernel for NVFP4 weights with two
// shared experts and Flint's shape otherwise (the Inkling shape of the
// Inkling-2-Small article's 48-layer MoE section, at Flint's widths): one
// layer per launch, no fused neighbours, every batch size.
// The kernel body is in decode_layer.h.
#define MOE_DECODE_INSTANTIATES
#include "decode_layer.h"

namespace moe {

template hipError_t launch_fused_ns2_fmt<FMT_NVFP4>(int, const uint16_t*, const uint16_t*,
                                                    const ExpertsDev&, const ExpertsDev&,
                                                    uint16_t*, int32_t*, float*, uint8_t*,
                                                    hipStream_t, hipEvent_t, hipEvent_t);
template bool occupancy_fused_ns2_fmt<FMT_NVFP4>();

}  // namespace moe
