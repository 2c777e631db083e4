// Instances of the stacked decode kernel (a stack of independent layers in one
// launch, k_decode_stack) for NVFP4 and BF16 weights, every batch size.  The
// kernel body is in decode_layer.h.
#define MOE_DECODE_INSTANTIATES
#include "decode_layer.h"

namespace moe {

template hipError_t launch_stack_fmt<FMT_NVFP4>(int, const uint16_t*, const LayerDev*, int,
                                                uint16_t*, int32_t*, uint8_t*, hipStream_t);
template bool occupancy_stack_fmt<FMT_NVFP4>();
template hipError_t launch_stack_fmt<FMT_BF16>(int, const uint16_t*, const LayerDev*, int,
                                               uint16_t*, int32_t*, uint8_t*, hipStream_t);
template bool occupancy_stack_fmt<FMT_BF16>();

}  // namespace moe
