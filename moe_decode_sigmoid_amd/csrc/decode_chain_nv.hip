// Instances of the single-launch decode kernels for NVFP4 weights: the chained
// residual stack (k_decode_chain: every batch size, with and without the
// RMSNorm).
// The kernel body is in decode_layer.h.
#define MOE_DECODE_INSTANTIATES
#include "decode_layer.h"

namespace moe {

template hipError_t launch_chain_fmt<FMT_NVFP4>(int, bool, const uint16_t*, const LayerDev*, int,
                                                const uint16_t*, float, uint16_t*, int32_t*,
                                                uint8_t*, hipStream_t);
template bool occupancy_chain_fmt<FMT_NVFP4>();

}  // namespace moe
