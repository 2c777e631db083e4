// The single-launch decode kernel in W4A4 (NVFP4 weights; NVFP4 activations
// with the Four Over Six block scale: the Inkling-2-Small article, 48-layer
// MoE section) for Flint's shape at batch 1: every workgroup quantises x
// after the router has read it, and every h pair after the h copy.
// The kernel body is in decode_layer.h.
#define MOE_DECODE_INSTANTIATES
#include "decode_layer.h"

namespace moe {

bool fused_a4_supported() {
  static int ok[64] = {0};
  int dev = 0;
  if (!fused_supported() || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (ok[dev] == 0) ok[dev] = one_per_cu(k_decode_fused<1, FMT_NVFP4, false, false, 1, true>) ? 1 : -1;
  return ok[dev] == 1;
}

hipError_t launch_decode_fused_a4(const uint16_t* x, const uint16_t* rw, const ExpertsDev& routed,
                                  const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                                  uint8_t* ws, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  auto k = k_decode_fused<1, FMT_NVFP4, false, false, 1, true>;
  if (e0 && e1)
    hipExtLaunchKernelGGL(k, dim3(kFusedGrid), dim3(kFusedThreads), 0, st, e0, e1, 0, x, rw, routed,
                          shared, out, ids, w, ws, FuseDev{});
  else
    hipLaunchKernelGGL(k, dim3(kFusedGrid), dim3(kFusedThreads), 0, st, x, rw, routed, shared, out,
                       ids, w, ws, FuseDev{});
  return hipGetLastError();
}

}  // namespace moe
