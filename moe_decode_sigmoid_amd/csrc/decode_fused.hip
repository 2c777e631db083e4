// Host side of the single-launch decode kernels (layer body in decode_layer.h,
// instances in decode_fused_*.hip, decode_stack.hip, decode_chain_*.hip):
// whether the device can run them, the dispatch by weight format, and the
// workspace's wait-status read-back.
//
// The kernels need all 256 workgroups resident at the same time (they hand
// data to each other inside the launch, with bounded waits).  A device with
// fewer compute units cannot run them (fused_supported() is false and the
// entry points fall back or return MOE_ERR_UNSUPPORTED); on a device that has
// them, other work occupying compute units during a call can leave
// workgroups undispatched while the others wait, the waits give up and the
// call's output is invalid: the error word records it and
// moe_workspace_status reads it back.
#include "decode_layer.h"

namespace moe {

// The workspace's wait status: the error word, copied to the caller and
// cleared in one atomic exchange (a kernel, so that it can be captured).
__global__ __launch_bounds__(64) void k_ws_status(uint8_t* __restrict__ ws,
                                                 int32_t* __restrict__ status) {
  if (threadIdx.x == 0) {
    DecodeCtl* ctl = reinterpret_cast<DecodeCtl*>(ws);
    const unsigned v =
        __hip_atomic_exchange(&ctl->err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *status = (int32_t)v;
  }
}

hipError_t launch_ws_status(uint8_t* ws, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_ws_status, dim3(1), dim3(64), 0, st, ws, status);
  return hipGetLastError();
}

static int g_fused_ok[64];   // per device: 0 unknown, 1 usable, -1 not

bool fused_supported() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (g_fused_ok[dev] == 0) {
    int cus = 0;
    const bool ok =
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus >= kFusedGrid && occupancy_fused_fmt<FMT_NVFP4>() &&
        occupancy_fused_fmt<FMT_BF16>() && occupancy_stack_fmt<FMT_NVFP4>() &&
        occupancy_stack_fmt<FMT_BF16>() && occupancy_chain_fmt<FMT_NVFP4>() &&
        occupancy_chain_fmt<FMT_BF16>();
    g_fused_ok[dev] = ok ? 1 : -1;
  }
  return g_fused_ok[dev] == 1;
}

hipError_t launch_decode_fused(int B, int fmt, const uint16_t* x, const uint16_t* rw,
                               const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                               int32_t* ids, float* w, uint8_t* ws, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1, const FuseDev& fz) {
  return fmt == FMT_NVFP4
             ? launch_fused_fmt<FMT_NVFP4>(B, x, rw, routed, shared, out, ids, w, ws, st, e0, e1, fz)
             : launch_fused_fmt<FMT_BF16>(B, x, rw, routed, shared, out, ids, w, ws, st, e0, e1, fz);
}

bool fused_ns2_supported() {
  static int ok[64] = {0};
  int dev = 0;
  if (!fused_supported() || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (ok[dev] == 0) ok[dev] = occupancy_fused_ns2_fmt<FMT_NVFP4>() ? 1 : -1;
  return ok[dev] == 1;
}

hipError_t launch_decode_fused_ns2(int B, const uint16_t* x, const uint16_t* rw,
                                   const ExpertsDev& routed, const ExpertsDev& shared,
                                   uint16_t* out, int32_t* ids, float* w, uint8_t* ws,
                                   hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return launch_fused_ns2_fmt<FMT_NVFP4>(B, x, rw, routed, shared, out, ids, w, ws, st, e0, e1);
}

hipError_t launch_decode_stack(int B, int fmt, const uint16_t* x, const LayerDev* layers, int L,
                               uint16_t* out, int32_t* ids, uint8_t* ws, hipStream_t st) {
  return fmt == FMT_NVFP4 ? launch_stack_fmt<FMT_NVFP4>(B, x, layers, L, out, ids, ws, st)
                          : launch_stack_fmt<FMT_BF16>(B, x, layers, L, out, ids, ws, st);
}

hipError_t launch_decode_chain(int B, int fmt, const uint16_t* x, const LayerDev* layers, int L,
                               const uint16_t* norm_w, float eps, uint16_t* out, int32_t* ids,
                               uint8_t* ws, hipStream_t st) {
  const bool norm = norm_w != nullptr;
  return fmt == FMT_NVFP4
             ? launch_chain_fmt<FMT_NVFP4>(B, norm, x, layers, L, norm_w, eps, out, ids, ws, st)
             : launch_chain_fmt<FMT_BF16>(B, norm, x, layers, L, norm_w, eps, out, ids, ws, st);
}

}  // namespace moe
