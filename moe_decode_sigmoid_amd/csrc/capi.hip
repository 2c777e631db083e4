// C ABI of the gfx950 MoE layer library: argument checks, workspace sizing and
// launches on the caller's stream.  Declarations and the contract of each
// entry point are in include/moe_decode.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_decode.h"
#include "common.h"
#include "launch.h"


using moe::ExpertsDev;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The Flint layer (every entry point; the fused kernels).
moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->wfmt != MOE_W_NVFP4 && s->wfmt != MOE_W_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->hidden != moe::kH || s->inter != moe::kI || s->n_experts != moe::kE ||
      s->top_k != moe::kK || s->n_shared != 1)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// A shape the general decode path serves (any other than Flint's fast path).
bool general_shape(const moe_shape* s, moe::GenShape* g) {
  if (!s) return false;
  if (s->wfmt != MOE_W_NVFP4 && s->wfmt != MOE_W_BF16 && s->wfmt != MOE_W_MXFP8 &&
      s->wfmt != MOE_W_NVFP4_A4)
    return false;
  const bool ok = s->hidden >= 32 && s->hidden <= 8192 && s->hidden % 32 == 0 &&
                  s->inter >= 32 && s->inter <= 4096 && s->inter % 32 == 0 && s->top_k >= 1 &&
                  s->top_k <= moe::kGenMaxK && s->n_experts >= s->top_k &&
                  s->n_experts <= moe::kGenMaxE && s->n_shared >= 0 &&
                  s->n_shared <= moe::kGenMaxNS;
  if (ok && g) *g = moe::GenShape{s->hidden, s->inter, s->n_experts, s->top_k, s->n_shared};
  return ok;
}

// Decode entry points: the Flint layer, or a shape of the general path.
moe_status check_shape_decode(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (check_shape(s) == MOE_OK || general_shape(s, nullptr)) return MOE_OK;
  return MOE_ERR_UNSUPPORTED;
}
bool fast_path(const moe_shape* s) { return check_shape(s) == MOE_OK; }
bool split_path_forced();
// Flint's shape with two shared experts and NVFP4 weights (the Inkling
// shape at Flint's widths): a general shape that the single-launch kernel
// also serves, for the plain layer.
// Flint's shape in W4A4 at batch 1 to 8: the single-launch kernel, every
// workgroup quantising all of x and all of h itself (the general path
// quantises h once per pair, in a launch of its own).
bool a4_path(const moe_shape* s, int B) {
  return s && s->wfmt == MOE_W_NVFP4_A4 && B >= 1 && B <= moe::kMaxB && s->hidden == moe::kH &&
         s->inter == moe::kI && s->n_experts == moe::kE && s->top_k == moe::kK &&
         s->n_shared == 1 && moe::fused_a4_supported(B) && !split_path_forced();
}
bool ns2_path(const moe_shape* s) {
  return s && s->wfmt == MOE_W_NVFP4 && s->hidden == moe::kH && s->inter == moe::kI &&
         s->n_experts == moe::kE && s->top_k == moe::kK && s->n_shared == 2 &&
         moe::fused_ns2_supported() && !split_path_forced();
}

// Workspace bytes of the decode entry points for a checked shape.
size_t decode_ws_need(const moe_shape* s) {
  if (fast_path(s)) return moe::kDecodeWsBytes;
  moe::GenShape g;
  return general_shape(s, &g) ? moe::gen_ws_bytes(g) : 0;
}

moe_status check_ptr(const void* p, uintptr_t a = 16) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (!aligned(p, a)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status check_experts(const moe_experts* X, int fmt) {
  if (!X) return MOE_ERR_INVALID_ARG;
  moe_status st;
  if ((st = check_ptr(X->w13)) != MOE_OK) return st;
  if ((st = check_ptr(X->w2)) != MOE_OK) return st;
  if (fmt == MOE_W_NVFP4 || fmt == MOE_W_NVFP4_A4) {
    if ((st = check_ptr(X->w13_scale)) != MOE_OK) return st;
    if ((st = check_ptr(X->w2_scale)) != MOE_OK) return st;
    if ((st = check_ptr(X->global)) != MOE_OK) return st;
  } else if (fmt == MOE_W_MXFP8) {
    if ((st = check_ptr(X->w13_scale)) != MOE_OK) return st;
    if ((st = check_ptr(X->w2_scale)) != MOE_OK) return st;
    if (X->global) return MOE_ERR_INVALID_ARG;
  } else if (X->w13_scale || X->w2_scale || X->global) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

ExpertsDev to_dev(const moe_experts* X) {
  if (!X) return ExpertsDev{};
  return ExpertsDev{static_cast<const uint8_t*>(X->w13), static_cast<const uint8_t*>(X->w13_scale),
                    static_cast<const uint8_t*>(X->w2), static_cast<const uint8_t*>(X->w2_scale),
                    X->global};
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Checks common to moe_decode_forward and moe_prefill_forward (decode: the
// general shapes are served too).  The shared set may be NULL only when the
// shape has no shared expert.
moe_status check_forward(const moe_shape* shape, const void* x, int32_t T, const void* router_w,
                         const moe_experts* routed, const moe_experts* shared, const void* out,
                         const int32_t* ids_out, const float* w_out, const void* ws,
                         size_t ws_bytes, size_t ws_need, bool decode = false) {
  moe_status st;
  if ((st = decode ? check_shape_decode(shape) : check_shape(shape)) != MOE_OK) return st;
  if (T < 1) return MOE_ERR_INVALID_ARG;
  if ((st = check_ptr(x)) != MOE_OK) return st;
  if ((st = check_ptr(router_w)) != MOE_OK) return st;
  if ((st = check_ptr(out)) != MOE_OK) return st;
  if ((st = check_experts(routed, shape->wfmt)) != MOE_OK) return st;
  if (shape->n_shared > 0 && (st = check_experts(shared, shape->wfmt)) != MOE_OK) return st;
  if (ids_out && !aligned(ids_out, 4)) return MOE_ERR_MISALIGNED;
  if (w_out && !aligned(w_out, 4)) return MOE_ERR_MISALIGNED;
  if (!ws || ws_need == 0 || ws_bytes < ws_need) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_MISALIGNED;
  const size_t xb = (size_t)T * shape->hidden * 2;
  if (overlap(out, xb, x, xb)) return MOE_ERR_INVALID_ARG;
  if (overlap(out, xb, ws, ws_bytes)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Checks of the fused neighbours for T tokens (fuse may be NULL) and their
// device form.
moe_status check_fuse(const moe_fuse* f, int32_t T, const void* x, const void* out,
                      const void* ws, size_t ws_bytes, moe::FuseDev* dev) {
  *dev = moe::FuseDev{};
  if (!f) return MOE_OK;
  moe_status st;
  const size_t xb = (size_t)T * moe::kH * 2, wb = (size_t)moe::kH * 2;
  if (f->norm_w) {
    if ((st = check_ptr(f->norm_w)) != MOE_OK) return st;
    if (!(f->norm_eps > 0.0f) || !(f->norm_eps < INFINITY)) return MOE_ERR_INVALID_ARG;
    if (overlap(f->norm_w, wb, out, xb) || overlap(f->norm_w, wb, ws, ws_bytes))
      return MOE_ERR_INVALID_ARG;
  }
  if (f->residual) {
    if ((st = check_ptr(f->residual)) != MOE_OK) return st;
    if (f->residual != out && overlap(f->residual, xb, out, xb)) return MOE_ERR_INVALID_ARG;
    if (overlap(f->residual, xb, ws, ws_bytes)) return MOE_ERR_INVALID_ARG;
  }
  if (f->xn_out) {
    if (!f->norm_w) return MOE_ERR_INVALID_ARG;
    if ((st = check_ptr(f->xn_out)) != MOE_OK) return st;
    if (overlap(f->xn_out, xb, x, xb) || overlap(f->xn_out, xb, out, xb) ||
        overlap(f->xn_out, xb, ws, ws_bytes) || overlap(f->xn_out, xb, f->norm_w, wb) ||
        (f->residual && overlap(f->xn_out, xb, f->residual, xb)))
      return MOE_ERR_INVALID_ARG;
  }
  dev->norm_w = static_cast<const uint16_t*>(f->norm_w);
  dev->eps = f->norm_eps;
  dev->resid = static_cast<const uint16_t*>(f->residual);
  dev->xn_out = static_cast<uint16_t*>(f->xn_out);
  return MOE_OK;
}

// MOE_DECODE_SPLIT=1 selects the three-launch decode path even where the
// fused kernel can run (both compute the same layer; read on every call so a
// test can compare the two in one process).
bool split_path_forced() {
  const char* v = getenv("MOE_DECODE_SPLIT");
  return v && v[0] == '1';
}

// ------------------------------------------------ the allocation-free variant
// The workspace of moe_decode_forward_noalloc: one per device (each GPU the
// library runs on holds its own copy until the process ends), the size of the
// Flint decode workspace.  In host code `scratch` is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[moe::kDecodeWsBytes];

__global__ __launch_bounds__(256) void k_zero_scratch(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];   // the device address of `scratch`, per device

// The current device's scratch address, looked up (and the array zero-filled
// by a kernel on `st`, ahead of the call that needs it) on the first call on
// that device.  nullptr on failure.
uint8_t* scratch_for_current_device(hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    // the decode kernels' call counters must start from zero: a fill kernel
    // (no memset node, so the first call may also be captured in a graph)
    hipLaunchKernelGGL(k_zero_scratch, dim3(256), dim3(256), 0, st, static_cast<uint4*>(ptr),
                       moe::kDecodeWsBytes / 16);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  return g_scratch_ptr[dev];
}
static_assert(moe::kDecodeWsBytes % 16 == 0, "scratch is cleared in 16-byte words");

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 1; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(const moe_shape* shape, int32_t tokens, int32_t prefill) {
  if (tokens < 1) return 0;
  if (!prefill) return tokens <= moe::kMaxB ? decode_ws_need(shape) : 0;
  if (check_shape(shape) != MOE_OK) return 0;
  return moe::prefill_ws_bytes(tokens);
}

moe_status moe_decode_route(const moe_shape* shape, const void* x, int32_t B, const void* router_w,
                            int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  if ((st = check_shape_decode(shape)) != MOE_OK) return st;
  if (B < 1) return MOE_ERR_INVALID_ARG;
  if (B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;
  if ((st = check_ptr(x)) != MOE_OK) return st;
  if ((st = check_ptr(router_w)) != MOE_OK) return st;
  if (!ids || !w) return MOE_ERR_INVALID_ARG;
  if (!aligned(ids, 4) || !aligned(w, 4)) return MOE_ERR_MISALIGNED;
  if (!ws || ws_bytes < decode_ws_need(shape)) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_MISALIGNED;
  moe::GenShape g;
  if (!fast_path(shape) && general_shape(shape, &g)) {
    const hipError_t e = moe::launch_route_general(
        B, g, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router_w), ids, w,
        static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  const ExpertsDev none{};
  hipError_t e = moe::launch_decode(B, shape->wfmt, true, static_cast<const uint16_t*>(x),
                                    static_cast<const uint16_t*>(router_w), none, none, nullptr,
                                    ids, w, static_cast<uint8_t*>(ws),
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_forward(const moe_shape* shape, const void* x, int32_t B,
                              const void* router_w, const moe_experts* routed,
                              const moe_experts* shared, void* out, int32_t* ids_out,
                              float* w_out, void* ws, size_t ws_bytes, void* stream) {
  if (shape && check_shape_decode(shape) == MOE_OK && B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_forward(shape, x, B, router_w, routed, shared, out, ids_out, w_out, ws,
                                ws_bytes, decode_ws_need(shape), true);
  if (st != MOE_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  moe::GenShape g;
  if (a4_path(shape, B)) {
    const hipError_t e = moe::launch_decode_fused_a4(
        B, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router_w), to_dev(routed),
        to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out, static_cast<uint8_t*>(ws), s);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  if (ns2_path(shape)) {
    const hipError_t e = moe::launch_decode_fused_ns2(
        B, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router_w), to_dev(routed),
        to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out, static_cast<uint8_t*>(ws), s);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  if (!fast_path(shape) && general_shape(shape, &g)) {
    const hipError_t e = moe::launch_decode_general(
        B, shape->wfmt, g, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router_w),
        to_dev(routed), to_dev(shape->n_shared > 0 ? shared : nullptr),
        static_cast<uint16_t*>(out), ids_out, w_out, static_cast<uint8_t*>(ws), s);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  const bool fused = moe::fused_supported() && !split_path_forced();
  const hipError_t e =
      fused ? moe::launch_decode_fused(B, shape->wfmt, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(router_w), to_dev(routed),
                                       to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                       static_cast<uint8_t*>(ws), s)
            : moe::launch_decode_split(B, shape->wfmt, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(router_w), to_dev(routed),
                                       to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                       static_cast<uint8_t*>(ws), s);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_forward_noalloc(const moe_shape* shape, const void* x, int32_t B,
                                      const void* router_w, const moe_experts* routed,
                                      const moe_experts* shared, void* out, int32_t* ids_out,
                                      float* w_out, void* stream) {
  moe_status st;
  if ((st = check_shape(shape)) != MOE_OK) return st;
  if (B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;   // beyond what the scratch array holds
  // the checks of moe_decode_forward; the workspace checks pass trivially (a
  // 256-byte host stand-in: the device array lies in no caller's allocation)
  alignas(256) static uint8_t ws_stand_in[256];
  if ((st = check_forward(shape, x, B, router_w, routed, shared, out, ids_out, w_out,
                          ws_stand_in, sizeof ws_stand_in, sizeof ws_stand_in, true)) != MOE_OK)
    return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = scratch_for_current_device(s);
  if (!ws) return MOE_ERR_HIP;
  const bool fused = moe::fused_supported() && !split_path_forced();
  const hipError_t e =
      fused ? moe::launch_decode_fused(B, shape->wfmt, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(router_w), to_dev(routed),
                                       to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                       ws, s)
            : moe::launch_decode_split(B, shape->wfmt, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(router_w), to_dev(routed),
                                       to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                       ws, s);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_forward_timed(const moe_shape* shape, const void* x, int32_t B,
                                    const void* router_w, const moe_experts* routed,
                                    const moe_experts* shared, void* out, int32_t* ids_out,
                                    float* w_out, void* ws, size_t ws_bytes, void* stream,
                                    void* ev_start, void* ev_stop) {
  if (!ev_start || !ev_stop) return MOE_ERR_INVALID_ARG;
  if (shape && check_shape_decode(shape) == MOE_OK && B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_forward(shape, x, B, router_w, routed, shared, out, ids_out, w_out, ws,
                                ws_bytes, decode_ws_need(shape), true);
  if (st != MOE_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
  hipError_t e;
  moe::GenShape g;
  if (a4_path(shape, B)) {
    e = moe::launch_decode_fused_a4(B, static_cast<const uint16_t*>(x),
                                    static_cast<const uint16_t*>(router_w), to_dev(routed),
                                    to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                    static_cast<uint8_t*>(ws), s, e0, e1);
  } else if (ns2_path(shape)) {
    e = moe::launch_decode_fused_ns2(B, static_cast<const uint16_t*>(x),
                                     static_cast<const uint16_t*>(router_w), to_dev(routed),
                                     to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                     static_cast<uint8_t*>(ws), s, e0, e1);
  } else if (!fast_path(shape) && general_shape(shape, &g)) {
    e = hipEventRecord(e0, s);
    if (e == hipSuccess)
      e = moe::launch_decode_general(
          B, shape->wfmt, g, static_cast<const uint16_t*>(x),
          static_cast<const uint16_t*>(router_w), to_dev(routed),
          to_dev(shape->n_shared > 0 ? shared : nullptr), static_cast<uint16_t*>(out), ids_out,
          w_out, static_cast<uint8_t*>(ws), s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
  } else if (moe::fused_supported() && !split_path_forced()) {
    e = moe::launch_decode_fused(B, shape->wfmt, static_cast<const uint16_t*>(x),
                                 static_cast<const uint16_t*>(router_w), to_dev(routed),
                                 to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                 static_cast<uint8_t*>(ws), s, e0, e1);
  } else {
    e = hipEventRecord(e0, s);
    if (e == hipSuccess)
      e = moe::launch_decode_split(B, shape->wfmt, static_cast<const uint16_t*>(x),
                                   static_cast<const uint16_t*>(router_w), to_dev(routed),
                                   to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                   static_cast<uint8_t*>(ws), s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_prefill_forward(const moe_shape* shape, const void* x, int32_t T,
                               const void* router_w, const moe_experts* routed,
                               const moe_experts* shared, void* out, int32_t* ids_out,
                               float* w_out, void* ws, size_t ws_bytes, void* stream) {
  const size_t need = (shape && check_shape(shape) == MOE_OK && T >= 1) ? moe::prefill_ws_bytes(T) : 0;
  moe_status st = check_forward(shape, x, T, router_w, routed, shared, out, ids_out, w_out, ws,
                                ws_bytes, need == 0 ? 1 : need);
  if (st != MOE_OK) return st;
  if (need == 0) return MOE_ERR_UNSUPPORTED;
  hipError_t e = moe::launch_prefill(T, shape->wfmt, static_cast<const uint16_t*>(x),
                                     static_cast<const uint16_t*>(router_w), to_dev(routed),
                                     to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                     static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_forward_ex(const moe_shape* shape, const void* x, int32_t B,
                                 const moe_fuse* fuse, const void* router_w,
                                 const moe_experts* routed, const moe_experts* shared, void* out,
                                 int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (shape && check_shape(shape) == MOE_OK && B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_forward(shape, x, B, router_w, routed, shared, out, ids_out, w_out, ws,
                                ws_bytes, moe::kDecodeWsBytes);
  if (st != MOE_OK) return st;   // shapes other than Flint's: MOE_ERR_UNSUPPORTED
  moe::FuseDev fz;
  if ((st = check_fuse(fuse, B, x, out, ws, ws_bytes, &fz)) != MOE_OK) return st;
  if (!moe::fused_supported()) return MOE_ERR_UNSUPPORTED;
  const hipError_t e = moe::launch_decode_fused(
      B, shape->wfmt, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router_w),
      to_dev(routed), to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
      static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream), nullptr, nullptr, fz);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_prefill_forward_ex(const moe_shape* shape, const void* x, int32_t T,
                                  const moe_fuse* fuse, const void* router_w,
                                  const moe_experts* routed, const moe_experts* shared, void* out,
                                  int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes,
                                  void* stream) {
  const size_t need = (shape && check_shape(shape) == MOE_OK && T >= 1) ? moe::prefill_ws_bytes(T) : 0;
  moe_status st = check_forward(shape, x, T, router_w, routed, shared, out, ids_out, w_out, ws,
                                ws_bytes, need == 0 ? 1 : need);
  if (st != MOE_OK) return st;
  if (need == 0) return MOE_ERR_UNSUPPORTED;
  moe::FuseDev fz;
  if ((st = check_fuse(fuse, T, x, out, ws, ws_bytes, &fz)) != MOE_OK) return st;
  hipError_t e = moe::launch_prefill(T, shape->wfmt, static_cast<const uint16_t*>(x),
                                     static_cast<const uint16_t*>(router_w), to_dev(routed),
                                     to_dev(shared), static_cast<uint16_t*>(out), ids_out, w_out,
                                     static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream),
                                     fz);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static_assert(sizeof(moe_layer) == sizeof(moe::LayerDev), "moe_layer is the device layer record");
static_assert(sizeof(moe_experts) == sizeof(moe::ExpertsDev), "moe_experts is the device set");

moe_status moe_decode_stack_forward(const moe_shape* shape, int32_t n_layers,
                                    const moe_layer* layers, const void* x, int32_t B, void* out,
                                    int32_t* ids_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  if ((st = check_shape(shape)) != MOE_OK) return st;
  if (B < 1 || n_layers < 1) return MOE_ERR_INVALID_ARG;
  if (B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;
  if (!layers) return MOE_ERR_INVALID_ARG;
  if (!aligned(layers, 8)) return MOE_ERR_MISALIGNED;
  if ((st = check_ptr(x)) != MOE_OK) return st;
  if ((st = check_ptr(out)) != MOE_OK) return st;
  if (ids_out && !aligned(ids_out, 4)) return MOE_ERR_MISALIGNED;
  if (!ws || ws_bytes < moe::kDecodeWsBytes) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_MISALIGNED;
  const size_t xb = (size_t)B * moe::kH * 2, ob = xb * (size_t)n_layers;
  if (overlap(out, ob, x, xb) || overlap(out, ob, ws, ws_bytes)) return MOE_ERR_INVALID_ARG;
  if (overlap(layers, sizeof(moe_layer) * (size_t)n_layers, out, ob)) return MOE_ERR_INVALID_ARG;
  if (!moe::fused_supported()) return MOE_ERR_UNSUPPORTED;
  const hipError_t e = moe::launch_decode_stack(
      B, shape->wfmt, static_cast<const uint16_t*>(x),
      reinterpret_cast<const moe::LayerDev*>(layers), n_layers, static_cast<uint16_t*>(out),
      ids_out, static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_chain_forward(const moe_shape* shape, int32_t n_layers,
                                    const moe_layer* layers, const void* x, int32_t B,
                                    const void* norm_w, float norm_eps, void* out,
                                    int32_t* ids_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  if ((st = check_shape(shape)) != MOE_OK) return st;
  if (B < 1 || n_layers < 1) return MOE_ERR_INVALID_ARG;
  if (B > moe::kMaxB) return MOE_ERR_UNSUPPORTED;
  if (!layers) return MOE_ERR_INVALID_ARG;
  if (!aligned(layers, 8)) return MOE_ERR_MISALIGNED;
  if ((st = check_ptr(x)) != MOE_OK) return st;
  if ((st = check_ptr(out)) != MOE_OK) return st;
  if (norm_w) {
    if ((st = check_ptr(norm_w)) != MOE_OK) return st;
    if (!(norm_eps > 0.0f) || !(norm_eps < INFINITY)) return MOE_ERR_INVALID_ARG;
  }
  if (ids_out && !aligned(ids_out, 4)) return MOE_ERR_MISALIGNED;
  if (!ws || ws_bytes < moe::kDecodeWsBytes) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_MISALIGNED;
  const size_t xb = (size_t)B * moe::kH * 2, ob = xb * (size_t)n_layers;
  const size_t nb = (size_t)n_layers * moe::kH * 2;
  if (overlap(out, ob, x, xb) || overlap(out, ob, ws, ws_bytes)) return MOE_ERR_INVALID_ARG;
  if (overlap(layers, sizeof(moe_layer) * (size_t)n_layers, out, ob)) return MOE_ERR_INVALID_ARG;
  if (norm_w && (overlap(norm_w, nb, out, ob) || overlap(norm_w, nb, ws, ws_bytes)))
    return MOE_ERR_INVALID_ARG;
  if (!moe::fused_supported()) return MOE_ERR_UNSUPPORTED;
  const hipError_t e = moe::launch_decode_chain(
      B, shape->wfmt, static_cast<const uint16_t*>(x),
      reinterpret_cast<const moe::LayerDev*>(layers), n_layers,
      static_cast<const uint16_t*>(norm_w), norm_eps, static_cast<uint16_t*>(out), ids_out,
      static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_workspace_status(void* ws, size_t ws_bytes, int32_t* status, void* stream) {
  if (!ws || ws_bytes < moe::kCtlBytes) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_MISALIGNED;
  if (!status) return MOE_ERR_INVALID_ARG;
  if (!aligned(status, 4)) return MOE_ERR_MISALIGNED;
  if (overlap(status, 4, ws, ws_bytes)) return MOE_ERR_INVALID_ARG;
  const hipError_t e = moe::launch_ws_status(static_cast<uint8_t*>(ws), status,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_general_workspace_layout(const moe_shape* shape, size_t offsets[8]) {
  moe::GenShape g;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (fast_path(shape) || !general_shape(shape, &g)) return MOE_ERR_UNSUPPORTED;
  static_assert(moe::kGenMaxEntries == 66 && moe::kMaxB == 8, "layout documented in the header");
  const moe::GenLayout L = moe::gen_layout(g);
  offsets[0] = L.ctl + offsetof(moe::GenCtl, n_entries);
  offsets[1] = L.ctl + offsetof(moe::GenCtl, entry);
  offsets[2] = L.ctl + offsetof(moe::GenCtl, amask);
  offsets[3] = L.h;
  offsets[4] = L.xq;
  offsets[5] = L.gx;
  offsets[6] = L.hq;
  offsets[7] = L.gh;
  return MOE_OK;
}

moe_status moe_nvfp4_dequant(const moe_shape* shape, const moe_experts* set, int32_t expert,
                             int32_t tensor, float* out, void* stream) {
  moe_status st;
  if ((st = check_shape(shape)) != MOE_OK) return st;
  if (shape->wfmt != MOE_W_NVFP4) return MOE_ERR_UNSUPPORTED;
  if ((st = check_experts(set, MOE_W_NVFP4)) != MOE_OK) return st;
  if ((st = check_ptr(out)) != MOE_OK) return st;
  if (expert < 0 || tensor < 0 || tensor > 2) return MOE_ERR_INVALID_ARG;
  const ExpertsDev X = to_dev(set);
  const size_t mat = (size_t)moe::kH * moe::kI;
  const uint8_t* codes;
  const uint8_t* scales;
  int rows, cols;
  if (tensor < 2) {
    codes = X.w13 + ((size_t)expert * 2 + tensor) * (mat / 2);
    scales = X.w13s + ((size_t)expert * 2 + tensor) * (mat / 16);
    rows = moe::kI;
    cols = moe::kH;
  } else {
    codes = X.w2 + (size_t)expert * (mat / 2);
    scales = X.w2s + (size_t)expert * (mat / 16);
    rows = moe::kH;
    cols = moe::kI;
  }
  hipError_t e = moe::launch_dequant(codes, scales, X.glob + (size_t)expert * 3 + tensor, rows,
                                     cols, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_a4_convert_check(uint64_t* counts, void* stream) {
  moe_status st;
  if ((st = check_ptr(counts, 8)) != MOE_OK) return st;
  hipError_t e = moe::launch_a4_convert_check(reinterpret_cast<unsigned long long*>(counts),
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_nvfp4_gemv(const void* x, int32_t B, int32_t K, int32_t N, const void* codes,
                          const void* scales, const float* global, void* y, void* stream) {
  moe_status st;
  if ((st = check_ptr(x)) != MOE_OK) return st;
  if ((st = check_ptr(codes)) != MOE_OK) return st;
  if ((st = check_ptr(scales, 2)) != MOE_OK) return st;
  if ((st = check_ptr(global, 4)) != MOE_OK) return st;
  if ((st = check_ptr(y, 2)) != MOE_OK) return st;
  if (B < 1 || N < 1 || K < 32 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (B > moe::kMaxB || K > moe::kGemvMaxK || B * K > moe::kGemvMaxBK) return MOE_ERR_UNSUPPORTED;
  if (overlap(y, (size_t)B * N * 2, x, (size_t)B * K * 2)) return MOE_ERR_INVALID_ARG;
  hipError_t e = moe::launch_nvfp4_gemv(B, K, N, static_cast<const uint16_t*>(x),
                                        static_cast<const uint8_t*>(codes),
                                        static_cast<const uint8_t*>(scales), global,
                                        static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
