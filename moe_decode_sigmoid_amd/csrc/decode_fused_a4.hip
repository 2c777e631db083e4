// The single-launch decode kernel in W4A4 (NVFP4 weights; NVFP4 activations
// with the Four Over Six block scale: the Inkling-2-Small article, 48-layer
// MoE section) for Flint's shape at batch 1 to 8: every workgroup quantises
// all of x after the router has read it, and every h pair after the h copy.
// The kernel body is in decode_layer.h.
#define MOE_DECODE_INSTANTIATES
#include "decode_layer.h"

namespace moe {

template <int B>
static bool a4_fits() {
  return one_per_cu(k_decode_fused<B, FMT_NVFP4, false, false, 1, true>);
}

bool fused_a4_supported(int B) {
  static int ok[64][kMaxB + 1] = {};
  int dev = 0;
  if (B < 1 || B > kMaxB) return false;
  if (!fused_supported() || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (ok[dev][B] == 0) {
    bool fits = false;
    switch (B) {
      case 1: fits = a4_fits<1>(); break;
      case 2: fits = a4_fits<2>(); break;
      case 3: fits = a4_fits<3>(); break;
      case 4: fits = a4_fits<4>(); break;
      case 5: fits = a4_fits<5>(); break;
      case 6: fits = a4_fits<6>(); break;
      case 7: fits = a4_fits<7>(); break;
      default: fits = a4_fits<8>(); break;
    }
    ok[dev][B] = fits ? 1 : -1;
  }
  return ok[dev][B] == 1;
}

template <int B>
static hipError_t launch_a4_b(const uint16_t* x, const uint16_t* rw, const ExpertsDev& routed,
                              const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                              uint8_t* ws, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  auto k = k_decode_fused<B, FMT_NVFP4, false, false, 1, true>;
  if (e0 && e1)
    hipExtLaunchKernelGGL(k, dim3(kFusedGrid), dim3(kFusedThreads), 0, st, e0, e1, 0, x, rw, routed,
                          shared, out, ids, w, ws, FuseDev{});
  else
    hipLaunchKernelGGL(k, dim3(kFusedGrid), dim3(kFusedThreads), 0, st, x, rw, routed, shared, out,
                       ids, w, ws, FuseDev{});
  return hipGetLastError();
}

hipError_t launch_decode_fused_a4(int B, const uint16_t* x, const uint16_t* rw,
                                  const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                                  int32_t* ids, float* w, uint8_t* ws, hipStream_t st, hipEvent_t e0,
                                  hipEvent_t e1) {
  switch (B) {
#define MOE_A4_CASE(b) \
  case b: return launch_a4_b<b>(x, rw, routed, shared, out, ids, w, ws, st, e0, e1);
    MOE_A4_CASE(1) MOE_A4_CASE(2) MOE_A4_CASE(3) MOE_A4_CASE(4)
    MOE_A4_CASE(5) MOE_A4_CASE(6) MOE_A4_CASE(7) MOE_A4_CASE(8)
#undef MOE_A4_CASE
    default: return hipErrorInvalidValue;
  }
}

// Exhaustive check of the converts the quantiser takes its roundings from
// (a4_e4m3_pk, a4_e2m1_pk8 / a4_e2m1_unpk8) against the roundings' own
// definitions (a4_e4m3_rne, a4_e2m1_rne): thread i of part p takes the 256
// fp32 bit patterns p 2^31 + 256 i + j.  counts[0]: E2M1 mismatches over all
// finite fp32 values; counts[1]: E4M3 mismatches over all non-negative
// finite ones.  A pattern's value is compared bit for bit.
constexpr int kCvtPerThread = 256;
__global__ __launch_bounds__(256) void k_a4_convert_check(unsigned long long* counts, uint32_t part) {
  const uint64_t base = ((uint64_t)part << 31) +
                        ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * kCvtPerThread;
  unsigned long long b0 = 0, b1 = 0;
  for (int j = 0; j < kCvtPerThread; j += 8) {
    float r[8], c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = (uint32_t)(base + j + i);
      r[i] = (u & 0x7F800000u) == 0x7F800000u ? 0.0f : __builtin_bit_cast(float, u);
    }
    a4_e2m1_unpk8(a4_e2m1_pk8(r), c);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (__builtin_bit_cast(uint32_t, c[i]) != __builtin_bit_cast(uint32_t, a4_e2m1_rne(r[i]))) b0++;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint32_t sc = a4_e4m3_pk(fabsf(r[i]), fabsf(r[i + 1]));
      if ((sc & 0xFFu) != a4_e4m3_rne(fabsf(r[i]))) b1++;
      if (((sc >> 8) & 0xFFu) != a4_e4m3_rne(fabsf(r[i + 1]))) b1++;
    }
  }
  if (b0) atomicAdd(counts + 0, b0);
  if (b1) atomicAdd(counts + 1, b1);
}

hipError_t launch_a4_convert_check(unsigned long long* counts, hipStream_t st) {
  hipError_t e = hipMemsetAsync(counts, 0, 2 * sizeof(unsigned long long), st);
  if (e != hipSuccess) return e;
  const unsigned blocks = (1u << 31) / kCvtPerThread / 256;
  for (uint32_t part = 0; part < 2; ++part)
    hipLaunchKernelGGL(k_a4_convert_check, dim3(blocks), dim3(256), 0, st, counts, part);
  return hipGetLastError();
}

}  // namespace moe
