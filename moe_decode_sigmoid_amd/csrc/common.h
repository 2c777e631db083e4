// Shared device-side definitions of the gfx950 MoE layer kernels.
//
// Shape ("Day-0 Support for Flint on vLLM", Model architecture): hidden 2048,
// 256 routed experts chosen by a sigmoid top-6, one shared expert; expert
// intermediate size 512.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kH = 2048;          // hidden
constexpr int kI = 512;           // expert intermediate
constexpr int kE = 256;           // routed experts
constexpr int kK = 6;             // experts per token
constexpr int kMaxB = 8;          // low-latency decode batch limit
constexpr int kMaxActive = kMaxB * kK + 1;   // distinct experts of one decode call + shared
constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// One expert set as the kernels see it (layouts in include/moe_decode.h).
struct ExpertsDev {
  const uint8_t* w13;    // NVFP4 codes u8 [n][2][I][H/2] | BF16 [n][2][I][H]
  const uint8_t* w13s;   // NVFP4 scales u8 [n][2][I][H/16]
  const uint8_t* w2;     // NVFP4 codes u8 [n][H][I/2]    | BF16 [n][H][I]
  const uint8_t* w2s;    // NVFP4 scales u8 [n][H][I/16]
  const float* glob;     // NVFP4 f32 [n][3]
};

enum { FMT_NVFP4 = 0, FMT_BF16 = 1 };

// ---------------------------------------------------------------- workspace
// Decode workspace, all offsets in bytes from a 256-byte-aligned base.
struct DecodeCtl {
  unsigned ticket;                       // route kernel arrival counter (self-resetting)
  int n_active;                          // routed experts touched + 1 (shared last)
  int pad0[62];
  int active_expert[64];                 // expert id; kE marks the shared expert
  unsigned active_mask[64];              // bit t set when token t uses the entry
  float wtab[64][kMaxB];                 // routing weight of token t for the entry
  int ids[kMaxB][kK];                    // routing of the call (descending score)
  float w[kMaxB][kK];
};
constexpr size_t kCtlBytes = (sizeof(DecodeCtl) + 255) / 256 * 256;
constexpr size_t kLogitsOff = kCtlBytes;                          // f32 [kMaxB][kE]
constexpr size_t kHOff = kLogitsOff + sizeof(float) * kMaxB * kE; // f32 [kMaxActive][kMaxB][kI]
constexpr size_t kDecodeWsBytes = kHOff + sizeof(float) * kMaxActive * kMaxB * kI;

// ---------------------------------------------------------------- numerics
// Two E2M1 codes (one byte of `w`, selected by SEL) to two fp32 values; the
// hardware scale operand is 1, so the values are the exact E2M1 grid points.
// Element 2j sits in the low nibble and lands in .x.
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

// One E4M3FN byte of `w` (byte SEL) to fp32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Butterfly sum over the 64 lanes of a wave; every lane ends with the sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over aligned groups of 16 lanes.
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace moe
