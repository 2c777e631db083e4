// Small-batch dense GEMV on packed NVFP4 weights (B <= 8 tokens), the kernel
// the pages list for the non-expert projections and the dense MLP of the
// first two layers ("Day-0 Support for Flint on vLLM", Optimization section,
// Fig. 2 change list; Model architecture section for the dense layers):
//
//   y[t][n] = global * sum_k e2m1(code[n][k]) * e4m3(scale[n][k / 16]) * x[t][k]
//
// fp32 accumulation, y rounded once to bf16.  A workgroup of 256 threads
// computes 16 output rows, 4 per wave.  x (bf16 [B][K]) is staged in LDS.
// Lane l of a wave covers the 32-element chunks c = l, l + 64, ... of K
// (16 code bytes + 2 scale bytes per row), loads all chunks of its 4 rows at
// once, decodes them with gfx950's FP4 -> bf16 converts and dot2 products
// against x, and keeps per-lane partial sums; the (row, token) sums are
// reduced over the 64 lanes 8 at a time with the half swaps and DPP steps of
// the decode kernel's gate/up batches.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kGvThreads = 256;
constexpr int kGvRows = 16;                 // output rows per workgroup (4 per wave)

__device__ __forceinline__ void gv_swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ void gv_swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Wave totals of 8 per-lane values: value j ends in lanes 8 j .. 8 j + 7.
__device__ __forceinline__ float gv_sum8(const float (&v)[8], int lane) {
  float w[4], u[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = v[j], b = v[4 + j];
    gv_swap32(a, b);
    w[j] = a + b;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float a = w[j], b = w[2 + j];
    gv_swap16(a, b);
    u[j] = a + b;
  }
  const bool hi = (lane & 8) != 0;
  float z = (hi ? u[1] : u[0]) + dpp_f32<0x128>(hi ? u[0] : u[1]);
  z += dpp_f32<0x141>(z);
  z += dpp_f32<0x4E>(z);
  z += dpp_f32<0xB1>(z);
  return z;
}

// sum over one 32-element chunk of w * x (x as 16 packed bf16 pairs), before
// the tensor scale: two 16-element blocks, each times its E4M3 scale
__device__ __forceinline__ float gv_dot(uint4 c, uint32_t s, const uint32_t (&xw)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    b0 = dot2_bf16(fp4x2_to_bf16<0>(w[d]), xw[4 * d + 0], b0);
    b0 = dot2_bf16(fp4x2_to_bf16<1>(w[d]), xw[4 * d + 1], b0);
    b0 = dot2_bf16(fp4x2_to_bf16<2>(w[d]), xw[4 * d + 2], b0);
    b0 = dot2_bf16(fp4x2_to_bf16<3>(w[d]), xw[4 * d + 3], b0);
  }
#pragma unroll
  for (int d = 2; d < 4; ++d) {
    b1 = dot2_bf16(fp4x2_to_bf16<0>(w[d]), xw[4 * d + 0], b1);
    b1 = dot2_bf16(fp4x2_to_bf16<1>(w[d]), xw[4 * d + 1], b1);
    b1 = dot2_bf16(fp4x2_to_bf16<2>(w[d]), xw[4 * d + 2], b1);
    b1 = dot2_bf16(fp4x2_to_bf16<3>(w[d]), xw[4 * d + 3], b1);
  }
  return b0 * e4m3_to_f32<0>(s) + b1 * e4m3_to_f32<1>(s);
}

// NC = chunk passes per lane (K / 32 chunks over 64 lanes, rounded up)
template <int B, int NC>
__global__ __launch_bounds__(kGvThreads) void k_nvfp4_gemv(const uint16_t* __restrict__ x, int K,
                                                         int N, const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ glob,
                                                         uint16_t* __restrict__ y) {
  extern __shared__ uint4 s_x[];                     // bf16 [B][K]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / 32;
  const int r0 = blockIdx.x * kGvRows + 4 * wave;
  // this wave's rows: every chunk of every row goes out before any is used
  uint4 c[4][NC];
  uint32_t s[4][NC];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int ch = lane + 64 * i, r = r0 + q;
      c[q][i] = make_uint4(0u, 0u, 0u, 0u);
      s[q][i] = 0u;
      if (r < N && ch < nch) {
        c[q][i] = *reinterpret_cast<const uint4*>(codes + (size_t)r * (K / 2) + 16 * ch);
        s[q][i] = *reinterpret_cast<const uint16_t*>(scales + (size_t)r * (K / 16) + 2 * ch);
      }
    }
  for (int i = tid; i < B * K / 8; i += kGvThreads) s_x[i] = reinterpret_cast<const uint4*>(x)[i];
  __syncthreads();
  float acc[4][B];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int t = 0; t < B; ++t) acc[q][t] = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
#pragma unroll
      for (int t = 0; t < B; ++t) {
        uint32_t xw[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = s_x[(t * K + 32 * ch) / 8 + j];
          xw[4 * j] = v.x; xw[4 * j + 1] = v.y; xw[4 * j + 2] = v.z; xw[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q][t] += gv_dot(c[q][i], s[q][i], xw);
      }
    }
  }
  // (row q, token t) pairs, 8 per reduction; pair j of a round lands in lanes 8 j ..
  const float gl = glob[0];
  constexpr int kPairs = 4 * B;
#pragma unroll
  for (int p0 = 0; p0 < kPairs; p0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pj = p0 + j;
      v[j] = pj < kPairs ? acc[pj % 4][pj / 4 < B ? pj / 4 : 0] : 0.0f;
    }
    const float z = gv_sum8(v, lane);
    const int pj = p0 + (lane >> 3), q = pj % 4, t = pj / 4;
    if ((lane & 7) == 0 && pj < kPairs && r0 + q < N)
      y[(size_t)t * N + r0 + q] = f32_to_bf16_rne(z * gl);
  }
}

template <int B>
static hipError_t launch_gemv_b(const uint16_t* x, int K, int N, const uint8_t* codes,
                                const uint8_t* scales, const float* glob, uint16_t* y,
                                hipStream_t st) {
  const dim3 grid((N + kGvRows - 1) / kGvRows), block(kGvThreads);
  const size_t lds = (size_t)B * K * 2;
  const int passes = (K / 32 + 63) / 64;
  if (passes == 1)
    hipLaunchKernelGGL((k_nvfp4_gemv<B, 1>), grid, block, lds, st, x, K, N, codes, scales, glob, y);
  else if (passes == 2)
    hipLaunchKernelGGL((k_nvfp4_gemv<B, 2>), grid, block, lds, st, x, K, N, codes, scales, glob, y);
  else
    hipLaunchKernelGGL((k_nvfp4_gemv<B, 4>), grid, block, lds, st, x, K, N, codes, scales, glob, y);
  return hipGetLastError();
}

hipError_t launch_nvfp4_gemv(int B, int K, int N, const uint16_t* x, const uint8_t* codes,
                             const uint8_t* scales, const float* glob, uint16_t* y,
                             hipStream_t st) {
  switch (B) {
    case 1: return launch_gemv_b<1>(x, K, N, codes, scales, glob, y, st);
    case 2: return launch_gemv_b<2>(x, K, N, codes, scales, glob, y, st);
    case 3: return launch_gemv_b<3>(x, K, N, codes, scales, glob, y, st);
    case 4: return launch_gemv_b<4>(x, K, N, codes, scales, glob, y, st);
    case 5: return launch_gemv_b<5>(x, K, N, codes, scales, glob, y, st);
    case 6: return launch_gemv_b<6>(x, K, N, codes, scales, glob, y, st);
    case 7: return launch_gemv_b<7>(x, K, N, codes, scales, glob, y, st);
    case 8: return launch_gemv_b<8>(x, K, N, codes, scales, glob, y, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
