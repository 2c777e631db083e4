// Small-batch dense GEMV on packed NVFP4 weights (B <= 8 tokens), the kernel
// the pages list for the non-expert projections and the dense MLP of the
// first two layers ("Day-0 Support for Flint on vLLM", Optimization section,
// Fig. 2 change list; Model architecture section for the dense layers):
//
//   y[t][n] = global * sum_k e2m1(code[n][k]) * e4m3(scale[n][k / 16]) * x[t][k]
//
// fp32 accumulation, y rounded once to bf16.  A workgroup of 256 threads
// computes 4 RW output rows, RW (4 or 2) per wave.  x (bf16 [B][K]) is staged
// in LDS.  Lane l of a wave covers the 32-element chunks c = l, l + 64, ... of
// K (16 code bytes + 2 scale bytes per row), loads all chunks of its rows at
// once, decodes them with gfx950's FP4 -> bf16 converts and dot2 products
// against x, and keeps per-lane partial sums; the (row, token) sums are
// reduced over the 64 lanes 8 at a time with the half swaps and DPP steps of
// the decode kernel's gate/up batches.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kGvThreads = 256;



// NC = chunk passes per lane (K / 32 chunks over 64 lanes, rounded up);
// RW = output rows per wave (4 waves per workgroup)
template <int B, int NC, int RW>
__global__ __launch_bounds__(kGvThreads) void k_nvfp4_gemv(const uint16_t* __restrict__ x, int K,
                                                         int N, const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ glob,
                                                         uint16_t* __restrict__ y) {
  extern __shared__ uint4 s_x[];                     // bf16 [B][K]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / 32;
  const int r0 = (blockIdx.x * 4 + wave) * RW;
  // x (B K / 8 16-byte pieces, at most B NC per thread) goes out first, then
  // every chunk of this wave's rows: loads return in issue order, so x can be
  // written to LDS as soon as it is in, while the weights are still on the way
  constexpr int XN = B * NC < 16 ? B * NC : 16;
  const int nx = B * K / 8;
  uint4 xr[XN];
#pragma unroll
  for (int j = 0; j < XN; ++j) {
    const int i = tid + kGvThreads * j;
    xr[j] = i < nx ? reinterpret_cast<const uint4*>(x)[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint4 c[RW][NC];
  uint32_t s[RW][NC];
#pragma unroll
  for (int q = 0; q < RW; ++q)
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
#pragma unroll
  for (int j = 0; j < XN; ++j) {
    const int i = tid + kGvThreads * j;
    if (i < nx) s_x[i] = xr[j];
  }
  __syncthreads();
  float acc[RW][B];
#pragma unroll
  for (int q = 0; q < RW; ++q)
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
        for (int q = 0; q < RW; ++q) acc[q][t] += nvfp4_dot32(c[q][i], s[q][i], xw);
      }
    }
  }
  // (row q, token t) pairs, 8 per reduction; pair j of a round lands in lanes 8 j ..
  const float gl = glob[0];
  constexpr int kPairs = RW * B;
#pragma unroll
  for (int p0 = 0; p0 < kPairs; p0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pj = p0 + j;
      v[j] = pj < kPairs ? acc[pj % RW][pj / RW < B ? pj / RW : 0] : 0.0f;
    }
    const float z = wave_sum8(v, lane);
    const int pj = p0 + (lane >> 3), q = pj % RW, t = pj / RW;
    if ((lane & 7) == 0 && pj < kPairs && r0 + q < N)
      y[(size_t)t * N + r0 + q] = f32_to_bf16_rne(z * gl);
  }
}

// 4 rows per wave unless that leaves fewer than kGvSplitBelow workgroups (2 per
// CU): measured on the two attention projections of the Flint shape, which
// both take 2 rows per wave, 2 rows are 4-27% faster
constexpr int kGvSplitBelow = 512;

template <int B, int NC>
static void launch_gemv_nc(int K, int N, const uint16_t* x, const uint8_t* codes,
                           const uint8_t* scales, const float* glob, uint16_t* y, hipStream_t st) {
  const size_t lds = (size_t)B * K * 2;
  const dim3 block(kGvThreads);
  if ((N + 15) / 16 >= kGvSplitBelow)
    hipLaunchKernelGGL((k_nvfp4_gemv<B, NC, 4>), dim3((N + 15) / 16), block, lds, st, x, K, N,
                       codes, scales, glob, y);
  else
    hipLaunchKernelGGL((k_nvfp4_gemv<B, NC, 2>), dim3((N + 7) / 8), block, lds, st, x, K, N,
                       codes, scales, glob, y);
}

template <int B>
static hipError_t launch_gemv_b(const uint16_t* x, int K, int N, const uint8_t* codes,
                                const uint8_t* scales, const float* glob, uint16_t* y,
                                hipStream_t st) {
  const int passes = (K / 32 + 63) / 64;
  if (passes == 1)
    launch_gemv_nc<B, 1>(K, N, x, codes, scales, glob, y, st);
  else if (passes == 2)
    launch_gemv_nc<B, 2>(K, N, x, codes, scales, glob, y, st);
  else
    launch_gemv_nc<B, 4>(K, N, x, codes, scales, glob, y, st);
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
