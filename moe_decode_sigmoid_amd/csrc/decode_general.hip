// General-shape decode path (B <= 8 tokens): the same layer for the other MoE
// shapes the pages name and the MXFP8 expert format.
//
// The pages describe, besides Flint's 256 experts / top-6 / one shared expert
// ("Day-0 Support for Flint on vLLM", Model architecture section), the earlier
// Inkling with 256 experts, top-6 and two shared experts, and Inkling-2-Small
// with 384 experts, top-8 and none, whose last 8 layers hold their experts in
// MXFP8 (the AREX article on vLLM's Day-0 support for Inkling-2-Small,
// 48-layer MoE section).  The Flint layer runs on the single-launch kernel;
// every other shape within the limits below runs here, as four launches:
//
//   route    one wave per router row: logits [B][E] (fp32 accumulate); W4A4:
//            also the experts' quantised x
//   select   one workgroup: per token the top-k logits (ties to the lower
//            index), sigmoid, w = s / sum s; the touched experts become
//            entries in ascending id, then the shared experts (weight 1)
//   gate/up  workgroup (entry, 4 rows): per wave one gate/up row pair over
//            the tokens of the entry: h = SiLU(g) * u, bf16, to the workspace
//   down     per workgroup 64 / L output rows (L lanes per row), its waves
//            splitting the entries by expert id: the weighted sum over the
//            entries, rounded once to bf16
//
// Limits: H and I multiples of 32 (one 32-element chunk per lane step: 16
// code bytes + 2 E4M3 scales in NVFP4, 32 E4M3 bytes + 1 E8M0 scale in MXFP8,
// 64 bytes in BF16), H <= 8192, I <= 4096, top_k <= 8, n_experts <= 512,
// n_shared <= 2.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kGenThreads = 256;

// ------------------------------------------------------------------ weights
// One 32-element chunk of a weight row: dot(xw) is sum_k w_k v_k over the
// chunk before the tensor scale (v: 32 bf16 values as 16 pairs).
template <int FMT>
struct GChunk;

template <>
struct GChunk<FMT_NVFP4> {
  uint4 c;
  uint32_t s;
  // row of `cols` inputs starting at element row * cols of tensor (codes, scales)
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, size_t row,
                                       int cols, int ch) {
    c = *reinterpret_cast<const uint4*>(codes + row * (cols / 2) + 16 * ch);
    s = *reinterpret_cast<const uint16_t*>(scales + row * (cols / 16) + 2 * ch);
  }
  __device__ __forceinline__ float dot(const uint32_t (&xw)[16]) const {
    return nvfp4_dot32(c, s, xw);
  }
};

template <>
struct GChunk<FMT_BF16> {
  uint4 w[4];
  __device__ __forceinline__ void load(const uint8_t* el, const uint8_t*, size_t row, int cols,
                                       int ch) {
    const uint4* p = reinterpret_cast<const uint4*>(el + (row * cols + 32 * ch) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = p[i];
  }
  __device__ __forceinline__ float dot(const uint32_t (&xw)[16]) const {
    return bf16_dot32(w, xw);
  }
};

// MXFP8: 32 E4M3 bytes converted pairwise to exact bf16 with gfx950's
// scaled FP8 convert (scale 1), dot2 against x, then times the block's E8M0
// scale 2^(b - 127), built as an fp32 bit pattern (b = 0 is the subnormal
// 2^-127).
template <>
struct GChunk<FMT_MXFP8> {
  uint4 c[2];
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* el, const uint8_t* scales, size_t row,
                                       int cols, int ch) {
    const uint4* p = reinterpret_cast<const uint4*>(el + row * cols + 32 * ch);
    c[0] = p[0];
    c[1] = p[1];
    s = scales[row * (cols / 32) + ch];
  }
  __device__ __forceinline__ float dot(const uint32_t (&xw)[16]) const {
    const uint32_t w[8] = {c[0].x, c[0].y, c[0].z, c[0].w, c[1].x, c[1].y, c[1].z, c[1].w};
    float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], 1.0f, false);
      const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], 1.0f, true);
      if (d & 1) {
        b1 = dot2_bf16(lo, xw[2 * d], b1);
        b1 = dot2_bf16(hi, xw[2 * d + 1], b1);
      } else {
        b0 = dot2_bf16(lo, xw[2 * d], b0);
        b0 = dot2_bf16(hi, xw[2 * d + 1], b0);
      }
    }
    const float sc = __builtin_bit_cast(float, s == 0u ? 0x00400000u : s << 23);
    return (b0 + b1) * sc;
  }
};

// tensor scale of matrix m (0 gate, 1 up, 2 down) of expert ee
template <int FMT>
__device__ __forceinline__ float gen_gscale(const ExpertsDev& X, size_t ee, int m) {
  if constexpr (FMT == FMT_NVFP4) return X.glob[ee * 3 + m];
  return 1.0f;
}

// x chunk ch of token t (32 bf16 values as 16 pairs)
__device__ __forceinline__ void load_x32(const uint16_t* x, int H, int t, int ch,
                                         uint32_t (&xw)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)t * H + 32 * ch);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = p[i];
    xw[4 * i] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
  }
}

// ------------------------------------------------------------------ W4A4 quantiser
// Four Over Six NVFP4 quantisation of activations (the AREX article on vLLM's
// Day-0 support for Inkling-2-Small, 48-layer MoE section: per-token global
// scale, per-16-block scale mapping the block maximum to 6 or to 4, whichever
// reconstructs with the smaller mean absolute error; a tie keeps 6).  Every
// operation is an explicitly rounded fp32 one in a fixed order (global =
// amax / 2688; candidate scale E4M3(bmax / M / g), nearest-even, saturating
// at 448; q = e4m3 * g; code E2M1(v / q), nearest-even, saturating at 6; MAE
// summed in element order over |v - e2m1 * q|), so every workgroup, and any
// other implementation of these steps, takes the same decisions.

// max over each aligned group of 16 lanes (a DPP row)
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_f32<0x128>(v));
  v = fmaxf(v, dpp_f32<0x124>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0xB1>(v));
  return v;
}

// sum of the 16 values of a lane group in lane order (each lane gets it),
// through the wave's 64-float LDS area (a wave's LDS accesses are ordered)
__device__ __forceinline__ float group16_sum_in_order(float v, int lane, float* lds) {
  lds[lane] = v;
  const float4* p = reinterpret_cast<const float4*>(lds + (lane & ~15));
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = p[i];
    s = __fadd_rn(__fadd_rn(__fadd_rn(__fadd_rn(s, q.x), q.y), q.z), q.w);
  }
  return s;
}

// One 16-block held by a group of 16 lanes (lane l: element l & 15, value v),
// global g: this lane's quantised value e2m1 * e4m3 (the global apart; exact
// in bf16).  Both candidates are evaluated element-wise and their errors
// summed in element order.
__device__ __forceinline__ float a4_quant_elem(float v, float g, int lane, float* lds) {
  const float bmax = group16_max(fabsf(v));
  if (g == 0.0f || bmax == 0.0f) return 0.0f;
  const uint32_t s6 = a4_e4m3_rne(__fdiv_rn(__fdiv_rn(bmax, 6.0f), g));
  const uint32_t s4 = a4_e4m3_rne(__fdiv_rn(__fdiv_rn(bmax, 4.0f), g));
  const float v6 = a4_e4m3_value(s6), v4 = a4_e4m3_value(s4);
  const float q6 = __fmul_rn(v6, g), q4 = __fmul_rn(v4, g);
  const float r6 = a4_e2m1_rne(__fdiv_rn(v, q6 > 0.0f ? q6 : 1.0f));   // no branch around the
  const float r4 = a4_e2m1_rne(__fdiv_rn(v, q4 > 0.0f ? q4 : 1.0f));   // divisions
  const float c6 = q6 > 0.0f ? r6 : 0.0f, c4 = q4 > 0.0f ? r4 : 0.0f;
  const float m6 = group16_sum_in_order(fabsf(__fsub_rn(v, __fmul_rn(c6, q6))), lane, lds);
  const float m4 = group16_sum_in_order(fabsf(__fsub_rn(v, __fmul_rn(c4, q4))), lane, lds + 64);
  return m4 < m6 ? c4 * v4 : c6 * v6;
}

// Quantise n bf16 values (a multiple of 16) at src into dst (bf16 e2m1 *
// e4m3) with global g, by the threads [0, nthreads) of the caller, 16 per
// block; lds: 128 floats per wave of the caller.
__device__ __forceinline__ void a4_quant_vector(const uint16_t* src, uint16_t* dst, int n, float g,
                                                int tid, int nthreads, float* lds) {
  const int lane = tid & 63;
  float* wl = lds + 128 * (tid >> 6);
  for (int i0 = 0; i0 < n; i0 += nthreads) {          // uniform trip count per wave
    const int i = i0 + tid;
    const float v = i < n ? __builtin_bit_cast(float, (uint32_t)src[i] << 16) : 0.0f;
    const float q = a4_quant_elem(v, g, lane, wl);
    if (i < n) dst[i] = f32_to_bf16_rne(q);
  }
}

// ------------------------------------------------------------------ route
// One wave per router row e: logits[t][e] = sum_k W_r[e][k] x[t][k].  W4A4:
// workgroup t < B also quantises token t's x for the experts (the router
// itself reads x), after its router rows.
__global__ __launch_bounds__(kGenThreads) void k_gen_route(const uint16_t* __restrict__ x, int B,
                                                           const uint16_t* __restrict__ rw,
                                                           GenShape S, uint8_t* __restrict__ ws,
                                                           int a4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x * (kGenThreads / 64) + wave;
  const GenLayout L = gen_layout(S);
  if (e < S.E) {
    float* logits = reinterpret_cast<float*>(ws + L.logits);
    float acc[kMaxB];
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) acc[t] = 0.0f;
    const uint4* wrow = reinterpret_cast<const uint4*>(rw + (size_t)e * S.H);
    for (int c = lane; c < S.H / 8; c += 64) {
      const uint4 w = wrow[c];
#pragma unroll
      for (int t = 0; t < kMaxB; ++t) {
        if (t < B) {
          const uint4 v = reinterpret_cast<const uint4*>(x + (size_t)t * S.H)[c];
          float a = dot2_bf16(w.x, v.x, acc[t]);
          a = dot2_bf16(w.y, v.y, a);
          a = dot2_bf16(w.z, v.z, a);
          acc[t] = dot2_bf16(w.w, v.w, a);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) {
      if (t < B) {
        const float z = wave_sum(acc[t]);
        if (lane == 0) logits[t * S.E + e] = z;
      }
    }
  }
  if (!a4 || (int)blockIdx.x >= B) return;
  const int t = blockIdx.x;
  __shared__ float s_amax[4];
  float m = 0.0f;
  for (int i = tid; i < S.H / 8; i += kGenThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(x + (size_t)t * S.H)[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[k])), fabsf(bf16_hi(u[k]))));
  }
  m = wave_max(m);
  if (lane == 0) s_amax[wave] = m;
  __syncthreads();
  const float g =
      __fdiv_rn(fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3])), 2688.0f);
  if (tid == 0) reinterpret_cast<float*>(ws + L.gx)[t] = g;
  __shared__ float s_q[kGenThreads / 64 * 128];
  a4_quant_vector(x + (size_t)t * S.H, reinterpret_cast<uint16_t*>(ws + L.xq) + (size_t)t * S.H,
                  S.H, g, tid, kGenThreads, s_q);
}

// ------------------------------------------------------------------ select
// Top-k of E <= 512 logits held 8 per lane (expert lane + 64 q in v[q]) under
// (value descending, index ascending): each round takes the wave maximum and
// the lowest index holding it.
__device__ __forceinline__ void wave_topk512(float (&v)[8], int lane, int K,
                                             int (&ids)[kGenMaxK], float (&vals)[kGenMaxK]) {
#pragma unroll
  for (int j = 0; j < kGenMaxK; ++j) {
    if (j >= K) break;
    float lm = v[0];
#pragma unroll
    for (int q = 1; q < 8; ++q) lm = fmaxf(lm, v[q]);
    const float m = wave_max(lm);
    int idx = -1;
#pragma unroll
    for (int q = 7; q >= 0; --q) {
      const uint64_t bal = __ballot(v[q] == m);
      if (bal) idx = 64 * q + __builtin_ctzll(bal);
    }
    if (idx < 0) idx = j;   // only when every value is NaN (outside the contract)
    ids[j] = idx;
    vals[j] = m;
    if ((idx & 63) == lane) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if ((idx >> 6) == q) v[q] = -INFINITY;
    }
  }
}

__global__ __launch_bounds__(kGenThreads) void k_gen_select(int B, GenShape S,
                                                            int32_t* __restrict__ ids_out,
                                                            float* __restrict__ w_out,
                                                            uint8_t* __restrict__ ws) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const GenLayout L = gen_layout(S);
  const float* logits = reinterpret_cast<const float*>(ws + L.logits);
  GenCtl* ctl = reinterpret_cast<GenCtl*>(ws + L.ctl);
  __shared__ int s_ids[kMaxB][kGenMaxK];
  __shared__ float s_w[kMaxB][kGenMaxK];
  __shared__ unsigned s_mask[kGenMaxE];
  __shared__ float s_wt[kGenMaxE][kMaxB];
  for (int t = wave; t < B; t += 4) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < S.E ? logits[t * S.E + e] : -INFINITY;
    }
    int sel_i[kGenMaxK];
    float sel_l[kGenMaxK];
    wave_topk512(v, lane, S.K, sel_i, sel_l);
    if (lane == 0) {
      float s[kGenMaxK], sum = 0.0f;
#pragma unroll
      for (int j = 0; j < kGenMaxK; ++j) {
        s[j] = j < S.K ? 1.0f / (1.0f + expf(-sel_l[j])) : 0.0f;
        sum += s[j];
      }
#pragma unroll
      for (int j = 0; j < kGenMaxK; ++j) {
        if (j < S.K) {
          s_ids[t][j] = sel_i[j];
          s_w[t][j] = s[j] / sum;
        }
      }
    }
  }
  for (int e = tid; e < S.E; e += kGenThreads) {
    s_mask[e] = 0u;
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) s_wt[e][t] = 0.0f;
  }
  __syncthreads();
  if (tid < B * S.K) {
    const int t = tid / S.K, j = tid % S.K;
    const int e = s_ids[t][j];
    atomicOr(&s_mask[e], 1u << t);
    s_wt[e][t] = s_w[t][j];
    if (ids_out) ids_out[t * S.K + j] = e;
    if (w_out) w_out[t * S.K + j] = s_w[t][j];
  }
  __syncthreads();
  if (wave == 0) {   // the touched experts in ascending id, then the shared ones
    int base = 0;
    for (int q = 0; q < kGenMaxE / 64; ++q) {
      const int e = 64 * q + lane;
      const unsigned m = e < S.E ? s_mask[e] : 0u;
      const uint64_t bal = __ballot(m != 0u);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (m != 0u) {
        ctl->entry[pos] = e;
        ctl->amask[pos] = m;
#pragma unroll
        for (int t = 0; t < kMaxB; ++t) ctl->wt[pos][t] = s_wt[e][t];
      }
      base += __popcll(bal);
    }
    if (lane < S.NS) {
      ctl->entry[base + lane] = S.E + lane;
      ctl->amask[base + lane] = (1u << B) - 1u;
#pragma unroll
      for (int t = 0; t < kMaxB; ++t) ctl->wt[base + lane][t] = t < B ? 1.0f : 0.0f;
    }
    if (lane == 0) ctl->n_entries = base + S.NS;
  }
}

// W4A4: h of each (entry, token) pair quantised like x (its own global from
// the pair's maximum over I), one workgroup per pair.  The pages quantise inside
// the SiLU kernel; here a pair's h is spread over several workgroups of the
// gate/up launch, so its maximum needs this separate pass.
__global__ __launch_bounds__(kGenThreads) void k_gen_quant_h(GenShape S, uint8_t* __restrict__ ws) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, a = blockIdx.x, t = blockIdx.y;
  const GenLayout L = gen_layout(S);
  const GenCtl* ctl = reinterpret_cast<const GenCtl*>(ws + L.ctl);
  if (a >= ctl->n_entries || !((ctl->amask[a] >> t) & 1u)) return;
  const uint16_t* h = reinterpret_cast<const uint16_t*>(ws + L.h) + ((size_t)a * kMaxB + t) * S.I;
  uint16_t* hq = reinterpret_cast<uint16_t*>(ws + L.hq) + ((size_t)a * kMaxB + t) * S.I;
  __shared__ float s_amax[kGenThreads / 64];
  __shared__ float s_q[kGenThreads / 64 * 128];
  float m = 0.0f;
  for (int i = tid; i < S.I / 8; i += kGenThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(h)[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[k])), fabsf(bf16_hi(u[k]))));
  }
  m = wave_max(m);
  if (lane == 0) s_amax[wave] = m;
  __syncthreads();
  const float g =
      __fdiv_rn(fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3])), 2688.0f);
  if (tid == 0) reinterpret_cast<float*>(ws + L.gh)[(size_t)a * kMaxB + t] = g;
  a4_quant_vector(h, hq, S.I, g, tid, kGenThreads, s_q);
}

// ------------------------------------------------------------------ gate/up
// Workgroup (entry a, rows 4 blockIdx.y + wave): h[a][t][r] = SiLU(g) * u for
// the entry's tokens, bf16.
template <int FMT, bool A4>
__global__ __launch_bounds__(kGenThreads) void k_gen_gateup(const uint16_t* __restrict__ x, int B,
                                                            GenShape S, ExpertsDev routed,
                                                            ExpertsDev shared,
                                                            uint8_t* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int a = blockIdx.x;
  const int r = blockIdx.y * (kGenThreads / 64) + (threadIdx.x >> 6);
  const GenLayout L = gen_layout(S);
  const GenCtl* ctl = reinterpret_cast<const GenCtl*>(ws + L.ctl);
  if (a >= ctl->n_entries || r >= S.I) return;
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + L.h);
  if constexpr (A4) x = reinterpret_cast<const uint16_t*>(ws + L.xq);   // e2m1 * e4m3, x global apart
  const int e = ctl->entry[a];
  const unsigned mask = ctl->amask[a];
  const bool sh = e >= S.E;
  const ExpertsDev& X = sh ? shared : routed;
  const size_t ee = sh ? (size_t)(e - S.E) : (size_t)e;
  const size_t rg = (ee * 2 + 0) * S.I + r, ru = (ee * 2 + 1) * S.I + r;
  float ag[kMaxB], au[kMaxB];
#pragma unroll
  for (int t = 0; t < kMaxB; ++t) ag[t] = au[t] = 0.0f;
  for (int ch = lane; ch < S.H / 32; ch += 64) {
    GChunk<FMT> cg, cu;
    cg.load(X.w13, X.w13s, rg, S.H, ch);
    cu.load(X.w13, X.w13s, ru, S.H, ch);
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) {
      if ((mask >> t) & 1u) {
        uint32_t xw[16];
        load_x32(x, S.H, t, ch, xw);
        ag[t] += cg.dot(xw);
        au[t] += cu.dot(xw);
      }
    }
  }
  const float sg = gen_gscale<FMT>(X, ee, 0), su = gen_gscale<FMT>(X, ee, 1);
#pragma unroll
  for (int t = 0; t < kMaxB; ++t) {
    if ((mask >> t) & 1u) {
      const float gxt = A4 ? reinterpret_cast<const float*>(ws + L.gx)[t] : 1.0f;
      const float g = wave_sum(ag[t]) * sg * gxt, u = wave_sum(au[t]) * su * gxt;
      if (lane == 0) hbuf[((size_t)a * kMaxB + t) * S.I + r] = f32_to_bf16_rne(silu_mul(g, u));
    }
  }
}

// ------------------------------------------------------------------ down + combine
// A workgroup covers 64 / LPR output rows (LPR lanes per row; LPR = 16, 32 or
// 64 by the chunk count of I).  Its 4 waves split the entries by expert id
// (wave w: routed experts in [w E / 4, (w + 1) E / 4), the shared experts in
// wave 3), each walking its entries in order, and the 4 partial sums are added
// in wave order: a token's sum depends only on its own experts, never on the
// rest of the batch.
template <int FMT, int LPR, bool A4>
__global__ __launch_bounds__(kGenThreads) void k_gen_down(int B, GenShape S, ExpertsDev routed,
                                                          ExpertsDev shared,
                                                          uint8_t* __restrict__ ws,
                                                          uint16_t* __restrict__ out) {
  constexpr int kRows = 64 / LPR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, sub = lane % LPR;
  const int q = lane / LPR;
  const int j = blockIdx.x * kRows + q;
  const GenLayout L = gen_layout(S);
  const GenCtl* ctl = reinterpret_cast<const GenCtl*>(ws + L.ctl);
  const uint16_t* hbuf = reinterpret_cast<const uint16_t*>(ws + (A4 ? L.hq : L.h));
  __shared__ float s_red[4][kRows][kMaxB];
  const bool live = j < S.H;
  const int na = ctl->n_entries;
  const int e_lo = (wave * S.E) / 4, e_hi = wave == 3 ? S.E + S.NS : ((wave + 1) * S.E) / 4;
  float acc[kMaxB];
#pragma unroll
  for (int t = 0; t < kMaxB; ++t) acc[t] = 0.0f;
  for (int a = 0; a < na; ++a) {
    const int e = ctl->entry[a];
    if (e < e_lo || e >= e_hi) continue;
    const unsigned mask = ctl->amask[a];
    const bool sh = e >= S.E;
    const ExpertsDev& X = sh ? shared : routed;
    const size_t ee = sh ? (size_t)(e - S.E) : (size_t)e;
    float part[kMaxB];
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) part[t] = 0.0f;
    if (live) {
      for (int ch = sub; ch < S.I / 32; ch += LPR) {
        GChunk<FMT> cd;
        cd.load(X.w2, X.w2s, ee * S.H + j, S.I, ch);
#pragma unroll
        for (int t = 0; t < kMaxB; ++t) {
          if ((mask >> t) & 1u) {
            uint32_t hw[16];
            const uint4* p = reinterpret_cast<const uint4*>(hbuf + ((size_t)a * kMaxB + t) * S.I +
                                                            32 * ch);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 v = p[i];
              hw[4 * i] = v.x; hw[4 * i + 1] = v.y; hw[4 * i + 2] = v.z; hw[4 * i + 3] = v.w;
            }
            part[t] += cd.dot(hw);
          }
        }
      }
    }
    const float sd = live ? gen_gscale<FMT>(X, ee, 2) : 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) {
      if ((mask >> t) & 1u) {
        float z = part[t];
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) z += __shfl_xor(z, o, 64);
        if constexpr (A4) z *= reinterpret_cast<const float*>(ws + L.gh)[(size_t)a * kMaxB + t];
        acc[t] += ctl->wt[a][t] * (z * sd);
      }
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) s_red[wave][q][t] = acc[t];
  }
  __syncthreads();
  if (tid < kRows * kMaxB) {
    const int rq = tid / kMaxB, t = tid % kMaxB, jj = blockIdx.x * kRows + rq;
    if (jj < S.H && t < B) {
      const float y = ((s_red[0][rq][t] + s_red[1][rq][t]) + s_red[2][rq][t]) + s_red[3][rq][t];
      out[(size_t)t * S.H + jj] = f32_to_bf16_rne(y);
    }
  }
}

// ------------------------------------------------------------------ launchers
size_t gen_ws_bytes(const GenShape& S) { return gen_layout(S).total; }

hipError_t launch_route_general(int B, const GenShape& S, const uint16_t* x, const uint16_t* rw,
                                int32_t* ids, float* w, uint8_t* ws, hipStream_t st, int a4) {
  const int nwg = (S.E + 3) / 4;
  hipLaunchKernelGGL(k_gen_route, dim3(a4 && nwg < B ? B : nwg), dim3(kGenThreads), 0, st, x, B, rw,
                     S, ws, a4);
  hipLaunchKernelGGL(k_gen_select, dim3(1), dim3(kGenThreads), 0, st, B, S, ids, w, ws);
  return hipGetLastError();
}

template <int FMT, bool A4 = false>
static void launch_experts_general(int B, const GenShape& S, const uint16_t* x,
                                   const ExpertsDev& routed, const ExpertsDev& shared,
                                   uint16_t* out, uint8_t* ws, hipStream_t st) {
  const int maxa = gen_max_entries(S, B);
  hipLaunchKernelGGL((k_gen_gateup<FMT, A4>), dim3(maxa, (S.I + 3) / 4), dim3(kGenThreads), 0, st,
                     x, B, S, routed, shared, ws);
  if constexpr (A4)
    hipLaunchKernelGGL(k_gen_quant_h, dim3(maxa, B), dim3(kGenThreads), 0, st, S, ws);
  const int nch = S.I / 32;
  if (nch <= 16)
    hipLaunchKernelGGL((k_gen_down<FMT, 16, A4>), dim3((S.H + 3) / 4), dim3(kGenThreads), 0, st, B,
                       S, routed, shared, ws, out);
  else if (nch <= 32)
    hipLaunchKernelGGL((k_gen_down<FMT, 32, A4>), dim3((S.H + 1) / 2), dim3(kGenThreads), 0, st, B,
                       S, routed, shared, ws, out);
  else
    hipLaunchKernelGGL((k_gen_down<FMT, 64, A4>), dim3(S.H), dim3(kGenThreads), 0, st, B, S,
                       routed, shared, ws, out);
}

hipError_t launch_decode_general(int B, int fmt, const GenShape& S, const uint16_t* x,
                                 const uint16_t* rw, const ExpertsDev& routed,
                                 const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                                 uint8_t* ws, hipStream_t st) {
  hipError_t e = launch_route_general(B, S, x, rw, ids, w, ws, st, fmt == FMT_NVFP4_A4);
  if (e != hipSuccess) return e;
  if (fmt == FMT_NVFP4_A4)
    launch_experts_general<FMT_NVFP4, true>(B, S, x, routed, shared, out, ws, st);
  else if (fmt == FMT_NVFP4)
    launch_experts_general<FMT_NVFP4>(B, S, x, routed, shared, out, ws, st);
  else if (fmt == FMT_BF16)
    launch_experts_general<FMT_BF16>(B, S, x, routed, shared, out, ws, st);
  else
    launch_experts_general<FMT_MXFP8>(B, S, x, routed, shared, out, ws, st);
  return hipGetLastError();
}

}  // namespace moe
