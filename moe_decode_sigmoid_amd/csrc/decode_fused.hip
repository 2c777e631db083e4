// Fused low-latency decode kernel (B <= 8 tokens) of the Flint-style MoE layer
// on gfx950: the whole layer in ONE launch.
//
// The pages describe a low-latency path for up to 8 requests in which routing
// and the expert combine are fused into the neighbouring GEMV kernels and each
// kernel starts loading its weights while the previous one still runs
// ("Day-0 Support for Flint on vLLM", Optimization section and Fig. 3).
// MI355X has no programmatic dependent launch, so the dependent steps live
// inside one kernel of 256 workgroups (one per CU, all resident) that hand
// data to each other through the workspace, and every workgroup issues the
// weight loads of a later step as soon as it knows their addresses:
//
//   A  router GEMV, one expert row per workgroup (the 4 waves split the 2048
//      columns) -> logit slots; the shared expert's gate/up rows 2g, 2g+1
//      (routing-independent) -> h.
//   B  every workgroup waits for the 256 x B logits and repeats the sigmoid /
//      top-6 / renormalisation / dispatch itself (identical result everywhere,
//      no extra round trip); it fetches the first down rows of its step-C
//      work; the routed experts' gate/up row pairs, cut into 256 contiguous
//      ranges, SiLU(g) * u -> h; then it counts in on an h-ready counter.
//   C  once all h is in: the down GEMV of the workgroup's 8 output rows over
//      every entry (shared + routed), weighted by the routing, summed in a
//      fixed order, rounded once to bf16.
//
// Hand-over between workgroups uses only device-coherent accesses (relaxed
// agent-scope atomics: no cache write-back or invalidation):
//  - call epoch: workgroup g keeps a private counter in the workspace; every
//    call adds one, so all counters agree (the workspace starts zeroed).
//  - logits: 8-byte slots {fp32 value, epoch}, one store each; readers poll
//    the slots until their epoch matches.
//  - h: plain coherent stores; after waiting for its stores a workgroup adds
//    1 to h-ready counter g % 64 (one 128-byte line each, so only 4 adds meet
//    on a line); readers poll the 64 counters until each holds 4 * epoch.
// Every wait is bounded (tens of ms); on time-out the workgroup sets the
// workspace error word and carries on, so the kernel always terminates.
// Results are reproducible bit for bit (fixed summation orders, no atomics
// on data).
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kFusedGrid = 256;             // workgroups (one per CU)
constexpr int kFusedThreads = 256;          // 4 waves, 16 groups of 16 lanes
constexpr int kRowsPerWg = kH / kFusedGrid; // 8 output rows per workgroup
constexpr int kUnitRows = 4;                // rows per down work unit (half a tile)
constexpr int kHBanks = 64;                 // h-ready counters, one 128-byte line each
constexpr int kSpinLimit = 1 << 18;

// ------------------------------------------------------------------ row chunks
// A lane's 32 consecutive elements of one weight row.
template <int FMT>
struct Chunk;

template <>
struct Chunk<FMT_NVFP4> {
  uint4 c;
  uint32_t s;
  __device__ __forceinline__ void load_gu(const ExpertsDev& X, size_t ee, int m, int row, int ch) {
    const size_t r = (ee * 2 + m) * kI + row;
    c = *reinterpret_cast<const uint4*>(X.w13 + r * (kH / 2) + 16 * ch);
    s = *reinterpret_cast<const uint16_t*>(X.w13s + r * (kH / 16) + 2 * ch);
  }
  __device__ __forceinline__ void load_dn(const ExpertsDev& X, size_t ee, int row, int ch) {
    const size_t r = ee * kH + row;
    c = *reinterpret_cast<const uint4*>(X.w2 + r * (kI / 2) + 16 * ch);
    s = *reinterpret_cast<const uint16_t*>(X.w2s + r * (kI / 16) + 2 * ch);
  }
  // sum_k w_k x_k over the chunk, without the tensor scale
  __device__ __forceinline__ float dot_x(const uint32_t (&xw)[16]) const {
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
  __device__ __forceinline__ float dot_h(const float (&h)[32]) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float b[2] = {0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f32x2 p;
      float& acc = b[d >> 1];
      p = fp4x2_to_f32<0>(w[d]); acc += p.x * h[8 * d + 0]; acc += p.y * h[8 * d + 1];
      p = fp4x2_to_f32<1>(w[d]); acc += p.x * h[8 * d + 2]; acc += p.y * h[8 * d + 3];
      p = fp4x2_to_f32<2>(w[d]); acc += p.x * h[8 * d + 4]; acc += p.y * h[8 * d + 5];
      p = fp4x2_to_f32<3>(w[d]); acc += p.x * h[8 * d + 6]; acc += p.y * h[8 * d + 7];
    }
    return b[0] * e4m3_to_f32<0>(s) + b[1] * e4m3_to_f32<1>(s);
  }
  __device__ __forceinline__ static float gscale(const ExpertsDev& X, size_t ee, int m) {
    return X.glob[ee * 3 + m];
  }
};

template <>
struct Chunk<FMT_BF16> {
  uint4 w[4];
  __device__ __forceinline__ void load_gu(const ExpertsDev& X, size_t ee, int m, int row, int ch) {
    const uint4* p = reinterpret_cast<const uint4*>(X.w13 + (((ee * 2 + m) * kI + row) * kH + 32 * ch) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = p[i];
  }
  __device__ __forceinline__ void load_dn(const ExpertsDev& X, size_t ee, int row, int ch) {
    const uint4* p = reinterpret_cast<const uint4*>(X.w2 + ((ee * kH + row) * kI + 32 * ch) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = p[i];
  }
  __device__ __forceinline__ float dot_x(const uint32_t (&xw)[16]) const {
    float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      b0 = dot2_bf16(w[i].x, xw[4 * i + 0], b0);
      b0 = dot2_bf16(w[i].y, xw[4 * i + 1], b0);
      b0 = dot2_bf16(w[i].z, xw[4 * i + 2], b0);
      b0 = dot2_bf16(w[i].w, xw[4 * i + 3], b0);
    }
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      b1 = dot2_bf16(w[i].x, xw[4 * i + 0], b1);
      b1 = dot2_bf16(w[i].y, xw[4 * i + 1], b1);
      b1 = dot2_bf16(w[i].z, xw[4 * i + 2], b1);
      b1 = dot2_bf16(w[i].w, xw[4 * i + 3], b1);
    }
    return b0 + b1;
  }
  __device__ __forceinline__ float dot_h(const float (&h)[32]) const {
    float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
      float& acc = i < 2 ? b0 : b1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc += bf16_lo(v[k]) * h[8 * i + 2 * k];
        acc += bf16_hi(v[k]) * h[8 * i + 2 * k + 1];
      }
    }
    return b0 + b1;
  }
  __device__ __forceinline__ static float gscale(const ExpertsDev&, size_t, int) { return 1.0f; }
};

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ void trace_stamp(uint8_t* ws, int k) {
#ifdef MOE_PHASE_TRACE
  if (threadIdx.x == 0)
    reinterpret_cast<unsigned long long*>(ws + kTraceOff)[blockIdx.x * 8 + k] =
        __builtin_amdgcn_s_memrealtime();
#else
  (void)ws;
  (void)k;
#endif
}

__device__ __forceinline__ void put_slot(uint64_t* p, float v, uint32_t epoch) {
  const uint64_t w = (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)epoch << 32);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_slot(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_flag(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_flag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-workgroup words in the workspace, one 128-byte line each:
// kind 0 = epoch counter, 1 = step A done, 2 = h rows done, 3 = partials done.
__device__ __forceinline__ uint32_t* flag_ptr(uint8_t* ws, int kind, int wg) {
  return reinterpret_cast<uint32_t*>(ws + kFlagOff + ((size_t)kind * kFusedGrid + wg) * kFlagStride);
}

// Reads N slots per lane (p[k * stride], k < N) into out[], polling until all
// of the active lanes' slots carry `epoch`.  Bounded.
template <int N>
__device__ __forceinline__ void wait_slots(const uint64_t* p, int stride, uint32_t epoch,
                                           float (&out)[N], unsigned* err) {
  uint32_t pending = (1u << N) - 1u;
  for (int spin = 0;; ++spin) {
    uint64_t w[N];
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (pending & (1u << k)) w[k] = get_slot(p + k * stride);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if ((pending & (1u << k)) && (uint32_t)(w[k] >> 32) == epoch) {
        out[k] = __builtin_bit_cast(float, (uint32_t)w[k]);
        pending &= ~(1u << k);
      }
    }
    if (__ballot(pending != 0u) == 0) break;
    if (spin > kSpinLimit) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// One gate/up row pair of expert `ee` for the tokens in `mask`; the wave's
// lanes cover the 2048 columns, lane 0 writes h = SiLU(g) * u.
template <int B, int FMT>
__device__ __forceinline__ void gateup_compute(const Chunk<FMT>& cg, const Chunk<FMT>& cu, float sg,
                                               float su, unsigned mask, const uint4* s_x,
                                               const uint32_t (&x0)[16], int lane,
                                               float* hrow /* entry h at row */) {
#pragma unroll
  for (int t = 0; t < B; ++t) {
    if (!((mask >> t) & 1u)) continue;
    uint32_t xw[16];
    if constexpr (B == 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) xw[i] = x0[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = s_x[t * (kH / 8) + 4 * lane + i];
        xw[4 * i] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
      }
    }
    const float g = wave_sum(cg.dot_x(xw)) * sg;
    const float u = wave_sum(cu.dot_x(xw)) * su;
    if (lane == 0) store_coherent(hrow + (size_t)t * kI, silu_mul(g, u));
  }
}

// Down contribution of one unit (kUnitRows rows of one entry) for the tokens
// in `mask`; acc[r][t] collects the 16-lane group's sums (same in every lane).
template <int B, int FMT>
__device__ __forceinline__ void down_unit(const Chunk<FMT> (&rows)[kUnitRows], float gl,
                                          unsigned mask, const float* __restrict__ wt,
                                          const float* hent /* entry h [kMaxB][kI] */, int c16,
                                          float (&acc)[kUnitRows][B]) {
#pragma unroll 1
  for (int t = 0; t < B; ++t) {
    if (!((mask >> t) & 1u)) continue;
    float h[32];
    const float* hp = hent + (size_t)t * kI + 32 * c16;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const f32x2 v = load_coherent2(hp + 2 * i);
      h[2 * i] = v.x;
      h[2 * i + 1] = v.y;
    }
    const float sc = wt[t] * gl;
#pragma unroll
    for (int r = 0; r < kUnitRows; ++r) {
      const float v = sc * group16_sum(rows[r].dot_h(h));
#pragma unroll
      for (int tt = 0; tt < B; ++tt)       // static register index for any t
        if (tt == t) acc[r][tt] += v;
    }
  }
}

// h-ready counter k (k < kHBanks), one 128-byte line each, after the flags.
__device__ __forceinline__ uint32_t* hready_bank(uint8_t* ws, int k) {
  return reinterpret_cast<uint32_t*>(ws + kFlagOff + ((size_t)4 * kFusedGrid + k) * kFlagStride);
}

// ------------------------------------------------------------------ kernel
template <int B, int FMT>
__global__ __launch_bounds__(kFusedThreads, 1) void k_decode_fused(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ rw, ExpertsDev routed,
    ExpertsDev shared, uint16_t* __restrict__ out, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, uint8_t* __restrict__ ws) {
  constexpr int kTB = FMT == FMT_NVFP4 ? 4 : 2;      // gate/up row pairs per batch
  const int g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = tid >> 4, c16 = tid & 15;
  DecodeCtl* ctl = reinterpret_cast<DecodeCtl*>(ws);
  uint64_t* lslots = reinterpret_cast<uint64_t*>(ws + kSlotLogitOff);
  float* hbuf = reinterpret_cast<float*>(ws + kHOff);

  __shared__ uint4 s_x[B * kH / 8];
  __shared__ float s_part[4][kMaxB];
  __shared__ int s_ids[kMaxB][kK];
  __shared__ float s_w[kMaxB][kK];
  __shared__ unsigned s_mask[kE];
  __shared__ int s_slot[kE];
  __shared__ int s_act[kMaxActive];
  __shared__ unsigned s_amask[kMaxActive];
  __shared__ float s_wt[kMaxActive][kMaxB];
  __shared__ int s_nr;
  __shared__ uint32_t s_epoch;

  trace_stamp(ws, 0);
  // ---------------------------------------------------------------- step A
  // router row g: wave w covers columns [512 w, 512 w + 512), 8 per lane
  const uint4 wr = *reinterpret_cast<const uint4*>(rw + (size_t)g * kH + 512 * wave + 8 * lane);
  // shared expert gate/up: rows 2g and 2g + 1 (waves 0 and 1)
  const int srow = 2 * g + wave;
  Chunk<FMT> scg, scu;
  if (wave < 2) {
    scg.load_gu(shared, 0, 0, srow, lane);
    scu.load_gu(shared, 0, 1, srow, lane);
  }
#pragma unroll
  for (int k = 0; k < B; ++k)
    s_x[k * (kH / 8) + tid] = reinterpret_cast<const uint4*>(x)[k * (kH / 8) + tid];
  uint32_t x0[16];
  if constexpr (B == 1) {
    const uint4* p = reinterpret_cast<const uint4*>(x + 32 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = p[i];
      x0[4 * i] = v.x; x0[4 * i + 1] = v.y; x0[4 * i + 2] = v.z; x0[4 * i + 3] = v.w;
    }
  }
  if (tid == 0) {                                    // this call's epoch
    uint32_t* ctr = flag_ptr(ws, 0, g);
    const uint32_t e = load_flag(ctr) + 1u;
    store_flag(ctr, e);
    s_epoch = e;
  }
  __syncthreads();
  const uint32_t epoch = s_epoch;
  {
    float acc[B];
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const uint4 xv = s_x[t * (kH / 8) + 64 * wave + lane];
      float a = dot2_bf16(wr.x, xv.x, 0.0f);
      a = dot2_bf16(wr.y, xv.y, a);
      a = dot2_bf16(wr.z, xv.z, a);
      a = dot2_bf16(wr.w, xv.w, a);
      acc[t] = wave_sum(a);
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < B; ++t) s_part[wave][t] = acc[t];
    }
  }
  __syncthreads();
  if (tid < B)
    put_slot(lslots + tid * kE + g, s_part[0][tid] + s_part[1][tid] + s_part[2][tid] + s_part[3][tid],
             epoch);
  if (wave < 2)
    gateup_compute<B, FMT>(scg, scu, Chunk<FMT>::gscale(shared, 0, 0),
                           Chunk<FMT>::gscale(shared, 0, 1), (1u << B) - 1u, s_x, x0, lane,
                           hbuf + (size_t)kShSlot * kMaxB * kI + srow);
  trace_stamp(ws, 1);

  // ---------------------------------------------------------------- step B
  // top-6 per token, repeated identically in every workgroup
  for (int t = wave; t < B; t += 4) {
    float v[4];
    wait_slots<4>(lslots + t * kE + lane, 64, epoch, v, &ctl->err);
    float sel_l[kK];
    int sel_i[kK];
    wave_topk256<kK>(v, lane, sel_i, sel_l);
    if (lane == 0) {
      float s[kK], sum = 0.0f;
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        s[j] = 1.0f / (1.0f + expf(-sel_l[j]));
        sum += s[j];
      }
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        s_ids[t][j] = sel_i[j];
        s_w[t][j] = s[j] / sum;
      }
    }
  }
  trace_stamp(ws, 2);
  for (int e = tid; e < kE; e += kFusedThreads) s_mask[e] = 0u;
  __syncthreads();
  if (tid < B * kK) {
    const int t = tid / kK, j = tid % kK;
    atomicOr(&s_mask[s_ids[t][j]], 1u << t);
    if (g == 0) {
      if (ids_out) ids_out[t * kK + j] = s_ids[t][j];
      if (w_out) w_out[t * kK + j] = s_w[t][j];
    }
  }
  __syncthreads();
  if (wave == 0) {                                   // touched experts, ascending id
    int base = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 64 * q + lane;
      const unsigned m = s_mask[e];
      const uint64_t bal = __ballot(m != 0u);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (m != 0u) {
        s_act[pos] = e;
        s_amask[pos] = m;
        s_slot[e] = pos;
      }
      base += __popcll(bal);
    }
    if (lane == 0) s_nr = base;
  }
  __syncthreads();
  const int nr = s_nr;
  for (int idx = tid; idx < nr * B; idx += kFusedThreads) {
    const int a = idx / B, t = idx % B;
    float wt = 0.0f;
#pragma unroll
    for (int j = 0; j < kK; ++j)
      if (s_slot[s_ids[t][j]] == a) wt = s_w[t][j];
    s_wt[a][t] = wt;
  }
  if (tid == 0) {                                    // the shared expert is entry nr
    s_act[nr] = 0;
    s_amask[nr] = (1u << B) - 1u;
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) s_wt[nr][t] = 1.0f;
  }
  __syncthreads();

  // step-C work of this workgroup: its 8 output rows over every entry, as
  // units of 4 rows (one half of the tile) of one entry.  Groups 0 and 1 take
  // the shared expert's two halves; group k >= 2 takes routed units
  // u = k - 2 + 14 p, u = (entry u / 2, half u % 2); a group always works on
  // half k % 2.  The first kDepth units are fetched now.
  constexpr int kDepth = FMT == FMT_NVFP4 ? 2 : 1;
  const int half = grp & 1;
  const int n_units = 2 * nr;
  auto load_unit = [&](Chunk<FMT> (&dst)[kUnitRows], int p) {
    const int u = grp - 2 + 14 * p;
    if (grp >= 2 && u < n_units) {
      const size_t ee = (size_t)s_act[u >> 1];
#pragma unroll
      for (int r = 0; r < kUnitRows; ++r)
        dst[r].load_dn(routed, ee, g * kRowsPerWg + half * kUnitRows + r, c16);
    }
  };
  Chunk<FMT> dsh[kUnitRows];
  if (grp < 2) {
#pragma unroll
    for (int r = 0; r < kUnitRows; ++r)
      dsh[r].load_dn(shared, 0, g * kRowsPerWg + half * kUnitRows + r, c16);
  }
  Chunk<FMT> dbuf[kDepth][kUnitRows];
#pragma unroll
  for (int q = 0; q < kDepth; ++q) load_unit(dbuf[q], q);

  // routed gate/up: the nr * 512 row pairs are cut into 256 contiguous
  // ranges, one per workgroup; wave w takes T0 + w, T0 + w + 4, ... in
  // batches of kTB, the next batch in flight while one computes
  const int T = nr * kI;
  const int T0 = (int)(((long long)g * T) >> 8), T1 = (int)(((long long)(g + 1) * T) >> 8);
  {
    Chunk<FMT> cg[2][kTB], cu[2][kTB];
    auto load_batch = [&](Chunk<FMT> (&bg)[kTB], Chunk<FMT> (&bu)[kTB], int j0) {
#pragma unroll
      for (int q = 0; q < kTB; ++q) {
        const int s = T0 + wave + 4 * (j0 + q);
        if (s < T1) {
          const size_t ee = (size_t)s_act[s / kI];
          bg[q].load_gu(routed, ee, 0, s % kI, lane);
          bu[q].load_gu(routed, ee, 1, s % kI, lane);
        }
      }
    };
    auto run_batch = [&](const Chunk<FMT> (&bg)[kTB], const Chunk<FMT> (&bu)[kTB], int j0) {
#pragma unroll
      for (int q = 0; q < kTB; ++q) {
        const int s = T0 + wave + 4 * (j0 + q);
        if (s < T1) {
          const int a = s / kI, row = s % kI;
          const size_t ee = (size_t)s_act[a];
          gateup_compute<B, FMT>(bg[q], bu[q], Chunk<FMT>::gscale(routed, ee, 0),
                                 Chunk<FMT>::gscale(routed, ee, 1), s_amask[a], s_x, x0, lane,
                                 hbuf + (size_t)a * kMaxB * kI + row);
        }
      }
    };
    load_batch(cg[0], cu[0], 0);
    for (int j0 = 0; T0 + wave + 4 * j0 < T1; j0 += 2 * kTB) {
      load_batch(cg[1], cu[1], j0 + kTB);
      run_batch(cg[0], cu[0], j0);
      load_batch(cg[0], cu[0], j0 + 2 * kTB);
      run_batch(cg[1], cu[1], j0 + kTB);
    }
  }
  // publish: wait for this workgroup's h stores, then count in on bank g % 64
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_add(hready_bank(ws, g % kHBanks), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  trace_stamp(ws, 3);

  // ---------------------------------------------------------------- step C
  // every bank gains 4 per call: wait until all 64 hold 4 * epoch
  if (tid < 64) {
    const uint32_t want = (uint32_t)(kFusedGrid / kHBanks) * epoch;
    for (int spin = 0;; ++spin) {
      const uint32_t v = load_flag(hready_bank(ws, tid));
      if (__ballot(v != want) == 0) break;
      if (spin > kSpinLimit) {
        if (tid == 0)
          __hip_atomic_fetch_or(&ctl->err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  __syncthreads();
  trace_stamp(ws, 4);

  float acc[kUnitRows][B];
#pragma unroll
  for (int r = 0; r < kUnitRows; ++r)
#pragma unroll
    for (int t = 0; t < B; ++t) acc[r][t] = 0.0f;
  if (grp < 2) {
    down_unit<B, FMT>(dsh, Chunk<FMT>::gscale(shared, 0, 2), (1u << B) - 1u, s_wt[nr],
                      hbuf + (size_t)kShSlot * kMaxB * kI, c16, acc);
  } else {
    for (int p = 0; grp - 2 + 14 * p < n_units; p += kDepth) {
      Chunk<FMT> nxt[kDepth][kUnitRows];
#pragma unroll
      for (int q = 0; q < kDepth; ++q) load_unit(nxt[q], p + kDepth + q);
#pragma unroll
      for (int q = 0; q < kDepth; ++q) {
        const int u = grp - 2 + 14 * (p + q);
        if (u < n_units) {
          const int a = u >> 1;
          down_unit<B, FMT>(dbuf[q], Chunk<FMT>::gscale(routed, (size_t)s_act[a], 2), s_amask[a],
                            s_wt[a], hbuf + (size_t)a * kMaxB * kI, c16, acc);
        }
      }
#pragma unroll
      for (int q = 0; q < kDepth; ++q)
#pragma unroll
        for (int r = 0; r < kUnitRows; ++r) dbuf[q][r] = nxt[q][r];
    }
  }
  trace_stamp(ws, 5);
  __shared__ float s_acc[16][kUnitRows][kMaxB];
  if (c16 == 0) {
#pragma unroll
    for (int r = 0; r < kUnitRows; ++r)
#pragma unroll
      for (int t = 0; t < B; ++t) s_acc[grp][r][t] = acc[r][t];
  }
  __syncthreads();
  if (tid < kRowsPerWg * B) {                        // fixed order over the groups of the half
    const int r8 = tid / B, t = tid % B;
    const int h2 = r8 / kUnitRows, r = r8 % kUnitRows;
    float y = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) y += s_acc[2 * k + h2][r][t];
    out[(size_t)t * kH + g * kRowsPerWg + r8] = f32_to_bf16_rne(y);
  }
  trace_stamp(ws, 6);
}

// ------------------------------------------------------------------ launcher
static int g_fused_ok[64];   // per device: 0 unknown, 1 usable, -1 not

bool fused_supported() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (g_fused_ok[dev] == 0) {
    int cus = 0, occ_nv = 0, occ_bf = 0;
    const bool ok =
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_nv, k_decode_fused<8, FMT_NVFP4>,
                                                     kFusedThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_bf, k_decode_fused<8, FMT_BF16>,
                                                     kFusedThreads, 0) == hipSuccess;
    g_fused_ok[dev] = (ok && cus >= kFusedGrid && occ_nv >= 1 && occ_bf >= 1) ? 1 : -1;
  }
  return g_fused_ok[dev] == 1;
}

template <int B>
static void launch_fused_b(int fmt, const uint16_t* x, const uint16_t* rw, const ExpertsDev& routed,
                           const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                           uint8_t* ws, hipStream_t st) {
  if (fmt == FMT_NVFP4)
    hipLaunchKernelGGL((k_decode_fused<B, FMT_NVFP4>), dim3(kFusedGrid), dim3(kFusedThreads), 0, st,
                       x, rw, routed, shared, out, ids, w, ws);
  else
    hipLaunchKernelGGL((k_decode_fused<B, FMT_BF16>), dim3(kFusedGrid), dim3(kFusedThreads), 0, st,
                       x, rw, routed, shared, out, ids, w, ws);
}

hipError_t launch_decode_fused(int B, int fmt, const uint16_t* x, const uint16_t* rw,
                               const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                               int32_t* ids, float* w, uint8_t* ws, hipStream_t st) {
  switch (B) {
    case 1: launch_fused_b<1>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 2: launch_fused_b<2>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 3: launch_fused_b<3>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 4: launch_fused_b<4>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 5: launch_fused_b<5>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 6: launch_fused_b<6>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 7: launch_fused_b<7>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    case 8: launch_fused_b<8>(fmt, x, rw, routed, shared, out, ids, w, ws, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
