// The layer body of the single-launch decode kernels (B <= 8 tokens) of the
// Flint-style MoE layer on gfx950: one layer, as each of 256 workgroups runs
// it, and the kernels built from it (one layer per launch, a stack of
// independent layers, a chained residual stack).  Each kernel instance is
// compiled in one of the decode_*.hip translation units.
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
//      columns) -> logit slots (batch 1 in a stacked launch: eight rows per
//      workgroup, every XCD computing all 256; see kXcdLogits); the shared
//      expert's gate/up rows 2g, 2g+1
//      (routing-independent) -> h; the shared expert's down rows of the
//      workgroup's 8 outputs are fetched.
//   B  every workgroup waits for the 256 x B logits and repeats the sigmoid /
//      top-6 / renormalisation / dispatch itself (identical result everywhere,
//      no extra round trip): touched experts become entries in ascending id,
//      and each (entry, token) pair a slot of a compact h array (routed
//      pairs first, then the shared expert's).  The routed gate/up row pairs,
//      cut into 256 contiguous ranges, give SiLU(g) * u per token; the
//      workgroup writes its h once, as bf16, then counts in on an h-ready
//      counter.
//   C  once all h is in: the 7 B h pairs are copied to LDS (batch 1: from
//      epoch-tagged slots that every thread polls; larger batches: by
//      global-to-LDS loads once the h-ready counters are full), then the down GEMV
//      of the workgroup's 8 output rows over every entry (wave w takes routed
//      entries a = w - 1 mod 4 and the shared expert's tokens w, w + 4),
//      weighted by the routing, summed in a fixed order, rounded once to bf16.
//
// The layer's neighbours can be fused in (template parameters NORM, RESID;
// the same section's low-latency path fuses norm and combine into the
// adjacent GEMVs): the pre-MoE RMSNorm of x at the start of step A (every
// workgroup normalises the same x, so no exchange is needed), and the
// residual add before the output rounding of step C.
//
// Hand-over between workgroups uses relaxed agent-scope atomics (no cache
// write-back or invalidation), and plain stores for the XCD-local logits:
//  - call epoch: workgroup g keeps a private counter in the workspace; every
//    call adds one, so all counters agree (the workspace starts zeroed).
//  - logits: 8-byte slots {fp32 value, epoch} in kLogitReps copies; readers
//    poll copy g % kLogitReps until the epochs match.  Batch 1 in a stacked
//    launch: one copy per XCD, written with plain stores and read by that
//    XCD's workgroups only (the lines stay in its L2).
//  - h: coherent stores; after waiting for them a workgroup adds 1 to
//    h-ready counter g % 64 of each of kBankReps copies (one 128-byte line
//    each); readers poll the 64 counters of copy g % kBankReps until each
//    holds 4 * epoch.  Batch 1 writes h as epoch-tagged slots instead, which
//    readers poll directly (the counters still advance).
// A wave's loads and stores complete in issue order, so the kernel keeps
// stores out of the way of loads it waits for: h is staged in LDS and stored
// in one go, and the polling wave issues its prefetches after its wait.
// Every wait is bounded (tens of ms); on time-out the workgroup sets the
// workspace error word and carries on, so the kernel always terminates.
// Results are reproducible bit for bit (fixed summation orders, no atomics
// on data).
#pragma once

#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kFusedGrid = 256;             // workgroups (one per CU)
constexpr int kFusedThreads = 256;          // 4 waves, 16 groups of 16 lanes
constexpr int kRowsPerWg = kH / kFusedGrid; // 8 output rows per workgroup
constexpr int kHBanks = 64;                 // h-ready counters, one 128-byte line each
constexpr int kMaxRange = (kMaxB * kK * kI + kFusedGrid - 1) / kFusedGrid;  // routed rows per workgroup
constexpr int kSpinLimit = 1 << 18;
// Batches up to kHTagMaxB hand h over as epoch-tagged slots, which need no
// wait for the stores' acknowledgement before counting in; larger batches
// store plain bf16 h (half the bytes for every workgroup to copy) and count in
// once the stores are acknowledged.  kHDirect: readers of tagged h poll the
// slots directly instead of waiting for the counters first.
#ifndef MOE_H_TAG_MAXB
#define MOE_H_TAG_MAXB 1
#endif
#ifndef MOE_H_DIRECT
#define MOE_H_DIRECT 1
#endif
constexpr int kHTagMaxB = MOE_H_TAG_MAXB;
constexpr bool kHDirect = MOE_H_DIRECT != 0;
// Gate/up ranges at B > 1: the row pairs are cut into 256 ranges of equal
// weight, a row pair of an entry with n tokens weighing kGuWeight + n (its
// bytes, then one share of arithmetic per token); 0 cuts by row pairs alone.
#ifndef MOE_GU_WEIGHT
#define MOE_GU_WEIGHT 1
#endif
constexpr int kGuWeight = MOE_GU_WEIGHT;
// Batch 1 in a stacked launch exchanges the router logits inside each XCD:
// the 32 workgroups of an XCD compute all 256 router rows, 8 each (workgroup
// g rows 8 (g / 8) + j), and hand the logits over through the XCD's own L2
// (plain stores stay there; agent-scope loads read them), a round trip about
// half as long as one through memory.  The next layer's eight router rows go
// to LDS during the current layer's h exchange, when nothing waits for
// memory; a one-layer launch would wait for them before its router dot,
// which costs more than the exchange saves, so it keeps the device-wide
// slots, as larger batches do.  The hardware deals a launch's workgroups out
// to the 8 XCDs in turn, starting where the previous dispatch stopped, so
// the workgroups of one XCD are g = c, c + 8, ... for some c: their g / 8
// are 0 .. 31.  The slots are indexed by the XCD a workgroup reads from its
// hardware register.  (Were the deal ever different, an XCD would miss some
// rows and its logit wait would give up, which the status word reports.)
#ifndef MOE_XCD_LOGITS
#define MOE_XCD_LOGITS 1
#endif
template <int B, int PF>
constexpr bool kXcdLogits = MOE_XCD_LOGITS != 0 && B == 1 && PF != 0;
static_assert(kGuWeight >= 0 && kGuWeight + kMaxB < 16, "a row pair's weight fits 4 bits");

// ------------------------------------------------------------------ row chunks
// Weight loads through global-address-space pointers.  The stacked launch
// reads its weight pointers from the layer table in memory, which the
// compiler cannot place, and a flat load also counts against the LDS wait
// counter: every LDS wait and barrier would then wait for the weights in
// flight.
// (HIP's uint4 is a struct, whose copy drops the address space: its loads
// go through a native vector type.)
template <typename T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <>
__device__ __forceinline__ uint4 gld<uint4>(const void* p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A lane's 32 consecutive elements of one weight row.
template <int FMT>
struct Chunk;

template <>
struct Chunk<FMT_NVFP4> {
  uint4 c;
  uint16_t s;   // the two E4M3 block scales, as loaded (a 16-bit register value)
  __device__ __forceinline__ void load_gu(const ExpertsDev& X, size_t ee, int m, int row, int ch) {
    const size_t r = (ee * 2 + m) * kI + row;
    c = gld<uint4>(X.w13 + r * (kH / 2) + 16 * ch);
    s = gld<uint16_t>(X.w13s + r * (kH / 16) + 2 * ch);
  }
  __device__ __forceinline__ void load_dn(const ExpertsDev& X, size_t ee, int row, int ch) {
    const size_t r = ee * kH + row;
    c = gld<uint4>(X.w2 + r * (kI / 2) + 16 * ch);
    s = gld<uint16_t>(X.w2s + r * (kI / 16) + 2 * ch);
  }
  // sum_k w_k v_k over the chunk (v: 32 bf16 values in pairs), without the
  // tensor scale; v is x for gate/up rows and h for down rows
  __device__ __forceinline__ float dot_x(const uint32_t (&xw)[16]) const {
    return nvfp4_dot32(c, s, xw);
  }
  __device__ __forceinline__ static float gscale(const ExpertsDev& X, size_t ee, int m) {
    return gld<float>(X.glob + ee * 3 + m);
  }
};

template <>
struct Chunk<FMT_BF16> {
  uint4 w[4];
  __device__ __forceinline__ void load_gu(const ExpertsDev& X, size_t ee, int m, int row, int ch) {
    const uint8_t* p = X.w13 + (((ee * 2 + m) * kI + row) * kH + 32 * ch) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = gld<uint4>(p + 16 * i);
  }
  __device__ __forceinline__ void load_dn(const ExpertsDev& X, size_t ee, int row, int ch) {
    const uint8_t* p = X.w2 + ((ee * kH + row) * kI + 32 * ch) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = gld<uint4>(p + 16 * i);
  }
  __device__ __forceinline__ float dot_x(const uint32_t (&xw)[16]) const { return bf16_dot32(w, xw); }
  __device__ __forceinline__ static float gscale(const ExpertsDev&, size_t, int) { return 1.0f; }
};

// ------------------------------------------------------------------ helpers
// Phase timestamps of a traced build (-DMOE_PHASE_TRACE): kept in LDS and
// written after the kernel's last step, so they add no stores to the
// memory queue of the phases they time.
#ifdef MOE_PHASE_TRACE
constexpr int kTraceStamps = 24;
__shared__ unsigned long long s_trace[kTraceStamps];
#endif
__device__ __forceinline__ void trace_stamp(uint8_t* ws, int k) {
#ifdef MOE_PHASE_TRACE
  if (threadIdx.x == 0) s_trace[k] = __builtin_amdgcn_s_memrealtime();
#else
  (void)ws;
  (void)k;
#endif
}
__device__ __forceinline__ void trace_flush(uint8_t* ws) {
#ifdef MOE_PHASE_TRACE
  __syncthreads();
  if (threadIdx.x < kTraceStamps)
    reinterpret_cast<unsigned long long*>(ws + kDecodeWsBytes)[blockIdx.x * kTraceStamps +
                                                               threadIdx.x] = s_trace[threadIdx.x];
#else
  (void)ws;
#endif
}

// A plain store: the line stays in this XCD's L2 (no write-through), where
// the agent-scope loads of the XCD's other workgroups find it.
__device__ __forceinline__ void put_slot_xcd(uint64_t* p, float v, uint32_t epoch) {
  const uint64_t w = (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)epoch << 32);
  *(__attribute__((address_space(1))) uint64_t*)p = w;
}

// Cache-policy operand of gfx950 memory instructions for a device-coherent
// access: the SC1 bit (device scope; the data may come from another XCD).
constexpr int kCpolDevice = 16;

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u);
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

// Per-workgroup epoch counter in the workspace, one 128-byte line each.
__device__ __forceinline__ uint32_t* epoch_ptr(uint8_t* ws, int wg) {
  return reinterpret_cast<uint32_t*>(ws + kFlagOff + (size_t)wg * kFlagStride);
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
      __hip_atomic_fetch_or(err, kErrLogits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Reads N tagged slots per lane (p[k * stride], k < N), polling until every
// slot carries `epoch`, and returns their 32-bit payloads.  Bounded: on
// time-out the error word gets `bit` and the payloads are whatever was read.
template <int N>
__device__ __forceinline__ void wait_slots_u32(const uint64_t* p, int stride, uint32_t epoch,
                                               uint32_t (&out)[N], unsigned* err, unsigned bit) {
  uint64_t pending = N >= 64 ? ~0ull : ((1ull << N) - 1ull);
  for (int spin = 0;; ++spin) {
    uint64_t w[N];
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (pending & (1ull << k)) w[k] = get_slot(p + k * stride);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if ((pending & (1ull << k)) && (uint32_t)(w[k] >> 32) == epoch) {
        out[k] = (uint32_t)w[k];
        pending &= ~(1ull << k);
      }
    }
    if (__ballot(pending != 0ull) == 0) break;
    if (spin > kSpinLimit) {
      __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// wait_slots_u32 with two poll rounds in flight: round r + 1 is issued
// before round r is checked, so a slot that lands just after a round left is
// seen half a round trip later rather than a whole one.  Four rounds in
// straight-line code (so that the loads in flight are counted exactly), then
// the plain loop; the rounds still in flight at an exit are discarded.  Only
// where no global-to-LDS load is in flight: behind one the compiler waits
// for every load before each check, which makes it slower than the loop.
template <int N, int R = 4>
__device__ __forceinline__ void wait_slots_u32_p2(const uint64_t* p, int stride, uint32_t epoch,
                                                  uint32_t (&out)[N], unsigned* err,
                                                  unsigned bit) {
  static_assert(R == 2 || R == 4, "two or four rounds");
  uint64_t w0[N], w1[N], w2[N], w3[N];   // (w2, w3 unused with two rounds)
  auto issue = [&](uint64_t (&w)[N]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < N; ++k) w[k] = get_slot(p + k * stride);
  };
  auto done = [&](const uint64_t (&w)[N]) __attribute__((always_inline)) {
    bool ok = true;
#pragma unroll
    for (int k = 0; k < N; ++k) ok &= (uint32_t)(w[k] >> 32) == epoch;
    if (__ballot(!ok) != 0) return false;
#pragma unroll
    for (int k = 0; k < N; ++k) out[k] = (uint32_t)w[k];
    return true;
  };
  issue(w0);
  issue(w1);
  if (done(w0)) return;
  if constexpr (R == 4) {
    issue(w2);
    if (done(w1)) return;
    issue(w3);
    if (done(w2)) return;
    if (done(w3)) return;
  } else {
    if (done(w1)) return;
  }
  wait_slots_u32<N>(p, stride, epoch, out, err, bit);
}

// The same for one token's 256 logits (4 per lane, stride 64), as floats.
__device__ __forceinline__ void wait_logits_p2(const uint64_t* p, uint32_t epoch, float (&v)[4],
                                               unsigned* err) {
  uint32_t w[4];
  wait_slots_u32_p2<4>(p, 64, epoch, w, err, kErrLogits);
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = __builtin_bit_cast(float, w[q]);
}

__device__ __forceinline__ void put_slot_u32(uint64_t* p, uint32_t v, uint32_t epoch) {
  const uint64_t w = (uint64_t)v | ((uint64_t)epoch << 32);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sortable integer key of a logit: order-preserving over all non-NaN floats,
// with -0 taken as +0 so that equal values compare equal.
__device__ __forceinline__ int logit_key(float f) {
  int b = __builtin_bit_cast(int, f);
  b = b == (int)0x80000000 ? 0 : b;
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_logit(int k) {
  return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF));
}

// The wave's maximum in every lane: within 16-lane rows by DPP, then across
// rows with gfx950's 16- and 32-lane half swaps (all vector instructions).
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = max((int)r16[0], (int)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return max((int)r32[0], (int)r32[1]);
}

__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true));
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true));
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Positions i, i + 1 of a lane's list, descending by key; a swap needs a
// strictly larger key, so equal keys keep their order (lower expert first).
__device__ __forceinline__ void cmpx(int (&k)[4], int (&q)[4], int i) {
  const bool sw = k[i + 1] > k[i];
  const int ka = k[i], qa = q[i];
  k[i] = sw ? k[i + 1] : ka;
  q[i] = sw ? q[i + 1] : qa;
  k[i + 1] = sw ? ka : k[i + 1];
  q[i + 1] = sw ? qa : q[i + 1];
}

// Top-6 of one token's 256 router logits (v[q] = logit of expert 64 q + lane)
// under the order (logit descending, expert ascending), as the pages' router
// selects ("Day-0 Support for Flint on vLLM", Model architecture).  Each lane
// first sorts its 4 logits (odd-even transposition, stable); each round takes
// the maximum of the lane heads and pops it.  Lane j < 6 returns choice j.
// N tokens at once (a wave with two tokens): their rounds are independent
// chains, interleaved in one loop so that each hides the other's latency.
template <int N>
__device__ __forceinline__ void wave_top6(const float (&v)[N][4], int lane, int (&my_id)[N],
                                          float (&my_l)[N]) {
  int k[N][4], q[N][4], myk[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[n][i] = logit_key(v[n][i]);
      q[n][i] = i;
    }
    cmpx(k[n], q[n], 0); cmpx(k[n], q[n], 2); cmpx(k[n], q[n], 1);
    cmpx(k[n], q[n], 0); cmpx(k[n], q[n], 2); cmpx(k[n], q[n], 1);
    myk[n] = 0;
    my_id[n] = 0;
  }
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    int m[N], sel[N];
#pragma unroll
    for (int n = 0; n < N; ++n) m[n] = wave_max_i32(k[n][0]);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const uint64_t bal = __ballot(k[n][0] == m[n]);
      if (__popcll(bal) == 1) {
        sel[n] = __builtin_ctzll(bal);
      } else {             // equal heads: the lowest expert id among them
        sel[n] = wave_min_i32(k[n][0] == m[n] ? 64 * q[n][0] + lane : 0x7FFFFFFF) & 63;
      }
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int e = 64 * __builtin_amdgcn_readlane(q[n][0], sel[n]) + sel[n];
      if (lane == j) {
        my_id[n] = e;
        myk[n] = m[n];
      }
      if (lane == sel[n]) {
        k[n][0] = k[n][1]; k[n][1] = k[n][2]; k[n][2] = k[n][3]; k[n][3] = (int)0x80000000;
        q[n][0] = q[n][1]; q[n][1] = q[n][2]; q[n][2] = q[n][3];
      }
    }
  }
#pragma unroll
  for (int n = 0; n < N; ++n) my_l[n] = key_logit(myk[n]);
}


// Four Over Six quantisation (W4A4) of 16-element blocks held by lane pairs:
// lane 2b holds elements 0..7 of block b as one 16-byte piece, lane 2b + 1
// elements 8..15; g is the vector's global scale (amax / 2688).  Returns this
// lane's 8 quantised values e2m1 * e4m3 (the global apart), exact in bf16.
// The decisions are the general path's and the oracle's: candidate scales
// E4M3(bmax / M / g) for M = 6 and 4, codes E2M1(v / (e4m3 * g)), and the
// block's absolute errors summed in element order (the even lane's eight
// from 0, the odd lane continuing from that sum); 4 only if strictly better.
__device__ __forceinline__ uint4 a4_quant_piece(uint4 piece, float g) {
  const uint32_t u[4] = {piece.x, piece.y, piece.z, piece.w};
  float v[8], m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(u[i]);
    v[2 * i + 1] = bf16_hi(u[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  const float bmax = fmaxf(m, dpp_f32<0xB1>(m));           // quad_perm [1,0,3,2]: the partner
  const bool zero = g == 0.0f || bmax == 0.0f;
  const float gg = zero ? 1.0f : g, bb = zero ? 1.0f : bmax;  // (no division by 0 on the way)
  // bmax / 6 through the reciprocal (bmax is a bf16 value; see
  // div_by_recip), bmax / 4 as a product (exact, or the same rounding when
  // it underflows); the divisions by the global stay divisions
  const float b6 = div_by_recip(bb, 6.0f, 0x1.555556p-3f), b4 = __fmul_rn(bb, 0.25f);
  const uint32_t sc = a4_e4m3_pk(__fdiv_rn(b6, gg),     // byte 0: M = 6
                                 __fdiv_rn(b4, gg));    // byte 1: M = 4
  const float v6 = e4m3_to_f32<0>(sc), v4 = e4m3_to_f32<1>(sc);
  const float q6 = __fmul_rn(v6, gg), q4 = __fmul_rn(v4, gg);
  // codes; a scale that rounded to 0 gives code 0 (the division by a
  // stand-in divisor keeps the code free of branches)
  const bool p6 = q6 > 0.0f, p4 = q4 > 0.0f;
  const float d6 = p6 ? q6 : 1.0f, d4 = p4 ? q4 : 1.0f;
  // the 16 quotients v / d, correctly rounded: from the reciprocal of each
  // divisor when every block of the wave has divisors in [2^-64, 2^64] (see
  // div_by_recip), else by division
  float r6[8], r4[8];
  const bool in_range = d6 >= 0x1p-64f && d6 <= 0x1p64f && d4 >= 0x1p-64f && d4 <= 0x1p64f;
  if (__builtin_expect(__ballot(!in_range) == 0ull, 1)) {
    const float y6 = __fdiv_rn(1.0f, d6), y4 = __fdiv_rn(1.0f, d4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r6[i] = div_by_recip(v[i], d6, y6);
      r4[i] = div_by_recip(v[i], d4, y4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r6[i] = __fdiv_rn(v[i], d6);
      r4[i] = __fdiv_rn(v[i], d4);
    }
  }
  float c6[8], c4[8], e6[8], e4[8], own6 = 0.0f, own4 = 0.0f;
  a4_e2m1_unpk8(a4_e2m1_pk8(r6), c6);
  a4_e2m1_unpk8(a4_e2m1_pk8(r4), c4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c6[i] = p6 ? c6[i] : 0.0f;
    c4[i] = p4 ? c4[i] : 0.0f;
    e6[i] = fabsf(__fsub_rn(v[i], __fmul_rn(c6[i], q6)));
    e4[i] = fabsf(__fsub_rn(v[i], __fmul_rn(c4[i], q4)));
    own6 = __fadd_rn(own6, e6[i]);
    own4 = __fadd_rn(own4, e4[i]);
  }
  // odd lane: continue from the even lane's sum over the block's first half
  float t6 = dpp_f32<0xA0>(own6), t4 = dpp_f32<0xA0>(own4);   // quad_perm [0,0,2,2]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t6 = __fadd_rn(t6, e6[i]);
    t4 = __fadd_rn(t4, e4[i]);
  }
  const float m6 = dpp_f32<0xF5>(t6), m4 = dpp_f32<0xF5>(t4);   // quad_perm [1,1,3,3]: the odd lane's
  const bool four = m4 < m6;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = zero ? 0.0f : (four ? c4[2 * i] * v4 : c6[2 * i] * v6);
    const float b = zero ? 0.0f : (four ? c4[2 * i + 1] * v4 : c6[2 * i + 1] * v6);
    o[i] = f32x2_to_bf16x2_rne(a, b);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// LDS position (16-byte units) of piece q (elements 8 q .. 8 q + 7) of token
// t's x row.  The low two bits of q are XORed with bits 3..4: a lane's
// 32-element chunk is pieces 4 l .. 4 l + 3, and with this swizzle the lanes
// reading piece 4 l + i hit distinct banks in every group of 8 lanes
// (unswizzled, their 64-byte stride puts four lanes on one bank), while 8
// consecutive pieces stay in one 128-byte group, so piece-per-thread and
// word-per-thread accesses stay conflict-free too.
__device__ __forceinline__ int sx_pos(int t, int q) { return t * (kH / 8) + (q ^ ((q >> 3) & 3)); }

// One gate/up row pair of an entry for the wave's tokens in `mask` (at most
// four: the tokens of parity `par`, token t in slot t / 2); the wave's lanes
// cover the 2048 columns.  The gate and up partial sums of every token are
// reduced together (wave_sum8: value j's total in lanes 8 j .. 8 j + 7, the
// same tree for every slot, so a token's h does not depend on its slot), and
// lane 16 i puts h = SiLU(g) * u of slot i's token t in hdst[t] (LDS: the
// workgroup writes its h to the workspace in one go, so that no store sits in
// front of the next weight loads in the wave's memory queue).
template <int B, int FMT, bool A4 = false>
__device__ __forceinline__ void gateup_compute(const Chunk<FMT>& cg, const Chunk<FMT>& cu, float sg,
                                               float su, unsigned mask, int par, const uint4* s_x,
                                               const uint32_t (&x0)[16], int lane, float* hdst,
                                               const float* gx = nullptr /* W4A4: x global by token */) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  if constexpr (B == 1) {
    if (mask & 1u) {
      v[0] = cg.dot_x(x0);
      v[1] = cu.dot_x(x0);
    }
  } else {
    // the tokens (a wave-uniform mask) in a rolled loop, for code size
#pragma unroll 1
    for (unsigned mm = __builtin_amdgcn_readfirstlane(mask); mm != 0u; mm &= mm - 1u) {
      const int t = __builtin_ctz(mm);
      uint32_t xw[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u4 = s_x[sx_pos(t, 4 * lane + i)];
        xw[4 * i] = u4.x; xw[4 * i + 1] = u4.y; xw[4 * i + 2] = u4.z; xw[4 * i + 3] = u4.w;
      }
      const float dg = cg.dot_x(xw), du = cu.dot_x(xw);
#pragma unroll
      for (int j = 0; j < 4; ++j)           // static register index for any t
        if (j == (t >> 1)) {
          v[2 * j] = dg;
          v[2 * j + 1] = du;
        }
    }
  }
  const float z = wave_sum8(v, lane);
  const float zu = dpp_f32<0x128>(z);
  const int t = 2 * (lane >> 4) + par;
  if ((lane & 15) == 0 && t < B && ((mask >> t) & 1u)) {
    if constexpr (A4)   // the dot products ran on e2m1 * e4m3: times the token's x global
      hdst[t] = silu_mul(z * sg * gx[t], zu * su * gx[t]);
    else
      hdst[t] = silu_mul(z * sg, zu * su);
  }
}

// 32 consecutive bf16 h values (chunk c16, as 16 packed pairs) of pair p
// from LDS.  A pair is 64 uint4s; uint4 (p, 4 c + i) sits at p * 64 + 16 i + c,
// so the 16 lanes of a row group read consecutive uint4s.
__device__ __forceinline__ void load_h(const uint4* s_h, int p, int c16, uint32_t (&h)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = s_h[p * 64 + 16 * i + c16];
    h[4 * i] = v.x; h[4 * i + 1] = v.y; h[4 * i + 2] = v.z; h[4 * i + 3] = v.w;
  }
}

// Down contribution of one entry to the workgroup's 8 output rows.  Lanes
// 16 j .. 16 j + 15 of a wave hold rows 2 j and 2 j + 1 (32 columns each);
// acc[r][t] gathers the lane's unreduced partial sums, scaled by the routing
// weight of token t and the tensor scale.  The entry's h pairs start at p0.
template <int B, int FMT, bool A4 = false>
__device__ __forceinline__ void down_entry(const Chunk<FMT> (&rows)[2], float gl, unsigned mask,
                                           const float* wt /* by token */, const uint4* s_h,
                                           int p0, int c16, float (&acc)[2][B],
                                           const float* gh = nullptr /* W4A4: h global by pair */) {
  auto token = [&](int t, int p) __attribute__((always_inline)) {
    uint32_t h[16];
    load_h(s_h, p, c16, h);
    const float sc = wt[t] * gl;
    float d0 = rows[0].dot_x(h), d1 = rows[1].dot_x(h);
    if constexpr (A4) {   // the dot products ran on e2m1 * e4m3: times the pair's global
      d0 *= gh[p];
      d1 *= gh[p];
    }
#pragma unroll
    for (int tt = 0; tt < B; ++tt)       // static register index for any t
      if (tt == t) {
        acc[0][tt] = __builtin_fmaf(sc, d0, acc[0][tt]);
        acc[1][tt] = __builtin_fmaf(sc, d1, acc[1][tt]);
      }
  };
  if constexpr (B == 1) {                // the one token (mask 1): a static index
    token(0, p0);
  } else {
    // the entry's tokens only: set bits in ascending order, as its h pairs
    int p = p0;
#pragma unroll 1
    for (unsigned m = mask; m != 0u; m &= m - 1u) token(__builtin_ctz(m), p++);
  }
}

// h-ready counter k (k < kHBanks) of copy r, one 128-byte line each, after
// the epoch counters.
__device__ __forceinline__ uint32_t* hready_bank(uint8_t* ws, int r, int k) {
  return reinterpret_cast<uint32_t*>(ws + kFlagOff +
                                     ((size_t)kFusedGrid + (size_t)r * kHBanks + k) * kFlagStride);
}

// The loads of a layer that depend on neither x nor the routing: router row
// g at B > 1 (wave w covers columns [512 w, 512 w + 512), 8 per lane; batch 1
// loads its eight rows at the start of the layer); each shared
// expert's gate/up row 2g + (w & 1) for the tokens of parity w >> 1 (at B = 1
// waves 0 and 1 only); its down rows of this workgroup's 8 outputs.  NS
// shared experts (1 for Flint; 2 for the Inkling shape, which is Flint's with
// two shared experts).
template <int FMT, int NS = 1>
struct StepAPre {
  uint4 wr;
  Chunk<FMT> scg[NS], scu[NS], dsh[NS][2];
};

template <int B>
__device__ __forceinline__ unsigned shared_token_mask(int wave) {
  return ((1u << B) - 1u) & ((wave >> 1) ? 0xAAAAAAAAu : 0x55555555u);
}

template <int B, int FMT, int NS, bool RW = true>
__device__ __forceinline__ void load_pre_gateup(StepAPre<FMT, NS>& p, const uint16_t* rw,
                                                const ExpertsDev& shared, int g, int wave,
                                                int lane) {
  if constexpr (RW) p.wr = gld<uint4>(rw + (size_t)g * kH + 512 * wave + 8 * lane);
  if (shared_token_mask<B>(wave)) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      p.scg[s].load_gu(shared, s, 0, 2 * g + (wave & 1), lane);
      p.scu[s].load_gu(shared, s, 1, 2 * g + (wave & 1), lane);
    }
  }
}

// The eight router rows of a batch-1 workgroup under the XCD-local logit
// exchange, rows 8 (g / 8) + j, straight to LDS (16-byte loads that bypass
// the registers: lane l of wave w lands at s_rw[64 (4 j + w) + l], its own
// columns 512 w + 8 l .. + 7 of row j, which only it reads back).
__device__ __forceinline__ void router_rows_to_lds(const uint16_t* rw, int g, int wave, int lane,
                                                   uint4* s_rw) {
  const uint16_t* rb = rw + (size_t)(8 * (g >> 3)) * kH + 512 * wave + 8 * lane;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(rb + (size_t)j * kH),
        (__attribute__((address_space(3))) void*)(s_rw + 64 * (4 * j + wave)), 16, 0, 0);
}

// Their LDS: one array per kernel, declared outside the layer template, whose
// instances (a stacked launch's first and later layers) would each get their
// own and read rows the previous layer never loaded.
__device__ __forceinline__ uint4* router_rows_lds() {
  __shared__ uint4 s_rw[8 * 4 * 64];
  return s_rw;
}

template <int FMT, int NS>
__device__ __forceinline__ void load_pre_down(StepAPre<FMT, NS>& p, const ExpertsDev& shared,
                                              int g, int lane) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int r = 0; r < 2; ++r)
      p.dsh[s][r].load_dn(shared, s, g * kRowsPerWg + 2 * (lane >> 4) + r, lane & 15);
}

// A stacked launch prefetches the next layer's step-A rows right after the
// h copy when this layer issues no load after it: each wave's routed
// entries (at most 6 B / 4 of them) all fit in the two down-row sets issued
// before the h-ready wait.  Otherwise the prefetch goes out behind the last
// down-row loads, so that none of them queues behind it.
// A set holds kDownDepth routed entries per wave: 4 for NVFP4, fewer when
// two sets already cover a wave's at most ceil(6 B / 4) entries (the loads
// are unconditional, so a slot past a wave's last entry is a wasted load).
template <int B, int FMT>
constexpr int kDownDepth =
    FMT == FMT_NVFP4 ? ((kK * B + 7) / 8 < 4 ? (kK * B + 7) / 8 : 4) : 1;
template <int B, int FMT>
constexpr bool kPrefetchNext = kK * B <= 4 * 2 * kDownDepth<B, FMT>;

// ------------------------------------------------------------------ kernel
// One layer, as one workgroup of the 256 runs it (the body of both kernels
// below).
// pre: the step-A loads of this layer.  PF: 0 none (one layer per launch);
// in a stacked launch 1 this layer issues its own step-A loads and, once
// nothing of its own queues behind them, those of `next` (see
// kPrefetchNext); 2 as 1, but this layer's were issued by the previous layer.  PF is static so that the
// compiler counts the loads in flight exactly (a load under a runtime branch
// makes it wait for all of them).  epoch_reg: this layer's epoch on return;
// on entry, when EPREG, the previous layer's (stacked launches).
// RES: the residual added before the output rounding: 0 none, 1 fz.resid from
// memory, 2 resid_reg (this thread's output element of the previous layer,
// which is this layer's input: a chained stack).  XIN: x from memory (0) or,
// 1, from the previous layer's output slots (a chained stack, where x of this
// layer is the residual stream the previous layer wrote).  XOUT: publish the
// output as tagged slots for the next layer, and keep this thread's output
// element in resid_reg.
template <int B, int FMT, bool NORM, int RES, int PF, bool EPREG, int XIN, bool XOUT, int NS = 1,
          bool A4 = false>
__device__ __forceinline__ void decode_layer(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ rw, const ExpertsDev& routed,
    const ExpertsDev& shared, uint16_t* __restrict__ out, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, uint8_t* __restrict__ ws, const FuseDev& fz, StepAPre<FMT, NS>& pre,
    const LayerDev& next, uint32_t& epoch_reg, float& resid_reg) {
  // early: after the h copy (every routed down row is already in flight);
  // late: behind step C's last down-row loads
  constexpr bool kPfEarly = PF != 0 && kPrefetchNext<B, FMT>;
  constexpr bool kPfLate = PF != 0 && !kPrefetchNext<B, FMT>;
  // gate/up row pairs per batch (at B = 1 a wave has exactly 3: 12 per workgroup)
#ifndef MOE_GU_TB
#define MOE_GU_TB 3
#endif
  constexpr int kTB = FMT == FMT_NVFP4 ? (B == 1 ? 3 : MOE_GU_TB) : 2;
  constexpr int kDepthC = kDownDepth<B, FMT>;           // entries of down rows in flight
  // batch 1 issues its routed down rows after publishing h instead of behind
  // the gate/up rows: the gate/up burst then carries only gate/up rows
  constexpr bool kLateDown = B == 1;
  static_assert(NS >= 1 && NS <= kMaxShared, "one or two shared experts");
  // W4A4 (NVFP4 activations with the Four Over Six block scale, FMT_NVFP4
  // weights): the plain layer; x and h are quantised by every workgroup
  // itself (all of x, and all of h after the h copy)
  static_assert(!A4 || (FMT == FMT_NVFP4 && !NORM && RES == 0 && XIN == 0 && !XOUT && NS == 1 &&
                        PF == 0), "W4A4: the plain NVFP4 layer");
  constexpr int kPairs = (kK + NS) * B;              // h pairs: 6 B routed + NS B shared
  constexpr bool kXL = kXcdLogits<B, PF>;
  const int g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp4 = lane >> 4, c16 = lane & 15;
  DecodeCtl* ctl = reinterpret_cast<DecodeCtl*>(ws);
  uint64_t* lslots = reinterpret_cast<uint64_t*>(ws + kSlotLogitOff);
  uint64_t* lxslots = reinterpret_cast<uint64_t*>(ws + kSlotLXOff);
  uint64_t* xslots = reinterpret_cast<uint64_t*>(ws + kSlotXOff);
  uint64_t* hslots = reinterpret_cast<uint64_t*>(ws + kSlotHOff);
  constexpr bool kTagH = B <= kHTagMaxB;
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + kHOff);

  // x (bf16 [B][2048]) in steps A and B; the h pairs (bf16 [7 B][512]) in step C
  __shared__ uint4 s_xh[kPairs * kI * 2 / 16];
  uint4* s_x = s_xh;
  const uint4* s_h = s_xh;
  __shared__ float s_part[4][kMaxB];
  __shared__ unsigned s_mask[kE];                    // tokens choosing each expert
  __shared__ float s_wfull[kE][kMaxB];               // routing weight (expert, token)
  __shared__ int s_act[kMaxActive];                  // entry -> expert (shared last)
  __shared__ unsigned s_amask[kMaxActive];
  __shared__ int s_pair0[kMaxActive];                // first h pair of each entry
  __shared__ float s_gs[kMaxActive][3];              // tensor scales of each routed entry
  __shared__ int s_nr;
  __shared__ int s_t01[2];                           // weighted gate/up range (B > 1)
  __shared__ uint32_t s_epoch;
  __shared__ float s_hsh[NS][2][kMaxB];              // this workgroup's shared-expert h
  __shared__ float s_hout[kMaxRange][kMaxB];         // its routed h, by row of its range

  trace_stamp(ws, 0);
  // ---------------------------------------------------------------- step A
  const unsigned smask = shared_token_mask<B>(wave);
  // batch 1 in a stacked launch: router rows 8 (g / 8) + j, j < 8 (the 32
  // workgroups of an XCD cover all 256), in LDS; the first layer loads its
  // own, a later one's came during the previous layer's h exchange
  uint4* const s_rw = kXL ? router_rows_lds() : nullptr;
  if constexpr (kXL && PF == 1) router_rows_to_lds(rw, g, wave, lane, s_rw);
  // this XCD's copy of the XCD-local logit slots
  uint64_t* const lxmine = lxslots + (xcc_id() & (kXcds - 1)) * kE;
  if constexpr (PF != 2) load_pre_gateup<B, FMT, NS, !kXL>(pre, rw, shared, g, wave, lane);
  // Every load of step A goes out before any of them is used (loads return
  // in issue order, so a wait for one is a wait for all before it): x, piece
  // tid of each token; the norm weight and the residual of this workgroup's
  // output elements (row g * 8 + tid / B, token tid % B), read from x when
  // not fused so that no branch splits the loads; x in registers at B = 1;
  // the shared expert's down rows of this workgroup (step C).
  __shared__ float s_rinv[kMaxB];
  uint4 xr[B], nw = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (XIN == 0) {
#pragma unroll
    for (int k = 0; k < B; ++k) xr[k] = reinterpret_cast<const uint4*>(x)[k * (kH / 8) + tid];
  }
  if constexpr (NORM) nw = reinterpret_cast<const uint4*>(fz.norm_w)[tid];
  uint16_t rv = 0;
  if constexpr (RES == 1) {
    const int ro = tid < kRowsPerWg * B ? (tid % B) * kH + g * kRowsPerWg + tid / B : 0;
    rv = fz.resid[ro];
  }
  uint32_t x0[16];
  if constexpr (B == 1 && XIN == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(x + 32 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = p[i];
      x0[4 * i] = v.x; x0[4 * i + 1] = v.y; x0[4 * i + 2] = v.z; x0[4 * i + 3] = v.w;
    }
  }
  float sh_sg[NS], sh_su[NS], sh_sd[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    sh_sg[s] = Chunk<FMT>::gscale(shared, s, 0);
    sh_su[s] = Chunk<FMT>::gscale(shared, s, 1);
    sh_sd[s] = Chunk<FMT>::gscale(shared, s, 2);
  }
  if constexpr (PF != 2) load_pre_down<FMT, NS>(pre, shared, g, lane);
  const float resid = RES == 2 ? resid_reg : __builtin_bit_cast(float, (uint32_t)rv << 16);
  // A chained stack's x is the previous layer's output, which every
  // workgroup publishes as tagged slots of its rows (epoch of that layer):
  // slot i of a copy holds bf16 elements 2 i, 2 i + 1 of the [B][2048] x, so
  // thread tid's slots tid + 256 k land in LDS as x's 32-bit words.
  if constexpr (XIN == 1) {
    uint32_t xs[4 * B];
    wait_slots_u32_p2<4 * B, (B <= 2 ? 4 : 2)>(xslots + (g % kXReps) * (kSlotXRep / 8) + tid,
                                               kFusedThreads, epoch_reg, xs, &ctl->err,
                                               kErrXReady);
    if constexpr (B > 1) trace_stamp(ws, 15);   // (stamp 15 is the top-6 at B = 1)
    uint32_t* s_x32 = reinterpret_cast<uint32_t*>(s_x);
#pragma unroll
    for (int k = 0; k < 4 * B; ++k)   // word tid + 256 k: token k / 4, piece 64 (k % 4) + tid / 4
      s_x32[4 * sx_pos(k >> 2, 64 * (k & 3) + (tid >> 2)) + (tid & 3)] = xs[k];
    __syncthreads();
    trace_stamp(ws, 16);
    if constexpr (B == 1) {
      xr[0] = s_x[sx_pos(0, tid)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = s_x[sx_pos(0, 4 * lane + i)];
        x0[4 * i] = v.x; x0[4 * i + 1] = v.y; x0[4 * i + 2] = v.z; x0[4 * i + 3] = v.w;
      }
    }
  }
  // x to LDS as is, or through the fused RMSNorm.  A row's mean square is
  // summed by one wave holding the row 32 elements per lane (the same order
  // on every path).  At B = 1 every wave already holds the row in x0, so
  // each thread normalises its piece before the barrier below and x0 is
  // reread from LDS after it; at B > 1 wave w sums the rows of tokens w and
  // w + 4 and the pieces are normalised after the barrier, behind a second
  // one.
  if constexpr (NORM) {
    if constexpr (B == 1) {
      const float r = row_rms_inv(x0, fz.eps);
      const uint4 v = rmsnorm8(xr[0], nw, r);
      if constexpr (XIN == 1) {
        // x in LDS is still being read (x0 of the other waves): the
        // normalised x goes to a buffer of its own, which serves as x from here
        __shared__ uint4 s_xn[kH / 8];
        s_xn[sx_pos(0, tid)] = v;
        s_x = s_xn;
      } else {
        s_x[sx_pos(0, tid)] = v;
      }
      if (fz.xn_out && g == 0) reinterpret_cast<uint4*>(fz.xn_out)[tid] = v;
    } else {
      // the four piece sums of token t's row, lane l's pieces 4 l .. 4 l + 3
      // (16-byte units; from LDS through the swizzle, conflict-free)
      auto row_pieces = [&](int t, float (&p)[4]) __attribute__((always_inline)) {
        if constexpr (XIN == 1) {
          uint4 u[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) u[k] = s_x[sx_pos(t, 4 * lane + k)];
#pragma unroll
          for (int k = 0; k < 4; ++k) p[k] = sumsq8(u[k].x, u[k].y, u[k].z, u[k].w);
        } else {
          const uint4* q = reinterpret_cast<const uint4*>(x + t * kH + 32 * lane);
          uint4 u[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) u[k] = q[k];
#pragma unroll
          for (int k = 0; k < 4; ++k) p[k] = sumsq8(u[k].x, u[k].y, u[k].z, u[k].w);
        }
      };
      // rows wave and wave + 4 side by side: independent sum chains
      if (wave + 4 < B) {
        float p0[4], p1[4];
        row_pieces(wave, p0);
        row_pieces(wave + 4, p1);
        const float r0 = rms_inv_from_pieces(p0[0], p0[1], p0[2], p0[3], fz.eps);
        const float r1 = rms_inv_from_pieces(p1[0], p1[1], p1[2], p1[3], fz.eps);
        if (lane == 0) {
          s_rinv[wave] = r0;
          s_rinv[wave + 4] = r1;
        }
      } else if (wave < B) {
        float p0[4];
        row_pieces(wave, p0);
        const float r0 = rms_inv_from_pieces(p0[0], p0[1], p0[2], p0[3], fz.eps);
        if (lane == 0) s_rinv[wave] = r0;
      }
    }
  } else if constexpr (XIN == 0) {
#pragma unroll
    for (int k = 0; k < B; ++k) s_x[sx_pos(k, tid)] = xr[k];
  }
  trace_stamp(ws, 17);
  if constexpr (B > 1) s_mask[tid] = 0u;
  // this call's epoch: the workgroup's counter + 1; layer l > 0 of a stacked
  // launch knows it already (the previous layer's + 1), which saves a memory
  // round trip at the start of each layer
  if (tid == 0) {
    uint32_t* ctr = epoch_ptr(ws, g);
    const uint32_t e = (EPREG ? epoch_reg : load_flag(ctr)) + 1u;
    store_flag(ctr, e);
    s_epoch = e;
  }
  __syncthreads();
  const uint32_t epoch = s_epoch;
  epoch_reg = epoch;
  trace_stamp(ws, 18);
  if constexpr (NORM && B > 1) {
    // the weight piece is the same for every token: widened once
    float nwf[8];
    {
      const uint32_t wu[4] = {nw.x, nw.y, nw.z, nw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nwf[2 * i] = bf16_lo(wu[i]);
        nwf[2 * i + 1] = bf16_hi(wu[i]);
      }
    }
    // a chained layer's x is in LDS already: each thread normalises its own
    // pieces in place (the row sums above read them before the barrier).
    // All reads first, then the arithmetic, then the writes: a store through
    // xn_out between them would keep the compiler from moving the next read
    // ahead of it.
    if constexpr (XIN == 1) {
#pragma unroll
      for (int k = 0; k < B; ++k) xr[k] = s_x[sx_pos(k, tid)];
    }
    float rk[B];
#pragma unroll
    for (int k = 0; k < B; ++k) rk[k] = s_rinv[k];
#pragma unroll
    for (int k = 0; k < B; ++k) xr[k] = rmsnorm8w(xr[k], nwf, rk[k]);
#pragma unroll
    for (int k = 0; k < B; ++k) s_x[sx_pos(k, tid)] = xr[k];
    if (fz.xn_out && g == 0) {
#pragma unroll
      for (int k = 0; k < B; ++k) reinterpret_cast<uint4*>(fz.xn_out)[k * (kH / 8) + tid] = xr[k];
    }
    __syncthreads();
  }
  trace_stamp(ws, 1);
  // W4A4: this wave's maximum |x| of each token (a token's global scale is
  // its amax / 2688), visible to every wave after the barrier behind the
  // router dot
  float(*s_a4max)[4] = nullptr;
  if constexpr (A4) {
    __shared__ float s_a4max_[kMaxB][4];
    s_a4max = s_a4max_;
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const uint32_t u[4] = {xr[t].x, xr[t].y, xr[t].z, xr[t].w};
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[i])), fabsf(bf16_hi(u[i]))));
      m = wave_max(m);
      if (lane == 0) s_a4max[t][wave] = m;
    }
  }
  if constexpr (kXL) {
    // eight rows: each row's wave total in wave_sum's order (the 16-lane
    // group sums, groups 0 + 1 and 2 + 3, then the two pairs), so that every
    // logit is bitwise the one a single-row workgroup computes.  Row j ends
    // in s_part[wave][j].
    const uint4 xv = s_x[sx_pos(0, 64 * wave + lane)];
    uint4 wr8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wr8[j] = s_rw[64 * (4 * j + wave) + lane];
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float d = dot2_bf16(wr8[j].x, xv.x, 0.0f);
      d = dot2_bf16(wr8[j].y, xv.y, d);
      d = dot2_bf16(wr8[j].z, xv.z, d);
      d = dot2_bf16(wr8[j].w, xv.w, d);
      a[j] = group16_sum(d);
    }
    float u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // lanes 0-15, 32-47: row 2q; 16-31, 48-63: row 2q + 1
      float lo = a[2 * q], hi = a[2 * q + 1];
      swap16(lo, hi);
      u[q] = lo + hi;
    }
    float r03 = u[0], r03b = u[1], r47 = u[2], r47b = u[3];
    swap32(r03, r03b);   // rows 0-3 (4-7) in lane groups 0-3
    swap32(r47, r47b);
    r03 = r03 + r03b;
    r47 = r47 + r47b;
    if ((lane & 15) == 0) {
      s_part[wave][lane >> 4] = r03;
      s_part[wave][4 + (lane >> 4)] = r47;
    }
  } else {
    float acc[B];
#pragma unroll
    for (int t = 0; t < B; ++t) {
      const uint4 xv = s_x[sx_pos(t, 64 * wave + lane)];
      float a = dot2_bf16(pre.wr.x, xv.x, 0.0f);
      a = dot2_bf16(pre.wr.y, xv.y, a);
      a = dot2_bf16(pre.wr.z, xv.z, a);
      a = dot2_bf16(pre.wr.w, xv.w, a);
      acc[t] = wave_sum(a);
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < B; ++t) s_part[wave][t] = acc[t];
    }
  }
  __syncthreads();
  // the last wave stores (wave 0 polls first).  Once every 65536 calls the
  // slots of tokens t >= B are stamped too, so no slot is ever 2^32 calls old
  // and a 32-bit tag cannot match a stale value; at that call batch 1 stamps
  // the device-wide slots and larger batches the XCD-local ones.
  {
    const bool wrap = (epoch & 0xFFFFu) == 0u;
    if constexpr (kXL) {
      const int j = tid - (kFusedThreads - 8);
      if (j >= 0) {
        const float v = s_part[0][j] + s_part[1][j] + s_part[2][j] + s_part[3][j];
        put_slot_xcd(lxmine + 8 * (g >> 3) + j, v, epoch);
      }
    } else if (wrap && tid < 8) {
      put_slot_xcd(lxmine + 8 * (g >> 3) + tid, 0.0f, epoch);
    }
    const int nt = wrap ? kMaxB : (kXL ? 0 : B);
    const int i = tid - (kFusedThreads - kMaxB * kLogitReps), t = i % kMaxB, r = i / kMaxB;
    if (i >= 0 && t < nt) {
      const float v =
          !kXL && t < B ? s_part[0][t] + s_part[1][t] + s_part[2][t] + s_part[3][t] : 0.0f;
      put_slot(lslots + r * (kSlotLogitRep / 8) + t * kE + g, v, epoch);
    }
  }
  trace_stamp(ws, 2);
  // x0 again, normalised (for the gate/up products; read only now, so that
  // these reads do not stand before the router's in LDS's in-order queue)
  if constexpr (NORM && B == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = s_x[sx_pos(0, 4 * lane + i)];
      x0[4 * i] = v.x; x0[4 * i + 1] = v.y; x0[4 * i + 2] = v.z; x0[4 * i + 3] = v.w;
    }
  }
  // W4A4: x quantised in place (the router has read it; every workgroup
  // quantises all of x, each thread its own piece of every token, read back
  // from LDS so that one copy of the quantiser's code serves them all); at
  // B = 1 x0 is reread
  float* s_gx = nullptr;
  if constexpr (A4) {
    __shared__ float s_gx_[kMaxB];
    s_gx = s_gx_;
    auto x_global = [&](int t) __attribute__((always_inline)) {
      return __fdiv_rn(fmaxf(fmaxf(s_a4max[t][0], s_a4max[t][1]),
                             fmaxf(s_a4max[t][2], s_a4max[t][3])), 2688.0f);
    };
    if constexpr (B == 1) {
      const float g = x_global(0);
      if (tid == 0) s_gx[0] = g;
      s_x[sx_pos(0, tid)] = a4_quant_piece(s_x[sx_pos(0, tid)], g);
    } else {
      // two tokens per round, their serial chains side by side (an odd last
      // token pairs with itself: the same value is written twice)
#pragma unroll 1
      for (int t = 0; t < B; t += 2) {
        const int t1 = t + 1 < B ? t + 1 : t;
        const float g0 = x_global(t), g1 = x_global(t1);
        if (tid == 0) {
          s_gx[t] = g0;
          s_gx[t1] = g1;
        }
        const uint4 p0 = s_x[sx_pos(t, tid)], p1 = s_x[sx_pos(t1, tid)];
        const uint4 q0 = a4_quant_piece(p0, g0), q1 = a4_quant_piece(p1, g1);
        s_x[sx_pos(t, tid)] = q0;
        s_x[sx_pos(t1, tid)] = q1;
      }
    }
    trace_stamp(ws, 22);
    __syncthreads();
    trace_stamp(ws, 23);
    if constexpr (B == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = s_x[sx_pos(0, 4 * lane + i)];
        x0[4 * i] = v.x; x0[4 * i + 1] = v.y; x0[4 * i + 2] = v.z; x0[4 * i + 3] = v.w;
      }
    }
  }
  if (smask) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      gateup_compute<B, FMT, A4>(pre.scg[s], pre.scu[s], sh_sg[s], sh_su[s], smask, wave >> 1, s_x,
                                 x0, lane, &s_hsh[s][wave & 1][0], s_gx);
  }
  trace_stamp(ws, 3);

  // ---------------------------------------------------------------- step B
  // top-6 per token (wave t % 4 takes token t), repeated identically in every
  // workgroup; sigmoid scores of the chosen six renormalised to sum to 1
  __shared__ float s_sl[kK];                  // B = 1: the six chosen logits, descending
  __shared__ int s_si[kK];                    //        and their experts
  if constexpr (B == 1) {
    // one token: its six experts are the routed entries, each with one h
    // pair, so wave 0 orders them by id (rank by counting) and writes the
    // entry tables itself, with no token masks and no barrier in between.
    // The routing weights are computed after the first gate/up loads have
    // gone out (step C needs them, the loads do not).
    if (wave == 0) {
      float v[1][4];
      {
        uint32_t lw[4];
        wait_slots_u32_p2<4>(kXL ? lxmine + lane
                                 : lslots + (g % kLogitReps) * (kSlotLogitRep / 8) + lane,
                             64, epoch, lw, &ctl->err, kErrLogits);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[0][q] = __builtin_bit_cast(float, lw[q]);
      }
      trace_stamp(ws, 4);
      int my_ids[1];
      float my_ls[1];
      wave_top6<1>(v, lane, my_ids, my_ls);
      const int my_id = my_ids[0];
      const float my_l = my_ls[0];
      trace_stamp(ws, 15);
      int rank = 0;
#pragma unroll
      for (int j = 0; j < kK; ++j) rank += __builtin_amdgcn_readlane(my_id, j) < my_id ? 1 : 0;
      if (lane < kK) {
        s_sl[lane] = my_l;
        s_si[lane] = my_id;
        s_act[rank] = my_id;
        s_amask[rank] = 1u;
        s_pair0[rank] = rank;
      }
      if (lane == 0) {
        s_nr = kK;
        s_act[kK] = 0;
        s_amask[kK] = 1u;
        s_pair0[kK] = kK;
      }
    }
    trace_stamp(ws, 5);
  } else {
  // token t's choices: sigmoid scores of the six renormalised to sum to 1
  auto finish = [&](int t, int my_id, float my_l) __attribute__((always_inline)) {
    const float s = 1.0f / (1.0f + expf(-my_l));
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kK; ++j) sum += readlane_f32(s, j);
    if (lane < kK) {
      const float wgt = s / sum;
      atomicOr(&s_mask[my_id], 1u << t);
      s_wfull[my_id][t] = wgt;
      if (g == 0) {
        if (ids_out) ids_out[t * kK + lane] = my_id;
        if (w_out) w_out[t * kK + lane] = wgt;
      }
    }
  };
  const uint64_t* lrep = lslots + (g % kLogitReps) * (kSlotLogitRep / 8) + lane;
  if (wave + 4 < B) {          // two tokens, wave and wave + 4: selected together
    float v[2][4];
    wait_logits_p2(lrep + wave * kE, epoch, v[0], &ctl->err);
    wait_logits_p2(lrep + (wave + 4) * kE, epoch, v[1], &ctl->err);
    trace_stamp(ws, 4);
    int my_id[2];
    float my_l[2];
    wave_top6<2>(v, lane, my_id, my_l);
    trace_stamp(ws, 19);
    // finish() for both tokens, the two chains side by side (same arithmetic)
    const float s0 = 1.0f / (1.0f + expf(-my_l[0])), s1 = 1.0f / (1.0f + expf(-my_l[1]));
    float sum0 = 0.0f, sum1 = 0.0f;
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      sum0 += readlane_f32(s0, j);
      sum1 += readlane_f32(s1, j);
    }
    if (lane < kK) {
      const float w0 = s0 / sum0, w1 = s1 / sum1;
      atomicOr(&s_mask[my_id[0]], 1u << wave);
      atomicOr(&s_mask[my_id[1]], 1u << (wave + 4));
      s_wfull[my_id[0]][wave] = w0;
      s_wfull[my_id[1]][wave + 4] = w1;
      if (g == 0) {
        if (ids_out) {
          ids_out[wave * kK + lane] = my_id[0];
          ids_out[(wave + 4) * kK + lane] = my_id[1];
        }
        if (w_out) {
          w_out[wave * kK + lane] = w0;
          w_out[(wave + 4) * kK + lane] = w1;
        }
      }
    }
  } else if (wave < B) {
    float v[1][4];
    wait_logits_p2(lrep + wave * kE, epoch, v[0], &ctl->err);
    trace_stamp(ws, 4);
    int my_id[1];
    float my_l[1];
    wave_top6<1>(v, lane, my_id, my_l);
    finish(wave, my_id[0], my_l[0]);
  }
  trace_stamp(ws, 5);
  __syncthreads();
  if (wave == 0) {            // entries: touched experts in ascending id, then the shared one
    int base = 0;
    unsigned mq[4];             // the four reads first: one LDS round trip, not four
#pragma unroll
    for (int q = 0; q < 4; ++q) mq[q] = s_mask[64 * q + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 64 * q + lane;
      const unsigned m = mq[q];
      const uint64_t bal = __ballot(m != 0u);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (m != 0u) {
        s_act[pos] = e;
        s_amask[pos] = m;
      }
      base += __popcll(bal);
    }
    // first h pair of each entry: exclusive prefix of the token counts (0..8),
    // bit by bit over ballots
    const unsigned ma = lane < base ? s_amask[lane] : 0u;
    const int cnt = __popc(ma);
    int excl = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint64_t bb = __ballot((cnt >> b) & 1);
      excl += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u)) << b;
    }
    if (lane < base) s_pair0[lane] = excl;
    if (lane == 0) {
      s_nr = base;
      s_act[base] = 0;
      s_amask[base] = (1u << B) - 1u;
      s_pair0[base] = kK * B;
    }
    if constexpr (kGuWeight > 0) {
      // this workgroup's range [T0, T1) of the nr * 512 row pairs: entry a
      // weighs 512 (kGuWeight + n_a); the cuts at g / 256 and (g + 1) / 256
      // of the total weight, rounded down to an even row
      const int wr = lane < base ? kGuWeight + cnt : 0;      // weight per row pair (< 16)
      int excl_r = 0;                                         // weight of the entries before
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint64_t bb = __ballot((wr >> b) & 1);
        excl_r += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u)) << b;
      }
      const int tot = __builtin_amdgcn_readlane(excl_r + wr, 63) * kI;
      auto cut = [&](int gg) -> int {
        if (gg >= kFusedGrid) return base * kI;
        const int tg = (int)(((long long)gg * tot) >> 8);     // weight before the cut
        const int excl_w = excl_r * kI;
        const uint64_t bal = __ballot(lane < base && tg >= excl_w && tg < excl_w + wr * kI);
        if (!bal) return base * kI;
        const int a = (int)__builtin_ctzll(bal);
        const int ew = __builtin_amdgcn_readlane(excl_w, a), aw = __builtin_amdgcn_readlane(wr, a);
        return (a * kI + (tg - ew) / aw) & ~1;
      };
      const int c0 = cut(g), c1 = cut(g + 1);
      if (lane == 0) {
        s_t01[0] = c0;
        s_t01[1] = c1;
      }
    }
  }
  }
  __syncthreads();
  const int nr = s_nr;
  trace_stamp(ws, 6);

  // routed gate/up: the nr * 512 row pairs are cut into 256 contiguous
  // ranges, one per workgroup; wave w takes T0 + w, T0 + w + 4, ... in
  // batches of kTB, the next batch in flight while one computes
  const int T = nr * kI;
  const bool weighted = B > 1 && kGuWeight > 0;
  const int T0 = weighted ? s_t01[0] : (int)(((long long)g * T) >> 8);
  const int T1 = weighted ? s_t01[1] : (int)(((long long)(g + 1) * T) >> 8);
  // step-C work of this wave: routed entries a = wsel + 4 k (and the shared
  // expert's tokens wave, wave + 4); the first kDepthC entries' down rows are
  // fetched behind the first gate/up batch
  const int wsel = (wave + 3) & 3;
  // Unconditional, like the gate/up loads: an entry past the last (there are
  // always at least kK) reads the last one's rows again and run_set drops
  // it.  Under a branch these loads would make the compiler wait for every
  // load in flight at the next barrier.
  auto load_entry = [&](Chunk<FMT> (&dst)[2], int a) {
    const size_t ee = (size_t)s_act[a < nr ? a : nr - 1];
#pragma unroll
    for (int r = 0; r < 2; ++r) dst[r].load_dn(routed, ee, g * kRowsPerWg + 2 * grp4 + r, c16);
  };
  Chunk<FMT> dbuf[kDepthC][2];
  {
    Chunk<FMT> cg[2][kTB], cu[2][kTB];
    // Loads are unconditional: a slot past the range reads the range's last
    // row again (a cache hit; run_batch drops its sums).  A load under a
    // branch would leave the compiler unsure how many loads are in flight,
    // and it would then wait for all of them before the next batch goes out.
    auto load_batch = [&](Chunk<FMT> (&bg)[kTB], Chunk<FMT> (&bu)[kTB], int j0) {
#pragma unroll
      for (int q = 0; q < kTB; ++q) {
        const int s0 = T0 + wave + 4 * (j0 + q), s = s0 < T1 ? s0 : T1 - 1;
        const size_t ee = (size_t)s_act[s / kI];
        bg[q].load_gu(routed, ee, 0, s % kI, lane);
        bu[q].load_gu(routed, ee, 1, s % kI, lane);
      }
    };
    // a batch for each token any of its row pairs uses: the 2 kTB gate and up
    // partial sums reduced together; gate/up of pair q land in lanes
    // 16 q .. 16 q + 7 / 16 q + 8 .. 16 q + 15, lane 16 q writes h
    auto run_batch = [&](const Chunk<FMT> (&bg)[kTB], const Chunk<FMT> (&bu)[kTB], int j0) {
      unsigned mq[kTB], um = 0u;
      float sgq[kTB], suq[kTB];
#pragma unroll
      for (int q = 0; q < kTB; ++q) {
        const int s = T0 + wave + 4 * (j0 + q);
        mq[q] = 0u;
        sgq[q] = suq[q] = 0.0f;
        if (s < T1) {
          const int a = s / kI;
          mq[q] = s_amask[a];
          sgq[q] = s_gs[a][0];
          suq[q] = s_gs[a][1];
          um |= mq[q];
        }
      }
      if (um == 0u) return;
      const int qme = lane >> 4;                     // the row pair this lane may write
      unsigned mme = 0u;
      float sgme = 0.0f, sume = 0.0f;
#pragma unroll
      for (int q = 0; q < kTB; ++q)
        if (qme == q) {
          mme = mq[q];
          sgme = sgq[q];
          sume = suq[q];
        }
      const int ime = T0 + wave + 4 * (j0 + qme) - T0;
      auto token = [&](int t, const uint32_t (&xw)[16]) __attribute__((always_inline)) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = q < kTB ? bg[q < kTB ? q : 0].dot_x(xw) : 0.0f;
          v[2 * q + 1] = q < kTB ? bu[q < kTB ? q : 0].dot_x(xw) : 0.0f;
        }
        const float z = wave_sum8(v, lane);
        const float zu = dpp_f32<0x128>(z);
        if ((lane & 15) == 0 && ((mme >> t) & 1u)) {
          if constexpr (A4)
            s_hout[ime][t] = silu_mul(z * sgme * s_gx[t], zu * sume * s_gx[t]);
          else
            s_hout[ime][t] = silu_mul(z * sgme, zu * sume);
        }
      };
      if constexpr (B == 1) {
        token(0, x0);
      } else {
        // the batch's tokens (a wave-uniform mask) in a rolled loop: unrolled
        // over 8 tokens, the five batch bodies of this loop came to most of
        // the kernel's code, more than the instruction cache holds
#pragma unroll 1
        for (unsigned mm = __builtin_amdgcn_readfirstlane(um); mm != 0u; mm &= mm - 1u) {
          const int t = __builtin_ctz(mm);
          uint32_t xw[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = s_x[sx_pos(t, 4 * lane + i)];
            xw[4 * i] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
          }
          token(t, xw);
        }
      }
    };
    // the routed entries' tensor scales: one thread each, fetched beside the
    // first weights and parked in LDS (no wave waits on them in its loop)
    const bool gs_mine = tid < 3 * nr;
    float gsv = 1.0f;
    if (gs_mine) gsv = Chunk<FMT>::gscale(routed, (size_t)s_act[tid / 3], tid % 3);
    load_batch(cg[0], cu[0], 0);
    // the first kDepthC entries' down rows of step C, behind the first batch
    // (at B = 1 after the h publish: the wait for the tensor scales below
    // waits for every load before it)
    if constexpr (!kLateDown) {
#pragma unroll
      for (int q = 0; q < kDepthC; ++q) load_entry(dbuf[q], wsel + 4 * q);
    }
    if constexpr (B == 1) {
      // the routing weights of the one token: sigmoid of the six logits in
      // descending order, renormalised (the same sums as every other path)
      if (wave == 0) {
        const float l = s_sl[lane < kK ? lane : 0];
        const float sc = 1.0f / (1.0f + expf(-l));
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < kK; ++j) sum += readlane_f32(sc, j);
        if (lane < kK) s_wfull[s_si[lane]][0] = sc / sum;
      }
    }
    if (gs_mine) s_gs[tid / 3][tid % 3] = gsv;
    __syncthreads();
    // this wave's row pairs T0 + wave + 4 j, j < nj; the loop runs while a
    // batch after the two in hand exists, the last one or two are peeled
    const int nj = T1 - T0 > wave ? (T1 - T0 - wave + 3) >> 2 : 0;
    int j0 = 0;
    for (; j0 + 2 * kTB < nj; j0 += 2 * kTB) {
      load_batch(cg[1], cu[1], j0 + kTB);
      run_batch(cg[0], cu[0], j0);
      load_batch(cg[0], cu[0], j0 + 2 * kTB);
      run_batch(cg[1], cu[1], j0 + kTB);
    }
    if (j0 + kTB < nj) {
      load_batch(cg[1], cu[1], j0 + kTB);
      run_batch(cg[0], cu[0], j0);
      run_batch(cg[1], cu[1], j0 + kTB);
    } else {
      run_batch(cg[0], cu[0], j0);
    }
  }
  trace_stamp(ws, 7);
  // write this workgroup's h to its pairs: shared (6 B + t, rows 2g, 2g + 1),
  // routed (pair0[a] + rank of t in the entry's tokens, row), consecutive
  // threads on consecutive rows
  __syncthreads();
  trace_stamp(ws, 13);
  // Every load of this wave has landed by now (the gate/up rows are used;
  // the rest went out long ago), but the compiler cannot count the h stores
  // below (a data-dependent loop): if a load were still outstanding on its
  // books, reusing its register after the stores would wait for the stores'
  // acknowledgements too.  Retire the loads here, before any store.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  // Once every 65536 epochs every h slot not written by this call is stamped
  // (workgroup g: slot g of each such pair), as the logit slots are, so that
  // no slot is ever 2^32 epochs old.
  if ((epoch & 0xFFFFu) == 0u) {
    for (int p = (kTagH ? kPairs : 0) + tid; p < kMaxB * (kK + kMaxShared); p += kFusedThreads)
      put_slot_u32(hslots + (size_t)p * kHSlots + g, 0u, epoch);
  }
  if constexpr (kTagH) {
    // h as tagged slots: slot k of a pair holds its rows 2 k, 2 k + 1 (a
    // workgroup's rows come in pairs: its range starts and ends on even rows)
    auto pack = [](float a, float b) {
      return (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
    };
    if (tid < NS * B) {   // shared expert s = tid / B, token t = tid % B: pair kK B + tid
      const int s = tid / B, t = tid - s * B;
      put_slot_u32(hslots + (size_t)(kK * B + tid) * kHSlots + g,
                   pack(s_hsh[s][0][t], s_hsh[s][1][t]), epoch);
    }
    const int nloc2 = (T1 - T0) >> 1;
    if constexpr (B == 1) {
      // one token: routed entry a is h pair a (every entry holds the token),
      // so no table lookups stand between the values and their store
      for (int j = tid; j < nloc2; j += kFusedThreads) {
        const int s = T0 + 2 * j;
        put_slot_u32(hslots + (size_t)(s / kI) * kHSlots + (s % kI) / 2,
                     pack(s_hout[2 * j][0], s_hout[2 * j + 1][0]), epoch);
      }
    } else {
      for (int idx = tid; idx < nloc2 * B; idx += kFusedThreads) {
        const int t = idx / nloc2, j = idx - t * nloc2;
        const int s = T0 + 2 * j, a = s / kI;
        const unsigned m = s_amask[a];
        if ((m >> t) & 1u)
          put_slot_u32(hslots + (size_t)(s_pair0[a] + __popc(m & ((1u << t) - 1u))) * kHSlots +
                           (s % kI) / 2,
                       pack(s_hout[2 * j][t], s_hout[2 * j + 1][t]), epoch);
      }
    }
    trace_stamp(ws, 14);
    // count in at once: the counters only tell the readers when to start
    // copying, each slot's tag tells them whether it has arrived (the
    // counters advance in every mode: a later call of another batch size
    // waits on them)
    __syncthreads();
    if (tid < kBankReps)
      __hip_atomic_fetch_add(hready_bank(ws, tid, g % kHBanks), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if (tid < NS * B) {   // shared expert s, rows 2 g and 2 g + 1, token t: pair kK B + s B + t
      const int s = tid / B, t = tid % B;
      store_coherent_u32(
          reinterpret_cast<uint32_t*>(hbuf + (size_t)(kK * B + s * B + t) * kI + 2 * g),
          f32x2_to_bf16x2_rne(s_hsh[s][0][t], s_hsh[s][1][t]));
    }
    {
      // rows in pairs (a workgroup's range starts and ends on even rows, and
      // a pair never straddles two entries): one 4-byte store per pair
      const int nloc2 = (T1 - T0) >> 1;
      for (int idx = tid; idx < nloc2 * B; idx += kFusedThreads) {
        const int t = idx / nloc2, j = idx - t * nloc2;
        const int s = T0 + 2 * j, a = s / kI;
        const unsigned m = s_amask[a];
        if ((m >> t) & 1u)
          store_coherent_u32(
              reinterpret_cast<uint32_t*>(hbuf + (size_t)(s_pair0[a] + __popc(m & ((1u << t) - 1u))) * kI +
                                          (s % kI)),
              f32x2_to_bf16x2_rne(s_hout[2 * j][t], s_hout[2 * j + 1][t]));
      }
    }
    // publish: wait for this workgroup's h stores, then count in on bank g % 64
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    trace_stamp(ws, 14);
    __syncthreads();
    if (tid < kBankReps)
      __hip_atomic_fetch_add(hready_bank(ws, tid, g % kHBanks), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  trace_stamp(ws, 8);

  // ---------------------------------------------------------------- step C
  // The next kDepthC entries' down rows go out now (not earlier: the h
  // stores above must not wait behind them), so they arrive during the wait.
  // Wave 3 polls, and issues its rows after the wait (its polls would
  // otherwise queue behind them).  Every bank of copy g % kBankReps must
  // reach 4 * epoch (each bank gains 4 per call).
  Chunk<FMT> dbuf2[kDepthC][2];
  auto prefetch = [&]() {
#pragma unroll
    for (int q = 0; q < kDepthC; ++q) load_entry(dbuf2[q], wsel + 4 * (kDepthC + q));
  };
  if constexpr (kLateDown) {   // HBM is idle while the h-ready counters fill
#pragma unroll
    for (int q = 0; q < kDepthC; ++q) load_entry(dbuf[q], wsel + 4 * q);
  }
  constexpr bool kPollCounters = !(kTagH && kHDirect);
  if (!kPollCounters || wave != 3) prefetch();
  if (kPollCounters && wave == 3) {
    const uint32_t want = (uint32_t)(kFusedGrid / kHBanks) * epoch;
    const uint32_t* bank = hready_bank(ws, g % kBankReps, lane);
    // first four polls with two in flight (as wait_slots_u32_p2), then the loop
    bool ready;
    {
      const uint32_t c0 = load_flag(bank), c1 = load_flag(bank);
      ready = __ballot(c0 != want) == 0;
      if (!ready) {
        const uint32_t c2 = load_flag(bank);
        ready = __ballot(c1 != want) == 0;
        if (!ready) {
          const uint32_t c3 = load_flag(bank);
          ready = __ballot(c2 != want) == 0 || __ballot(c3 != want) == 0;
        }
      }
    }
    for (int spin = 0; !ready; ++spin) {
      const uint32_t v = load_flag(bank);
      if (__ballot(v != want) == 0) break;
      if (spin > kSpinLimit) {
        if (lane == 0)
          __hip_atomic_fetch_or(&ctl->err, kErrHReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    prefetch();
  }
  // (with direct polling no wave waits for another here: every LDS use
  // before the h copy ended at the barrier behind the gate/up rows)
  if constexpr (kPollCounters) __syncthreads();
  // The next layer's router rows (XCD-local logits) go to LDS behind the
  // down rows and arrive while the h slots fill (the barrier behind the h
  // copy waits for them).
  if constexpr (kXL) router_rows_to_lds(next.rw, g, wave, lane, s_rw);
  trace_stamp(ws, 9);

  if constexpr (kTagH) {
    // all 7 B h pairs into LDS: thread tid reads slot tid of every pair,
    // polling until each carries this call's epoch, and puts its two values
    // where load_h expects them (uint4 c of a pair at 16 (c % 4) + c / 4)
    uint32_t hv[kPairs];
    if constexpr (kXL)   // the next layer's router rows are in flight to LDS
      wait_slots_u32<kPairs>(hslots + tid, (int)kHSlots, epoch, hv, &ctl->err, kErrHReady);
    else
      wait_slots_u32_p2<kPairs>(hslots + tid, (int)kHSlots, epoch, hv, &ctl->err, kErrHReady);
    uint32_t* s_h32 = reinterpret_cast<uint32_t*>(s_xh);
    const int c = tid >> 2, wd = tid & 3;
#pragma unroll
    for (int p = 0; p < kPairs; ++p) s_h32[4 * (p * 64 + 16 * (c & 3) + (c >> 2)) + wd] = hv[p];
  } else {
  // all 7 B h pairs of the call into LDS: 16-byte device-coherent loads
  // (device-scope bit) straight to LDS, no registers, all in flight at once:
  // wave w takes pairs w, w + 4, ...; lane i brings the piece that belongs
  // at position i of the pair (uint4 c of a pair sits at 16 (c % 4) + c / 4,
  // where load_h expects it).  The barrier below waits for them.
  {
    const uint8_t* hb = reinterpret_cast<const uint8_t*>(hbuf);
    const int c = 4 * (lane & 15) + (lane >> 4);
#pragma unroll
    for (int k = 0; k < (kPairs + 3) / 4; ++k) {
      const int p = wave + 4 * k;
      if (p < kPairs)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(hb + (size_t)p * (2 * kI) + 16 * c),
            (__attribute__((address_space(3))) void*)(s_xh + 64 * p), 16, 0, kCpolDevice);
    }
  }
  }
  __syncthreads();
  trace_stamp(ws, 10);
  // W4A4: every h pair quantised in place with its own global (amax / 2688):
  // wave w takes pairs w, w + 4, ..., lane l its 16-byte chunk l (elements 8 l
  // .. 8 l + 7, at LDS position 16 (l % 4) + l / 4 of the pair), so that the
  // lanes of a 16-element block are a lane pair
  float* s_gh = nullptr;
  if constexpr (A4) {
    __shared__ float s_gh_[kPairs];
    s_gh = s_gh_;
    // pairs w + 8 r and w + 8 r + 4 in one round, their serial chains side
    // by side (without a second pair the first is taken twice: the same
    // values are written twice)
    auto h_global = [&](uint4 v) __attribute__((always_inline)) {
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[i])), fabsf(bf16_hi(u[i]))));
      return __fdiv_rn(wave_max(m), 2688.0f);
    };
#pragma unroll 1
    for (int r = 0; r < (kPairs + 7) / 8; ++r) {
      const int pa = wave + 8 * r;
      if (pa < kPairs) {
        const int pb = pa + 4 < kPairs ? pa + 4 : pa;
        uint4* ca = s_xh + pa * 64 + 16 * (lane & 3) + (lane >> 2);
        uint4* cb = s_xh + pb * 64 + 16 * (lane & 3) + (lane >> 2);
        const uint4 va = *ca, vb = *cb;
        const float ga = h_global(va), gb = h_global(vb);
        if (lane == 0) {
          s_gh[pa] = ga;
          s_gh[pb] = gb;
        }
        const uint4 qa = a4_quant_piece(va, ga), qb = a4_quant_piece(vb, gb);
        *ca = qa;
        *cb = qb;
      }
    }
    trace_stamp(ws, 20);
    __syncthreads();
    trace_stamp(ws, 21);
  }
  // The next layer's router row and shared gate/up rows (registers free
  // since step A): no load of this layer is issued after this point when
  // every routed entry's down rows are already in flight, so these wait
  // behind nothing and arrive while this layer finishes.
  if constexpr (kPfEarly) load_pre_gateup<B, FMT, NS, !kXL>(pre, next.rw, next.shared, g, wave, lane);

  float acc[2][B], accs[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int t = 0; t < B; ++t) acc[r][t] = 0.0f;
    accs[r][0] = accs[r][1] = 0.0f;
  }
  // shared experts in order, tokens wave and wave + 4
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float gl = sh_sd[s];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = wave + 4 * j;
      if (t < B) {
        uint32_t h[16];
        load_h(s_h, kK * B + s * B + t, c16, h);
        float d0 = pre.dsh[s][0].dot_x(h), d1 = pre.dsh[s][1].dot_x(h);
        if constexpr (A4) {
          d0 *= s_gh[kK * B + s * B + t];
          d1 *= s_gh[kK * B + s * B + t];
        }
        accs[0][j] = __builtin_fmaf(gl, d0, accs[0][j]);
        accs[1][j] = __builtin_fmaf(gl, d1, accs[1][j]);
      }
    }
  }
  if constexpr (kPfEarly) load_pre_down<FMT, NS>(pre, next.shared, g, lane);  // the next layer's
  // routed entries of this wave in order, two sets of kDepthC in flight
  const int n_mine = nr > wsel ? (nr - wsel + 3) >> 2 : 0;
  auto run_set = [&](const Chunk<FMT> (&buf)[kDepthC][2], int k0) {
#pragma unroll
    for (int q = 0; q < kDepthC; ++q) {
      if (k0 + q < n_mine) {
        const int a = wsel + 4 * (k0 + q);
        const int e = s_act[a];
        down_entry<B, FMT, A4>(buf[q], s_gs[a][2], s_amask[a],
                               &s_wfull[e][0], s_h, s_pair0[a], c16, acc, s_gh);
      }
    }
  };
  if constexpr (kPrefetchNext<B, FMT>) {   // every entry of this wave is in the two sets
    run_set(dbuf, 0);
    run_set(dbuf2, kDepthC);
  } else {
    // loads in the loop are unconditional (as in the gate/up loop): an entry
    // past this wave's last reads the last one's rows again
    auto load_set = [&](Chunk<FMT> (&buf)[kDepthC][2], int k) {
#pragma unroll
      for (int q = 0; q < kDepthC; ++q) {
        const int kk = k + q < n_mine ? k + q : n_mine - 1;
        const size_t ee = (size_t)s_act[wsel + 4 * kk];
#pragma unroll
        for (int r = 0; r < 2; ++r) buf[q][r].load_dn(routed, ee, g * kRowsPerWg + 2 * grp4 + r, c16);
      }
    };
    int k0 = 0;
    for (; k0 + 2 * kDepthC < n_mine; k0 += 2 * kDepthC) {
      run_set(dbuf, k0);
      load_set(dbuf, k0 + 2 * kDepthC);
      run_set(dbuf2, k0 + kDepthC);
      load_set(dbuf2, k0 + 3 * kDepthC);
    }
    if constexpr (kPfLate) {     // the next layer's step-A rows, behind these
      load_pre_gateup<B, FMT, NS, !kXL>(pre, next.rw, next.shared, g, wave, lane);
      load_pre_down<FMT, NS>(pre, next.shared, g, lane);
    }
    run_set(dbuf, k0);
    run_set(dbuf2, k0 + kDepthC);
  }
  trace_stamp(ws, 11);
  // reduce over the 16 lanes of each row group, then over the waves in a
  // fixed order; the shared expert's term of token t comes from wave t % 4
  __shared__ float s_red[4][kRowsPerWg][kMaxB];
  __shared__ float s_redsh[4][kRowsPerWg][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int t = 0; t < B; ++t) acc[r][t] = group16_sum(acc[r][t]);
    accs[r][0] = group16_sum(accs[r][0]);
    accs[r][1] = group16_sum(accs[r][1]);
  }
  if (c16 == 0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int t = 0; t < B; ++t) s_red[wave][2 * grp4 + r][t] = acc[r][t];
      s_redsh[wave][2 * grp4 + r][0] = accs[r][0];
      s_redsh[wave][2 * grp4 + r][1] = accs[r][1];
    }
  }
  __syncthreads();
  if (tid < kRowsPerWg * B) {
    const int r8 = tid / B, t = tid % B;
    float y = (s_red[0][r8][t] + s_red[1][r8][t]) + (s_red[2][r8][t] + s_red[3][r8][t]);
    y += s_redsh[t & 3][r8][t >> 2];
    if constexpr (RES != 0) y += resid;
    const uint16_t o = f32_to_bf16_rne(y);
    out[(size_t)t * kH + g * kRowsPerWg + r8] = o;
    if constexpr (XOUT) {
      resid_reg = __builtin_bit_cast(float, (uint32_t)o << 16);
      // this workgroup's rows of the next layer's x, two rows to a slot, in
      // every copy: rows 2 pp and 2 pp + 1 of token t are threads tid and
      // tid + B of wave 0, so the even row's thread publishes both
      const uint32_t o1 = __shfl_down((uint32_t)o, B);
      if ((r8 & 1) == 0) {
        const uint32_t v = (uint32_t)o | (o1 << 16);
#pragma unroll
        for (int rep = 0; rep < kXReps; ++rep)
          put_slot_u32(xslots + rep * (kSlotXRep / 8) + t * (kH / 2) + g * (kRowsPerWg / 2) +
                           (r8 >> 1),
                       v, epoch);
      }
    }
  }
  if constexpr (XOUT && B < kMaxB) {
    // once every 65536 epochs the slots of the tokens t >= B are stamped too,
    // as the logit slots are
    if ((epoch & 0xFFFFu) == 0u) {
      constexpr int n4 = (kMaxB - B) * (kRowsPerWg / 2);
      for (int i = tid; i < n4 * kXReps; i += kFusedThreads) {
        const int rep = i / n4, j = i - rep * n4;
        put_slot_u32(xslots + rep * (kSlotXRep / 8) + (B + j / (kRowsPerWg / 2)) * (kH / 2) +
                         g * (kRowsPerWg / 2) + j % (kRowsPerWg / 2),
                     0u, epoch);
      }
    }
  }
  if constexpr (B == 1) {
    // the routing of the call, once nothing of the layer is loaded any more
    if (g == 0 && tid < kK) {
      if (ids_out) ids_out[tid] = s_si[tid];
      if (w_out) w_out[tid] = s_wfull[s_si[tid]][0];
    }
  }
  trace_stamp(ws, 12);
  trace_flush(ws);
}

template <int B, int FMT, bool NORM, bool RESID, int NS = 1, bool A4 = false>
__global__ __launch_bounds__(kFusedThreads, 1) void k_decode_fused(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ rw, ExpertsDev routed,
    ExpertsDev shared, uint16_t* __restrict__ out, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, uint8_t* __restrict__ ws, FuseDev fz) {
  StepAPre<FMT, NS> pre;
  uint32_t epoch = 0;
  float resid = 0.0f;
  decode_layer<B, FMT, NORM, RESID ? 1 : 0, 0, false, 0, false, NS, A4>(
      x, rw, routed, shared, out, ids_out, w_out, ws, fz, pre, LayerDev{}, epoch, resid);
}

// A stack of L layers in one launch, one after another: every workgroup
// runs layer l + 1 as soon as it has finished its part of layer l (the
// layers read the same x), so its first loads of layer l + 1 overlap the
// other workgroups' tail of layer l, and the loads of layer l + 1 that
// depend on neither x nor its routing go out inside layer l's step C (see
// kPrefetchNext).  The hand-over protocol already orders
// consecutive layers: a workgroup can only publish layer l + 1's logits after
// it has read all of layer l's, and only write layer l + 1's h after every
// workgroup has published layer l + 1's logits, i.e. after each has copied
// layer l's h.  So the per-layer epochs are all the kernel needs, and the
// launch gap between layers disappears (the pages hide it with programmatic
// dependent launch).
template <int B, int FMT>
__global__ __launch_bounds__(kFusedThreads, 1) void k_decode_stack(
    const uint16_t* __restrict__ x, const LayerDev* __restrict__ layers, int L,
    uint16_t* __restrict__ out, int32_t* __restrict__ ids_out, uint8_t* __restrict__ ws) {
  StepAPre<FMT> pre;
  // the last layer "prefetches" its own rows again (cache hits, unused), so
  // that every layer body has the same static load count
  uint32_t epoch = 0;
  float resid = 0.0f;
  auto layer = [&](auto pf, auto epreg, int l) __attribute__((always_inline)) {
    const LayerDev d = layers[l], dn = layers[l + 1 < L ? l + 1 : l];
    decode_layer<B, FMT, false, 0, decltype(pf)::value, decltype(epreg)::value, 0, false>(
        x, d.rw, d.routed, d.shared, out + (size_t)l * B * kH,
        ids_out ? ids_out + (size_t)l * B * kK : nullptr, nullptr, ws, FuseDev{}, pre, dn, epoch,
        resid);
  };
  layer(std::integral_constant<int, 1>{}, std::false_type{}, 0);
  for (int l = 1; l < L; ++l) {
    __syncthreads();
    layer(std::integral_constant<int, 2>{}, std::true_type{}, l);
  }
}


// A chained residual stack of L layers in one launch: x_0 = x and
//   x_{l+1} = x_l + layer_l(norm_l(x_l)),   out[l] = x_{l+1},
// norm_l the pre-MoE RMSNorm with weight norm_w[l] when NORM (the stack of
// pre-norm decoder layers, "Day-0 Support for Flint on vLLM", Model
// architecture; here the MoE layers only).  Each layer is the fused layer
// with its input normalised and its input added as the residual: it equals
// moe_decode_forward_ex on (x_l, norm_w[l], residual x_l) bit for bit.  The
// dependency between layers is kept: a workgroup publishes its rows of
// x_{l+1} as tagged slots (epoch of layer l) and every workgroup waits for
// all of them before layer l + 1 reads x.  Only the weight loads of layer
// l + 1 that depend on neither its input nor its routing (router row, the
// shared expert's rows) go out early, inside layer l's step C, as the pages'
// low-latency path loads the next kernel's weights early under programmatic
// dependent launch (Optimization section, Fig. 3).  The residual of a
// workgroup's output rows is its own output of the previous layer, kept in a
// register.  Ordering: a workgroup overwrites the x slots only at the end of
// layer l + 1, after layer l + 1's logit exchange, which every workgroup
// joins only after it has read layer l's x from them.
template <int B, int FMT, bool NORM>
__global__ __launch_bounds__(kFusedThreads, 1) void k_decode_chain(
    const uint16_t* __restrict__ x, const LayerDev* __restrict__ layers, int L,
    const uint16_t* __restrict__ norm_w, float eps, uint16_t* __restrict__ out,
    int32_t* __restrict__ ids_out, uint8_t* __restrict__ ws) {
  StepAPre<FMT> pre;
  uint32_t epoch = 0;
  float resid = 0.0f;
  auto layer = [&](auto pf, auto epreg, auto xin, auto res, int l) __attribute__((always_inline)) {
    const LayerDev d = layers[l], dn = layers[l + 1 < L ? l + 1 : l];
    const FuseDev fz{NORM ? norm_w + (size_t)l * kH : nullptr, eps,
                     decltype(res)::value == 1 ? x : nullptr, nullptr};
    decode_layer<B, FMT, NORM, decltype(res)::value, decltype(pf)::value, decltype(epreg)::value,
                 decltype(xin)::value, true>(
        x, d.rw, d.routed, d.shared, out + (size_t)l * B * kH,
        ids_out ? ids_out + (size_t)l * B * kK : nullptr, nullptr, ws, fz, pre, dn, epoch, resid);
  };
  layer(std::integral_constant<int, 1>{}, std::false_type{}, std::integral_constant<int, 0>{},
        std::integral_constant<int, 1>{}, 0);
  for (int l = 1; l < L; ++l) {
    __syncthreads();
    layer(std::integral_constant<int, 2>{}, std::true_type{}, std::integral_constant<int, 1>{},
          std::integral_constant<int, 2>{}, l);
  }
}

}  // namespace moe

// ------------------------------------------------------------------ launchers
// Host-side launch templates of the kernels above, one per weight format;
// each format's instances are compiled in a translation unit of their own
// (explicit instantiations in decode_fused_*.hip, decode_stack.hip and
// decode_chain_*.hip), which keeps the build parallel.
namespace moe {

template <int FMT, int B>
hipError_t launch_fused_fb(const uint16_t* x, const uint16_t* rw, const ExpertsDev& routed,
                           const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                           uint8_t* ws, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                           const FuseDev& fz) {
  // one instance per fused combination: without fusion the kernel carries
  // none of its code (the schedule of the plain layer is left as it is)
  using K = decltype(&k_decode_fused<B, FMT, false, false>);
  static const K table[2][2] = {
      {k_decode_fused<B, FMT, false, false>, k_decode_fused<B, FMT, false, true>},
      {k_decode_fused<B, FMT, true, false>, k_decode_fused<B, FMT, true, true>}};
  const K k = table[fz.norm_w ? 1 : 0][fz.resid ? 1 : 0];
  if (e0 && e1)
    hipExtLaunchKernelGGL(k, dim3(kFusedGrid), dim3(kFusedThreads), 0, st, e0, e1, 0, x, rw, routed,
                          shared, out, ids, w, ws, fz);
  else
    hipLaunchKernelGGL(k, dim3(kFusedGrid), dim3(kFusedThreads), 0, st, x, rw, routed, shared, out,
                       ids, w, ws, fz);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fused_fmt(int B, const uint16_t* x, const uint16_t* rw, const ExpertsDev& routed,
                            const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                            uint8_t* ws, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                            const FuseDev& fz) {
  switch (B) {
#define MOE_CASE(b) \
  case b: return launch_fused_fb<FMT, b>(x, rw, routed, shared, out, ids, w, ws, st, e0, e1, fz);
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
  }
}

// The plain layer (no fused neighbours) with two shared experts: Flint's
// shape otherwise (the Inkling shape, served in one launch).
template <int FMT>
hipError_t launch_fused_ns2_fmt(int B, const uint16_t* x, const uint16_t* rw,
                                const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                                int32_t* ids, float* w, uint8_t* ws, hipStream_t st, hipEvent_t e0,
                                hipEvent_t e1) {
  switch (B) {
#define MOE_CASE(b)                                                                             \
  case b:                                                                                       \
    if (e0 && e1)                                                                               \
      hipExtLaunchKernelGGL((k_decode_fused<b, FMT, false, false, 2>), dim3(kFusedGrid),        \
                            dim3(kFusedThreads), 0, st, e0, e1, 0, x, rw, routed, shared, out,  \
                            ids, w, ws, FuseDev{});                                             \
    else                                                                                        \
      hipLaunchKernelGGL((k_decode_fused<b, FMT, false, false, 2>), dim3(kFusedGrid),           \
                         dim3(kFusedThreads), 0, st, x, rw, routed, shared, out, ids, w, ws,    \
                         FuseDev{});                                                            \
    break;
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Every instance of a kernel family can have one workgroup resident per CU.
template <typename K>
bool one_per_cu(K k) {
  int occ = 0;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, kFusedThreads, 0) == hipSuccess &&
         occ >= 1;
}

template <int FMT>
bool occupancy_fused_fmt() {
  return one_per_cu(k_decode_fused<8, FMT, false, false>) &&
         one_per_cu(k_decode_fused<8, FMT, true, true>) &&
         one_per_cu(k_decode_fused<1, FMT, true, true>);
}

template <int FMT>
hipError_t launch_stack_fmt(int B, const uint16_t* x, const LayerDev* layers, int L, uint16_t* out,
                            int32_t* ids, uint8_t* ws, hipStream_t st) {
  switch (B) {
#define MOE_CASE(b)                                                                              \
  case b:                                                                                        \
    hipLaunchKernelGGL((k_decode_stack<b, FMT>), dim3(kFusedGrid), dim3(kFusedThreads), 0, st, x, \
                       layers, L, out, ids, ws);                                                 \
    break;
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
bool occupancy_fused_ns2_fmt() {
  return one_per_cu(k_decode_fused<8, FMT, false, false, 2>) &&
         one_per_cu(k_decode_fused<1, FMT, false, false, 2>);
}

template <int FMT>
bool occupancy_stack_fmt() {
  return one_per_cu(k_decode_stack<8, FMT>) && one_per_cu(k_decode_stack<1, FMT>);
}

template <int FMT>
hipError_t launch_chain_fmt(int B, bool norm, const uint16_t* x, const LayerDev* layers, int L,
                            const uint16_t* norm_w, float eps, uint16_t* out, int32_t* ids,
                            uint8_t* ws, hipStream_t st) {
  switch (B) {
#define MOE_CASE(b)                                                                            \
  case b:                                                                                      \
    if (norm)                                                                                  \
      hipLaunchKernelGGL((k_decode_chain<b, FMT, true>), dim3(kFusedGrid), dim3(kFusedThreads), \
                         0, st, x, layers, L, norm_w, eps, out, ids, ws);                      \
    else                                                                                       \
      hipLaunchKernelGGL((k_decode_chain<b, FMT, false>), dim3(kFusedGrid),                    \
                         dim3(kFusedThreads), 0, st, x, layers, L, norm_w, eps, out, ids, ws); \
    break;
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
bool occupancy_chain_fmt() {
  return one_per_cu(k_decode_chain<8, FMT, true>) && one_per_cu(k_decode_chain<8, FMT, false>) &&
         one_per_cu(k_decode_chain<1, FMT, true>);
}

#define MOE_EXTERN_FMT(F)                                                                       \
  extern template hipError_t launch_fused_fmt<F>(int, const uint16_t*, const uint16_t*,        \
                                                 const ExpertsDev&, const ExpertsDev&,         \
                                                 uint16_t*, int32_t*, float*, uint8_t*,        \
                                                 hipStream_t, hipEvent_t, hipEvent_t,          \
                                                 const FuseDev&);                              \
  extern template bool occupancy_fused_fmt<F>();                                                \
  extern template hipError_t launch_stack_fmt<F>(int, const uint16_t*, const LayerDev*, int,    \
                                                 uint16_t*, int32_t*, uint8_t*, hipStream_t);  \
  extern template bool occupancy_stack_fmt<F>();                                                \
  extern template hipError_t launch_chain_fmt<F>(int, bool, const uint16_t*, const LayerDev*,   \
                                                 int, const uint16_t*, float, uint16_t*,       \
                                                 int32_t*, uint8_t*, hipStream_t);             \
  extern template bool occupancy_chain_fmt<F>();
#ifndef MOE_DECODE_INSTANTIATES
MOE_EXTERN_FMT(FMT_NVFP4)
MOE_EXTERN_FMT(FMT_BF16)
extern template hipError_t launch_fused_ns2_fmt<FMT_NVFP4>(int, const uint16_t*, const uint16_t*,
                                                           const ExpertsDev&, const ExpertsDev&,
                                                           uint16_t*, int32_t*, float*, uint8_t*,
                                                           hipStream_t, hipEvent_t, hipEvent_t);
extern template bool occupancy_fused_ns2_fmt<FMT_NVFP4>();
#endif
#undef MOE_EXTERN_FMT

}  // namespace moe
