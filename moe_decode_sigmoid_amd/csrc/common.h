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
constexpr int kMaxShared = 2;   // shared experts the single-launch decode kernels serve (1 or 2)
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

enum { FMT_NVFP4 = 0, FMT_BF16 = 1, FMT_MXFP8 = 2, FMT_NVFP4_A4 = 3 };

// One layer of a stack as the stacked decode kernel reads it (device memory).
struct LayerDev {
  const uint16_t* rw;    // router bf16 [E][H]
  ExpertsDev routed;
  ExpertsDev shared;
};

// ------------------------------------------------------------ general shapes
// Layer shape of the general decode path (any served H, I, E, top-k, shared
// count; see decode_general.hip for the limits).
struct GenShape {
  int H, I, E, K, NS;
};
constexpr int kGenMaxE = 512;
constexpr int kGenMaxK = 8;
constexpr int kGenMaxNS = 2;
constexpr int kGenMaxEntries = kMaxB * kGenMaxK + kGenMaxNS;

// Dispatch of one call: the touched experts in ascending id, then the shared
// experts (entry value E + s), each with its token mask and weights.
struct GenCtl {
  int n_entries;
  int entry[kGenMaxEntries];
  unsigned amask[kGenMaxEntries];
  float wt[kGenMaxEntries][kMaxB];
};


// ---------------------------------------------------------------- workspace
// Decode workspace, all offsets in bytes from a 256-byte-aligned base.
struct DecodeCtl {
  unsigned ticket;                       // 0: route kernel arrival counter (self-resetting)
  int n_active;                          // 4: dispatch entries of the split path (shared last)
  unsigned err;                          // 8: kErr* bits of device-side waits that timed out
  unsigned pad0[61];                     // 12
  int active_expert[64];                 // expert id; kE marks the shared expert
  unsigned active_mask[64];              // bit t set when token t uses the entry
  float wtab[64][kMaxB];                 // routing weight of token t for the entry
  int ids[kMaxB][kK];                    // routing of the call (descending score)
  float w[kMaxB][kK];
};
// Bits of DecodeCtl::err: a bounded wait of the single-launch decode kernels
// gave up (its data never arrived), so the call's output is not valid.  The
// word is sticky until moe_workspace_status reads and clears it.
constexpr unsigned kErrLogits = 1u;   // the router logits exchange
constexpr unsigned kErrHReady = 2u;   // the h hand-over between the GEMVs
constexpr unsigned kErrXReady = 4u;   // the residual stream hand-over of a chained stack
constexpr size_t kCtlBytes = (sizeof(DecodeCtl) + 255) / 256 * 256;
constexpr size_t kLogitsOff = kCtlBytes;                          // f32 [kMaxB][kE]
constexpr size_t kHOff = kLogitsOff + sizeof(float) * kMaxB * kE; // f32 [kMaxActive][kMaxB][kI]
// Fused kernel: tagged 8-byte logit slots {fp32 value, call epoch}, written
// in kLogitReps copies (readers poll copy g % kLogitReps, which spreads the
// polling over more memory lines); then u32 words on 128-byte lines: one
// epoch counter per workgroup, then kBankReps copies of 64 h-ready counters.
constexpr int kLogitReps = 4;
constexpr int kBankReps = 4;
constexpr size_t kSlotLogitRep = 8 * kMaxB * kE;                                  // [kMaxB][kE]
constexpr size_t kSlotLogitOff = kHOff + sizeof(float) * kMaxActive * kMaxB * kI;
constexpr size_t kFlagOff = kSlotLogitOff + kSlotLogitRep * kLogitReps;
constexpr size_t kFlagStride = 128;
// Chained stack: the residual stream x_{l+1} as tagged 8-byte slots {two
// bf16 elements, epoch of layer l}, [kMaxB][kH / 2] per copy, kXReps copies.
constexpr int kXReps = 4;
constexpr size_t kSlotXRep = 8 * kMaxB * (kH / 2);
constexpr size_t kSlotXOff = kFlagOff + (256 + 64 * kBankReps) * kFlagStride;
// Everything below kDecodeWsBytes is the single-launch decode kernels'; the
// epoch counters, h-ready counters and tagged slots keep their values from
// call to call, so no other path writes below this offset.
// h as tagged 8-byte slots {two bf16 values, epoch}: [kMaxB * (kK + kMaxShared)
// pairs][kI / 2 slots] (the small-batch hand-over between the GEMVs).
constexpr size_t kHSlots = kI / 2;
constexpr size_t kSlotHOff = kSlotXOff + kSlotXRep * kXReps;
// Batch 1: the XCD-local logit slots, one copy per XCD ({fp32 value, epoch},
// [kE] each, 2 KB apart): written and read only by the workgroups running on
// that XCD.
constexpr int kXcds = 8;
constexpr size_t kSlotLXRep = 8 * kE;
constexpr size_t kSlotLXOff = kSlotHOff + 8 * kMaxB * (kK + kMaxShared) * kHSlots;
constexpr size_t kDecodeWsBytes = kSlotLXOff + kSlotLXRep * kXcds;
static_assert(kSlotLXOff % 128 == 0 && kSlotLXRep % 128 == 0, "each XCD's slots on lines of their own");
constexpr size_t kGenBase = kDecodeWsBytes;

// Workspace of the general path: logits f32 [kMaxB][E], the dispatch, h
// bf16 [entry][kMaxB][I] (and for W4A4 the quantised x and h), after the Flint paths' region (kGenBase bytes), so
// that one workspace can serve both without either touching the other's
// counters.
struct GenLayout {
  size_t logits, ctl, h, xq, gx, hq, gh, total;
};
__host__ __device__ inline GenLayout gen_layout(const GenShape& S) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  GenLayout L;
  L.logits = al(kGenBase);
  L.ctl = al(L.logits + sizeof(float) * kMaxB * (size_t)S.E);
  L.h = al(L.ctl + sizeof(GenCtl));
  // W4A4 only: the quantised x and h (bf16 e2m1 * e4m3, exact) and their
  // per-vector global scales
  L.xq = al(L.h + 2 * (size_t)kGenMaxEntries * kMaxB * S.I);
  L.gx = al(L.xq + 2 * (size_t)kMaxB * S.H);
  L.hq = al(L.gx + sizeof(float) * kMaxB);
  L.gh = al(L.hq + 2 * (size_t)kGenMaxEntries * kMaxB * S.I);
  L.total = al(L.gh + sizeof(float) * kGenMaxEntries * kMaxB);
  return L;
}
// upper bound of the entries of a call of B tokens
__host__ __device__ inline int gen_max_entries(const GenShape& S, int B) {
  return (S.E < B * S.K ? S.E : B * S.K) + S.NS;
}
constexpr int kShSlot = kMaxActive - 1;  // h entry of the shared expert in the fused kernel

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

// sum_k w_k v_k over one 32-element NVFP4 chunk of a weight row (16 code
// bytes c, the two E4M3 block scales in the low bytes of s) against 32 bf16
// values v given as 16 pairs, without the tensor scale: each 16-element
// block is summed in fp32 and multiplied by its scale.  S is the type the
// scales were loaded as (a 16-bit load kept at its width is not re-masked).
template <typename S>
__device__ __forceinline__ float nvfp4_dot32(uint4 c, S s, const uint32_t (&v)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    b0 = dot2_bf16(fp4x2_to_bf16<0>(w[d]), v[4 * d + 0], b0);
    b0 = dot2_bf16(fp4x2_to_bf16<1>(w[d]), v[4 * d + 1], b0);
    b0 = dot2_bf16(fp4x2_to_bf16<2>(w[d]), v[4 * d + 2], b0);
    b0 = dot2_bf16(fp4x2_to_bf16<3>(w[d]), v[4 * d + 3], b0);
  }
#pragma unroll
  for (int d = 2; d < 4; ++d) {
    b1 = dot2_bf16(fp4x2_to_bf16<0>(w[d]), v[4 * d + 0], b1);
    b1 = dot2_bf16(fp4x2_to_bf16<1>(w[d]), v[4 * d + 1], b1);
    b1 = dot2_bf16(fp4x2_to_bf16<2>(w[d]), v[4 * d + 2], b1);
    b1 = dot2_bf16(fp4x2_to_bf16<3>(w[d]), v[4 * d + 3], b1);
  }
  return b0 * e4m3_to_f32<0>(s) + b1 * e4m3_to_f32<1>(s);
}

// The same for a 32-element bf16 chunk (w: four uint4 of 8 bf16 each).
__device__ __forceinline__ float bf16_dot32(const uint4 (&w)[4], const uint32_t (&v)[16]) {
  float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    b0 = dot2_bf16(w[i].x, v[4 * i + 0], b0);
    b0 = dot2_bf16(w[i].y, v[4 * i + 1], b0);
    b0 = dot2_bf16(w[i].z, v[4 * i + 2], b0);
    b0 = dot2_bf16(w[i].w, v[4 * i + 3], b0);
  }
#pragma unroll
  for (int i = 2; i < 4; ++i) {
    b1 = dot2_bf16(w[i].x, v[4 * i + 0], b1);
    b1 = dot2_bf16(w[i].y, v[4 * i + 1], b1);
    b1 = dot2_bf16(w[i].z, v[4 * i + 2], b1);
    b1 = dot2_bf16(w[i].w, v[4 * i + 3], b1);
  }
  return b0 + b1;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here), with
// gfx950's v_cvt_pk_bf16_f32.  Checked on the GPU against the integer form
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16 over every non-NaN fp32 pattern: equal.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two at once, packed: lo in bits 0..15, hi in bits 16..31 (one instruction).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ------------------------------------------------------------ Four Over Six
// Scalar steps of the NVFP4 activation quantiser with the Four Over Six block
// scale (the Inkling-2-Small article, 48-layer MoE section), shared by the
// general path and the single-launch W4A4 layer so that both take the same
// decisions.
// nearest-even onto the E4M3FN grid of a finite s >= 0, saturating at 448.
// Branch-free (both the subnormal and the normal rounding are computed and
// one is selected): called by every lane of a wave with lane-dependent s.
__device__ __forceinline__ uint32_t a4_e4m3_rne(float s) {
  // subnormal: multiples of 2^-9 (s < 2^-6)
  const float ms = __builtin_rintf(__builtin_ldexpf(s, 9));
  const uint32_t sub = ms >= 8.0f ? 0x08u : (uint32_t)fmaxf(ms, 0.0f);
  // normal: 3 mantissa bits, carry into the exponent; past 448 saturates
  int e = (int)((__builtin_bit_cast(uint32_t, s) >> 23) & 0xFF) - 127;
  float m = __builtin_rintf(__fmul_rn(__fsub_rn(__builtin_ldexpf(s, -e), 1.0f), 8.0f));
  const bool carry = m >= 8.0f;
  m = carry ? 0.0f : m;
  e = carry ? e + 1 : e;
  const bool big = e > 8 || (e == 8 && m > 6.0f);
  const uint32_t nor = big ? 0x7Eu : (uint32_t)(((e + 7) << 3) | (int)m);
  return !(s > 0.0f) ? 0u : s >= 448.0f ? 0x7Eu : s < 0.015625f ? sub : nor;
}

// nearest-even onto the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at
// 6, as a signed value: midpoints go to the neighbour with the even mantissa
// bit (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4).
// The grid's step is 0.5 below 2, 1 below 4 and 2 above, so this is
// round-to-nearest-even at that step (v_rndne_f32 on an exactly scaled
// value); the result is the same as the chain of comparisons the definition
// reads as, for every input including the infinities.
__device__ __forceinline__ float a4_e2m1_rne(float v) {
  const float a = fabsf(v);
  const float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);   // selects of constants
  const float inv = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
  return __builtin_copysignf(fminf(__builtin_rintf(a * inv) * step, 6.0f), v);
}

__device__ __forceinline__ float a4_e4m3_value(uint32_t b) { return e4m3_to_f32<0>(b); }

// The same two roundings by gfx950's converts, equal to the functions above
// for every input (an exhaustive GPU check, moe_a4_convert_check: every fp32
// bit pattern for E2M1, every non-negative finite fp32 for E4M3):
//  - a4_e4m3_pk: E4M3 codes of two scales s >= 0 in bytes 0 and 1 (the fp32
//    -> FP8 convert rounds to nearest-even; 448 is its largest finite value,
//    and min(s, 448) makes it saturate there);
//  - a4_e2m1_pk8 / a4_e2m1_unpk8: E2M1 codes of 8 values, two per byte
//    (value 2 j in the low nibble of byte j), and their values (the fp32 ->
//    FP4 convert rounds to nearest-even and saturates at 6; a scale operand
//    of 1 leaves the values unscaled).
__device__ __forceinline__ uint32_t a4_e4m3_pk(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(a, 448.0f), fminf(b, 448.0f), 0, false);
}
__device__ __forceinline__ uint32_t a4_e2m1_pk8(const float (&r)[8]) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r[0], r[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[2], r[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[4], r[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[6], r[7], 1.0f, 3);
}
__device__ __forceinline__ void a4_e2m1_unpk8(uint32_t w, float (&c)[8]) {
  const f32x2 c0 = fp4x2_to_f32<0>(w), c1 = fp4x2_to_f32<1>(w), c2 = fp4x2_to_f32<2>(w),
              c3 = fp4x2_to_f32<3>(w);
  c[0] = c0[0]; c[1] = c0[1]; c[2] = c1[0]; c[3] = c1[1];
  c[4] = c2[0]; c[5] = c2[1]; c[6] = c3[0]; c[7] = c3[1];
}

// v / d rounded to nearest even, given y = RN(1 / d) (d > 0): the product
// q = RN(v y) is within an ulp of v / d, and one residual step RN(q + (v - d q) y),
// the residual exact by FMA, gives the correctly rounded quotient (Markstein's
// theorem on division through a correctly rounded reciprocal).  Every step
// scales exactly with the exponents of v and d while v, d, y, q and the
// residual are normal numbers, so a host check of every bf16 significand of v
// against every fp32 significand of d covers the normal range; callers keep d
// in [2^-64, 2^64], where a quotient of 1/8 or more leaves every step normal
// and a smaller one stays below the first E2M1 midpoint (1/4) either way.  A
// zero quotient takes v's sign, as the division's does.
__device__ __forceinline__ float div_by_recip(float v, float d, float y) {
  const float q = __fmul_rn(v, y);
  const float r = __builtin_fmaf(-d, q, v);
  return __builtin_copysignf(__builtin_fmaf(r, y, q), v);
}

// s_waitcnt immediate that waits for this wave's vector memory operations
// only (vmcnt 0; expcnt 7 and lgkmcnt 15 are "no wait" in gfx9's encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int kWaitVm0 = 0x0F70;

// Device-coherent accesses for data one workgroup hands to others inside a
// kernel: relaxed atomics at agent scope are issued with device-scope
// coherence (they bypass the per-XCD L2 copies), so no cache write-back or
// invalidation is needed; ordering comes from waiting for the stores before
// counting in at a barrier.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u16(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two consecutive floats (8-byte aligned) in one coherent load.
__device__ __forceinline__ f32x2 load_coherent2(const float* p) {
  const unsigned long long v = __hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(f32x2, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Cross-lane moves through DPP (no LDS round trip).  Controls (GFX9 DPP):
// quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E; row_ror:4 = 0x124, row_ror:8 = 0x128.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}

// Sum over each aligned group of 16 lanes (a DPP row); every lane of the
// group ends with the group's sum.
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_f32<0x128>(v);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0xB1>(v);
  return v;
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of a wave, returned uniformly (same value in every lane).
__device__ __forceinline__ float wave_sum(float v) {
  v = group16_sum(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// ------------------------------------------------------------ fused neighbours
// The pre-MoE RMSNorm and the residual add, fused into the layer's kernels
// ("Day-0 Support for Flint on vLLM", Optimization section, low-latency
// path).  A null pointer switches each part off.
struct FuseDev {
  const uint16_t* norm_w;   // bf16 [H]
  float eps;
  const uint16_t* resid;    // bf16 [T][H]: out = bf16(resid + y)
  uint16_t* xn_out;         // bf16 [T][H]: the normalised input, as used
};

// Sum of squares of the 8 bf16 elements of one 16-byte piece: a chain of
// v_dot2_f32_bf16 over its four bf16 pairs in element order (one instruction
// per pair, straight from the packed words).
__device__ __forceinline__ float sumsq8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return dot2_bf16(d, d, dot2_bf16(c, c, dot2_bf16(b, b, dot2_bf16(a, a, 0.0f))));
}

// 1 / sqrt(mean square + eps) of a row of kH bf16 values held by one wave,
// 32 per lane (lane l: elements 32 l .. 32 l + 31, four 8-element pieces).
// Each piece is summed in element order (sumsq8), a lane combines its four
// piece sums as (p0 + p2) + (p1 + p3), and the wave sums the lanes in
// wave_sum's fixed order.  Every path that normalises a row uses this one
// order.  The lane combination is the same value whichever piece a lane
// takes first (a rotation only swaps the two bracketed sums, and fp32
// addition is commutative), so a lane may read its pieces starting anywhere.
// Division and square root are the correctly rounded fp32 ones.
__device__ __forceinline__ float rms_inv_from_pieces(float p0, float p1, float p2, float p3,
                                                     float eps) {
  const float ss = wave_sum((p0 + p2) + (p1 + p3));
  return 1.0f / sqrtf(ss * (1.0f / kH) + eps);
}
__device__ __forceinline__ float row_rms_inv(const uint32_t (&v)[16], float eps) {
  float p[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) p[c] = sumsq8(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  return rms_inv_from_pieces(p[0], p[1], p[2], p[3], eps);
}

// bf16(x * r * w) for the 8 elements of one 16-byte piece: x * r and then
// * w in fp32, rounded once to bf16.
__device__ __forceinline__ uint4 rmsnorm8(uint4 x, uint4 w, float r) {
  const uint32_t xu[4] = {x.x, x.y, x.z, x.w}, wu[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32x2_to_bf16x2_rne((bf16_lo(xu[i]) * r) * bf16_lo(wu[i]),
                               (bf16_hi(xu[i]) * r) * bf16_hi(wu[i]));
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// The same with the weight piece already widened to fp32 (w[2 i], w[2 i + 1]
// are the low and high element of word i), for a weight shared by B rows.
__device__ __forceinline__ uint4 rmsnorm8w(uint4 x, const float (&w)[8], float r) {
  const uint32_t xu[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32x2_to_bf16x2_rne((bf16_lo(xu[i]) * r) * w[2 * i], (bf16_hi(xu[i]) * r) * w[2 * i + 1]);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Maximum over the 64 lanes of a wave, returned uniformly.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0x128>(v));
  v = fmaxf(v, dpp_f32<0x124>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0xB1>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// 32-lane and 16-lane half swaps of gfx950 (v_permlane32_swap: a keeps lanes
// 0-31 and takes b's 0-31 as its 32-63, b gets a's 32-63 and its own 32-63;
// v_permlane16_swap does the same within each 32-lane half).
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Wave totals of 8 per-lane values at once: value j's sum over the 64 lanes
// ends in lanes 8 j .. 8 j + 7 (halving exchanges across 32 and 16 lanes,
// then within rows: rotate by 8, half-row mirror, quad swaps).
__device__ __forceinline__ float wave_sum8(const float (&v)[8], int lane) {
  float w[4], u[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = v[j], b = v[4 + j];
    swap32(a, b);
    w[j] = a + b;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float a = w[j], b = w[2 + j];
    swap16(a, b);
    u[j] = a + b;
  }
  const bool hi = (lane & 8) != 0;
  float z = (hi ? u[1] : u[0]) + dpp_f32<0x128>(hi ? u[0] : u[1]);
  z += dpp_f32<0x141>(z);
  z += dpp_f32<0x4E>(z);
  z += dpp_f32<0xB1>(z);
  return z;
}

// Top-k of 256 scores held 4 per lane (expert e = lane + 64 q in v[q]) under
// the total order (value descending, index ascending).  Each round takes the
// wave maximum, then the lowest index holding it (q-major ballots: indices of
// v[0] are all below those of v[1], ...).  Every lane returns the same ids and
// values; the chosen entries of v are set to -inf.
template <int K>
__device__ __forceinline__ void wave_topk256(float (&v)[4], int lane, int (&ids)[K],
                                             float (&vals)[K]) {
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float m = wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    int idx = -1;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      const uint64_t bal = __ballot(v[q] == m);
      if (bal) idx = 64 * q + __builtin_ctzll(bal);
    }
    if (idx < 0) idx = j;   // only when every value is NaN (outside the contract): stay in range
    ids[j] = idx;
    vals[j] = m;
    if ((idx & 63) == lane) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((idx >> 6) == q) v[q] = -INFINITY;
    }
  }
}

}  // namespace moe
