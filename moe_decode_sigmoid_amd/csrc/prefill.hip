// Prefill path (T >= 1 tokens) of the Flint-style MoE layer on gfx950.
//
// The pages report the small-batch MoE kernels as also the largest prefill
// gain, measured on an 8,192-token prefill ("Day-0 Support for Flint on
// vLLM", Optimization section, Fig. 2 caption and change list).  At prefill
// sizes every expert sees ~T*6/256 tokens, so the experts run as dense
// bf16 matrix-core GEMMs over their token groups:
//
//   P1 router GEMM  x[T][2048] . W_r[256][2048]^T (bf16 MFMA, fp32 accumulate);
//      its epilogue keeps the 32 x 256 logit tile in LDS and does sigmoid /
//      top-6 / renormalisation per token, and counts the tile's tokens per
//      expert.
//   P2 scan         per-expert totals, per-tile bases and expert offsets give
//      a stable counting sort (token order inside each expert), and the list
//      of 128-row GEMM work items.
//   P3 positions    each (token, slot) gets its row in the expert-grouped
//      order; rows T*6 .. T*7-1 are the shared expert's (token order).
//   P4 GEMM 1       per work item and 128-column slice: [gate; up] rows of the
//      expert, NVFP4 decoded to bf16 in LDS, times the gathered x rows;
//      SiLU(g) * u in registers -> h (bf16) [T*7][512].
//   P5 GEMM 2       h rows . D_e^T, times the routing weight -> fp16 partial
//      rows [T*7][2048].
//   P6 combine      y[t] = sum over the token's six routed rows (ascending
//      expert id) + its shared row, fp32, rounded once to bf16.
//
// GEMM 1 (and GEMM 2 of bf16 experts) tiles are 128 x 256: eight waves of
// 64 x 64 (2 x 2 MFMA blocks each), A and B staged in LDS as bf16 with K = 64
// per stage in two LDS buffers (110 KB, one workgroup per CU), NVFP4 decoded
// to bf16 as it is written to LDS; the global loads of the next kRingDepth
// stages are held in registers, so the HBM / gather latency of one stage
// hides behind the MFMA work of the others.  GEMM 2 of NVFP4 experts keeps
// the weights in registers instead (see its section).  The router GEMM keeps
// K = 64 per stage.  Work items are mapped so that the column slices of one
// item run on one XCD (workgroup b lands on XCD b % 8) and share its L2.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Lane l supplies A[row l%32][k 8(l/32)..+7]
// and B[k 8(l/32)..+7][col l%32]; result element i of lane l is
// C[(i%4) + 8(i/4) + 4(l/32)][l%32].  The weight matrices are stored
// output-major with K contiguous, so B rows come straight from memory.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16;

constexpr int kLdsPad = 8;               // bf16 elements of padding per LDS row
constexpr int kRBK = 64;                 // router GEMM: K per pipeline stage
constexpr int kRLdsRow = kRBK + kLdsPad; //   and its LDS row pitch (bf16 elements)
constexpr int kGBK1 = 64;                // GEMM 1 (gate/up): K per pipeline stage
constexpr int kGBK2 = 64;                // GEMM 2 (down): K per pipeline stage
constexpr int kPTile = 32;               // router tile (tokens)
constexpr int kGBM = 128;                // grouped GEMM rows per work item
constexpr int kGBN = 256;                // grouped GEMM B rows per tile
constexpr int kPThreads = 256;
constexpr int kSlices1 = kI / (kGBN / 2);  // gate/up column slices (128 h columns each)
constexpr int kSlices2 = kH / kGBN;        // down column slices

// ------------------------------------------------------------------ workspace
struct PrefillLayout {
  size_t ids, w, hist, base, cnt, off, nitems, items, perm, pos, wpos, h, part, xn, total;
  int T, ntiles, max_items;
};

__host__ __device__ inline size_t al256(size_t v) { return (v + 255) / 256 * 256; }

__host__ __device__ inline PrefillLayout prefill_layout(int T) {
  PrefillLayout L;
  L.T = T;
  L.ntiles = (T + kPTile - 1) / kPTile;
  L.max_items = (T * kK + kGBM - 1) / kGBM + kE + (T + kGBM - 1) / kGBM;
  // after the decode kernels' region: the epoch counters, h-ready counters
  // and tagged logit slots there persist from call to call, and a byte of
  // prefill data left in them would desynchronise later decode calls on a
  // shared workspace
  size_t o = al256(kDecodeWsBytes);
  L.ids = o;    o = al256(o + sizeof(int) * (size_t)T * kK);
  L.w = o;      o = al256(o + sizeof(float) * (size_t)T * kK);
  L.hist = o;   o = al256(o + sizeof(int) * (size_t)L.ntiles * kE);
  L.base = o;   o = al256(o + sizeof(int) * (size_t)L.ntiles * kE);
  L.cnt = o;    o = al256(o + sizeof(int) * (kE + 1));
  L.off = o;    o = al256(o + sizeof(int) * (kE + 2));
  L.nitems = o; o = al256(o + sizeof(int) * 4);
  L.items = o;  o = al256(o + sizeof(int2) * (size_t)L.max_items);
  L.perm = o;   o = al256(o + sizeof(int) * (size_t)T * (kK + 1));
  L.pos = o;    o = al256(o + sizeof(int) * (size_t)T * kK);
  L.wpos = o;   o = al256(o + sizeof(float) * (size_t)T * (kK + 1));
  L.h = o;      o = al256(o + 2 * (size_t)T * (kK + 1) * kI);
  L.part = o;   o = al256(o + 2 * (size_t)T * (kK + 1) * kH);
  L.xn = o;     o = al256(o + 2 * (size_t)T * kH);   // normalised input (fused RMSNorm)
  L.total = o;
  return L;
}

size_t prefill_ws_bytes(int T) {
  if (T < 1 || T > (1 << 20)) return 0;
  return prefill_layout(T).total;
}

template <typename P>
__device__ __forceinline__ P* wsp(uint8_t* ws, size_t off) {
  return reinterpret_cast<P*>(ws + off);
}

// ------------------------------------------------------------------ MFMA tile core
// One workgroup tile: C[BM][BN] += A[BM][K] . B[BN][K]^T with A, B staged in
// LDS as bf16 [rows][BK + kLdsPad].  WM x WN waves; wave tile (BM/WM) x (BN/WN)
// made of 32x32 blocks.
template <int BM, int BN, int WM, int WN, int BK>
struct TileAcc {
  static constexpr int LR = BK + kLdsPad;   // LDS row pitch
  static constexpr int MB = BM / WM / 32, NB = BN / WN / 32;
  f32x16 c[MB][NB];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) c[i][j][k] = 0.0f;
  }
  // one BK stage from LDS
  __device__ __forceinline__ void mma(const __bf16* sA, const __bf16* sB, int wave, int lane) {
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * (BM / WM) + 32 * i + r) * LR + ks + kh);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(sB + (wn * (BN / WN) + 32 * j + r) * LR + ks + kh);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], c[i][j], 0, 0, 0);
    }
  }
  // row / column (within the tile) of accumulator element k of block (i, j)
  __device__ __forceinline__ static int row_of(int wave, int lane, int i, int k) {
    return (wave / WN) * (BM / WM) + 32 * i + (k % 4) + 8 * (k / 4) + 4 * (lane >> 5);
  }
  __device__ __forceinline__ static int col_of(int wave, int lane, int j) {
    return (wave % WN) * (BN / WN) + 32 * j + (lane & 31);
  }
};

// 16 bf16 (one uint4 pair) of a bf16 row segment into LDS
__device__ __forceinline__ void st_lds16(__bf16* dst, uint4 v) { *reinterpret_cast<uint4*>(dst) = v; }

// E4M3 byte j (static after unrolling) of a word, as fp32.
__device__ __forceinline__ float e4m3_sel(uint32_t w, int j) {
  return j == 0 ? e4m3_to_f32<0>(w) : j == 1 ? e4m3_to_f32<1>(w) : j == 2 ? e4m3_to_f32<2>(w)
                                                                           : e4m3_to_f32<3>(w);
}

// 8 NVFP4 codes (one dword) times their block scale -> 8 exact bf16 values
// (4 dwords).  e2m1 (exact in fp32) * e4m3 (exact) is exact in fp32 and,
// having at most six significant bits, in bf16 too, so truncation is exact.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s) {
  const f32x2 p0 = fp4x2_to_f32<0>(w), p1 = fp4x2_to_f32<1>(w), p2 = fp4x2_to_f32<2>(w),
              p3 = fp4x2_to_f32<3>(w);
  auto pk = [&](f32x2 p) {           // high halves of the two products, one byte permute
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, p.y * s),
                                 __builtin_bit_cast(uint32_t, p.x * s), 0x07060302u);
  };
  return make_uint4(pk(p0), pk(p1), pk(p2), pk(p3));
}

// E NVFP4 codes of one row (E / 32 uint4) with their E / 16 block scales
// (bytes of sc) -> E bf16 in LDS.
template <int E>
__device__ __forceinline__ void dequant_to_lds(__bf16* dst, const uint4 (&c)[E / 32], uint32_t sc) {
  uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < E / 32; ++i) {
    const float s0 = e4m3_sel(sc, 2 * i), s1 = e4m3_sel(sc, 2 * i + 1);
    d[4 * i + 0] = dequant8(c[i].x, s0);
    d[4 * i + 1] = dequant8(c[i].y, s0);
    d[4 * i + 2] = dequant8(c[i].z, s1);
    d[4 * i + 3] = dequant8(c[i].w, s1);
  }
}

// K pipeline over NK stages: register ring of D stages in flight, two LDS
// buffers.  gload(slot, kt) issues stage kt's global loads into a ring slot;
// sstore(slot, buf) writes a slot to LDS buffer buf; mma(buf) consumes it.
// Slot of stage s is s % D.  Every load is unconditional: the main loop
// (unrolled by D, so slots are static) runs the blocks whose refills all
// exist, and the last blocks are unrolled with static conditions.  A load
// under a runtime branch would leave the compiler unsure how many loads are
// in flight, and it would then drain the ring at every block.
// f(integral_constant<int, J0>), ..., f(integral_constant<int, J0 + N - 1>)
template <int J0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    f(std::integral_constant<int, J0>{});
    static_for<J0 + 1, N - 1>(f);
  }
}

template <int D, int NK, typename Slot, typename GL, typename SS, typename MM>
__device__ __forceinline__ void kpipeline(Slot (&ring)[D], GL gload, SS sstore, MM mma) {
  static_assert(D % 2 == 0, "a block of D stages starts on LDS buffer 0");
  // stage kt held in slot Q = kt % D (LDS buffer kt & 1 = Q & 1): consume it,
  // stage the next one into LDS and refill its slot (LOAD), if any (NEXT)
  auto stage = [&](auto Q, int kt, auto LOAD, auto NEXT) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
    mma(q & 1);
    if constexpr (decltype(NEXT)::value) {
      sstore(ring[(q + 1) % D], (q + 1) & 1);
      if constexpr (decltype(LOAD)::value) gload(ring[(q + 1) % D], kt + 1 + D);
    }
    __syncthreads();
  };
#pragma unroll
  for (int q = 0; q < D; ++q)
    if (q < NK) gload(ring[q], q);
  sstore(ring[0], 0);
  if constexpr (D < NK) gload(ring[0], D);
  __syncthreads();
  constexpr int kMain = NK > 2 * D ? (NK - 2 * D) / D * D : 0;   // blocks with every refill
  for (int kt0 = 0; kt0 < kMain; kt0 += D)
    static_for<0, D>([&](auto Q) __attribute__((always_inline)) {
      stage(Q, kt0 + decltype(Q)::value, std::true_type{}, std::true_type{});
    });
  static_for<0, NK - kMain>([&](auto J) __attribute__((always_inline)) {
    constexpr int kt = kMain + decltype(J)::value;
    stage(std::integral_constant<int, kt % D>{}, kt, std::bool_constant<(kt + 1 + D < NK)>{},
          std::bool_constant<(kt + 1 < NK)>{});
  });
}

// ------------------------------------------------------------------ P1 router + top-6
// Tile of kPTile tokens x 256 experts; kRWaves waves side by side, each 32
// tokens x 256 / kRWaves experts.
constexpr int kRWaves = 8;   // two per SIMD (4 measured 53.5 against 44.6 us at 8192 tokens)
constexpr int kRRing = 4;    // stages of global loads in flight (2: 44.6 us, 4: 43.6, 6: 43.7)
constexpr int kRThreads = 64 * kRWaves;
__global__ __launch_bounds__(kRThreads) void k_prefill_route(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ rw, int T,
                                                             uint8_t* __restrict__ ws,
                                                             int32_t* __restrict__ ids_out,
                                                             float* __restrict__ w_out) {
  using Acc = TileAcc<kPTile, kE, 1, kRWaves, kRBK>;
  const PrefillLayout L = prefill_layout(T);
  const int tile = blockIdx.x, t0 = tile * kPTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ __align__(16) __bf16 sA[2][kPTile * kRLdsRow];
  __shared__ __align__(16) __bf16 sB[2][kE * kRLdsRow];
  // A: 32 rows x 128 B per stage, split evenly over the threads (16 or 8
  // bytes each); B: 256 router rows x 128 B, thread tid takes rows
  // (kRThreads / 8) i + tid / 8, segment tid % 8, so that 8 consecutive
  // lanes read one row's 128 B (a load touches 8 cache lines, not 64)
  constexpr int kAB = kPTile * kRBK * 2 / kRThreads;      // A bytes per thread per stage
  constexpr int kBRows = kRThreads / 8, kBN = kE / kBRows;  // B rows per pass, passes
  using AVec = std::conditional_t<kAB == 16, uint4, uint2>;
  const int ar = tid / (128 / kAB), aseg = tid % (128 / kAB);
  const AVec* ap = reinterpret_cast<const AVec*>(x + (size_t)min(t0 + ar, T - 1) * kH) + aseg;
  const int br = tid >> 3, bseg = tid & 7;
  const uint4* bp = reinterpret_cast<const uint4*>(rw + (size_t)br * kH) + bseg;
  struct Slot { AVec a; uint4 b[kBN]; };
  Slot ring[kRRing];
  auto gload = [&](Slot& sl, int kt) {
    sl.a = ap[kt * (kRBK * 2 / kAB)];
#pragma unroll
    for (int i = 0; i < kBN; ++i) sl.b[i] = bp[(size_t)i * kBRows * (kH / 8) + kt * 8];
  };
  auto sstore = [&](const Slot& sl, int buf) {
    *reinterpret_cast<AVec*>(&sA[buf][ar * kRLdsRow + aseg * (kAB / 2)]) = sl.a;
#pragma unroll
    for (int i = 0; i < kBN; ++i)
      st_lds16(&sB[buf][(kBRows * i + br) * kRLdsRow + bseg * 8], sl.b[i]);
  };
  Acc acc;
  acc.zero();
  kpipeline<kRRing, kH / kRBK>(ring, gload, sstore,
                               [&](int buf) { acc.mma(sA[buf], sB[buf], wave, lane); });
  // logits tile -> LDS (reuse sB as fp32 [32][256 + 4])
  float* sL = reinterpret_cast<float*>(&sB[0][0]);
  constexpr int LP = kE + 4;
#pragma unroll
  for (int j = 0; j < Acc::NB; ++j)
#pragma unroll
    for (int k = 0; k < 16; ++k)
      sL[Acc::row_of(wave, lane, 0, k) * LP + Acc::col_of(wave, lane, j)] = acc.c[0][j][k];
  __syncthreads();
  int* gids = wsp<int>(ws, L.ids);
  float* gw = wsp<float>(ws, L.w);
  __shared__ int s_ids[kPTile][kK];
  for (int r = wave; r < kPTile; r += kRWaves) {
    const int t = t0 + r;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = sL[r * LP + lane + 64 * q];
    int sel_i[kK];
    float sel_l[kK];
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
        s_ids[r][j] = t < T ? sel_i[j] : -1;
        if (t < T) {
          gids[(size_t)t * kK + j] = sel_i[j];
          gw[(size_t)t * kK + j] = s[j] / sum;
          if (ids_out) ids_out[(size_t)t * kK + j] = sel_i[j];
          if (w_out) w_out[(size_t)t * kK + j] = s[j] / sum;
        }
      }
    }
  }
  __syncthreads();
  // tokens of this tile per expert (thread e counts expert e)
  if (tid < kE) {
    int c = 0;
    for (int i = 0; i < kPTile * kK; ++i) c += (s_ids[i / kK][i % kK] == tid) ? 1 : 0;
    wsp<int>(ws, L.hist)[(size_t)tile * kE + tid] = c;
  }
}

// ------------------------------------------------------------------ P2 scan
// One workgroup of 1024 threads: thread (q, e) sums quarter q of the router
// tiles for expert e, then the quarters are chained in order.  Stable order:
// tiles in order, and inside a tile tokens in order (positions kernel).
// Work items of kGBM rows per expert, then the shared expert's.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_prefill_scan(int T, uint8_t* __restrict__ ws) {
  const PrefillLayout L = prefill_layout(T);
  const int e = threadIdx.x % kE, q = threadIdx.x / kE;   // q in 0..3
  const int* hist = wsp<int>(ws, L.hist);
  int* base = wsp<int>(ws, L.base);
  const int per = (L.ntiles + 3) / 4, lo = q * per, hi = min(L.ntiles, lo + per);
  __shared__ int s_q[4][kE];
  int sum = 0;
  for (int t0 = lo; t0 < hi; t0 += 16) {                 // 16 independent loads in flight
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = t0 + i < hi ? hist[(size_t)(t0 + i) * kE + e] : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += v[i];
  }
  s_q[q][e] = sum;
  __syncthreads();
  int run = 0;
  for (int k = 0; k < q; ++k) run += s_q[k][e];
  for (int t0 = lo; t0 < hi; t0 += 16) {
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = t0 + i < hi ? hist[(size_t)(t0 + i) * kE + e] : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (t0 + i < hi) {
        base[(size_t)(t0 + i) * kE + e] = run;
        run += v[i];
      }
  }
  __shared__ int s_cnt[kE], s_first[kE + 1];
  if (q == 3) {
    s_cnt[e] = run;
    wsp<int>(ws, L.cnt)[e] = run;
  }
  __syncthreads();
  if (threadIdx.x < 64) {                                // expert offsets and first work item
    const int lane = threadIdx.x;
    int o = 0, it = 0;
    for (int c = 0; c < kE / 64; ++c) {
      const int x = 64 * c + lane;
      int cnt = s_cnt[x], tiles = (cnt + kGBM - 1) / kGBM;
      // inclusive scans across the wave
      int ic = cnt, itl = tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int a = __shfl_up(ic, d, 64), b = __shfl_up(itl, d, 64);
        if (lane >= d) { ic += a; itl += b; }
      }
      wsp<int>(ws, L.off)[x] = o + ic - cnt;
      s_first[x] = it + itl - tiles;
      o += __shfl(ic, 63, 64);
      it += __shfl(itl, 63, 64);
    }
    if (lane == 0) {
      int* off = wsp<int>(ws, L.off);
      off[kE] = o;                                       // = T * 6: shared rows start here
      off[kE + 1] = o + T;
      wsp<int>(ws, L.cnt)[kE] = T;
      s_first[kE] = it;
      wsp<int>(ws, L.nitems)[0] = it + (T + kGBM - 1) / kGBM;
    }
  }
  __syncthreads();
  int2* items = wsp<int2>(ws, L.items);
  for (int x = threadIdx.x; x < kE; x += kScanThreads)
    for (int m = 0; m * kGBM < s_cnt[x]; ++m) items[s_first[x] + m] = make_int2(x, m * kGBM);
  for (int m = threadIdx.x; m * kGBM < T; m += kScanThreads)
    items[s_first[kE] + m] = make_int2(kE, m * kGBM);
}

// ------------------------------------------------------------------ P3 positions
// One workgroup per router tile; thread i < 192 owns (token t0 + i/6, slot i%6).
__global__ __launch_bounds__(kPThreads) void k_prefill_positions(int T, uint8_t* __restrict__ ws) {
  const PrefillLayout L = prefill_layout(T);
  const int tile = blockIdx.x, t0 = tile * kPTile, i = threadIdx.x;
  __shared__ int s_e[kPTile * kK];
  const int* ids = wsp<int>(ws, L.ids);
  const int t = t0 + i / kK;
  if (i < kPTile * kK) s_e[i] = t < T ? ids[(size_t)t0 * kK + i] : -1;
  __syncthreads();
  int* perm = wsp<int>(ws, L.perm);
  float* wpos = wsp<float>(ws, L.wpos);
  if (i < kPTile * kK && t < T) {
    const int e = s_e[i];
    int rank = 0;
    for (int q = 0; q < i; ++q) rank += (s_e[q] == e) ? 1 : 0;
    const int p = wsp<int>(ws, L.off)[e] + wsp<int>(ws, L.base)[(size_t)tile * kE + e] + rank;
    perm[p] = t;
    wsp<int>(ws, L.pos)[(size_t)t * kK + (i % kK)] = p;
    wpos[p] = wsp<float>(ws, L.w)[(size_t)t * kK + (i % kK)];
  }
  if (i < kPTile && t0 + i < T) {                      // shared rows
    const int p = T * kK + t0 + i;
    perm[p] = t0 + i;
    wpos[p] = 1.0f;
  }
}

// ------------------------------------------------------------------ grouped GEMM stages
// One pipeline stage of a grouped GEMM with NT threads: A = 128 rows x BK
// bf16, TA = NT / 128 threads per row, EA elements each; B = 256 rows x BK
// weights, TB = NT / 256 threads per row, EB elements each (NVFP4: EB / 2
// code bytes + EB / 16 scale bytes; bf16: 2 EB bytes).
template <int BK, int NT>
struct GShape {
  static constexpr int TA = NT / kGBM, TB = NT / kGBN;
  static constexpr int EA = BK / TA, EB = BK / TB;
  static constexpr int LR = BK + kLdsPad;       // LDS row pitch (bf16)
};

template <int FMT, int EA, int EB>
struct GSlot;
template <int EA, int EB>
struct GSlot<FMT_NVFP4, EA, EB> {
  uint4 a[EA / 8], c[EB / 32];
  // the block scales as loaded (kept at their width: a widened copy is
  // re-masked at the loop back-edge, which waits for the load)
  std::conditional_t<EB == 64, uint32_t, uint16_t> s;
};
template <int EA, int EB>
struct GSlot<FMT_BF16, EA, EB> {
  uint4 a[EA / 8], b[EB / 8];
};
template <int FMT>
constexpr int kRingDepth = FMT == FMT_NVFP4 ? 4 : 2;

// Work item and column slice of grouped-GEMM workgroup b with NS slices:
// b = ((item / 8) * NS + slice) * 8 + item % 8, so one item's slices share
// an XCD.
template <int NS>
__device__ __forceinline__ void item_slice(int b, int& item, int& slice) {
  slice = (b / 8) % NS;
  item = (b / (8 * NS)) * 8 + b % 8;
}

// Stage kt of a thread's B share: bcodes / bscales already point at the
// thread's first element of its row.
template <int FMT, int BK, int EA, int EB>
__device__ __forceinline__ void g_load_b(GSlot<FMT, EA, EB>& sl, const uint8_t* bcodes,
                                         const uint8_t* bscales, int kt) {
  if constexpr (FMT == FMT_NVFP4) {
    const uint4* cp = reinterpret_cast<const uint4*>(bcodes + (size_t)kt * (BK / 2));
#pragma unroll
    for (int i = 0; i < EB / 32; ++i) sl.c[i] = cp[i];
    if constexpr (EB == 64)
      sl.s = *reinterpret_cast<const uint32_t*>(bscales + (size_t)kt * (BK / 16));
    else
      sl.s = *reinterpret_cast<const uint16_t*>(bscales + (size_t)kt * (BK / 16));
  } else {
    const uint4* bp = reinterpret_cast<const uint4*>(bcodes + (size_t)kt * BK * 2);
#pragma unroll
    for (int i = 0; i < EB / 8; ++i) sl.b[i] = bp[i];
  }
}

// A slot into LDS: A row tid / TA at column (tid % TA) EA; B row tid / TB at
// column (tid % TB) EB, NVFP4 decoded to bf16.
template <int FMT, int BK, int NT, int EA, int EB>
__device__ __forceinline__ void g_store(const GSlot<FMT, EA, EB>& sl, __bf16* sA, __bf16* sB,
                                        int tid) {
  using G = GShape<BK, NT>;
  __bf16* da = sA + (tid / G::TA) * G::LR + (tid % G::TA) * EA;
#pragma unroll
  for (int i = 0; i < EA / 8; ++i) st_lds16(da + 8 * i, sl.a[i]);
  __bf16* db = sB + (tid / G::TB) * G::LR + (tid % G::TB) * EB;
  if constexpr (FMT == FMT_NVFP4) {
    dequant_to_lds<EB>(db, sl.c, sl.s);
  } else {
#pragma unroll
    for (int i = 0; i < EB / 8; ++i) st_lds16(db + 8 * i, sl.b[i]);
  }
}

// ------------------------------------------------------------------ P4 GEMM 1
// Work item (expert e, row m0) x column slice n (h columns [128 n, 128 n +
// 128)), 512 threads as 2 x 4 waves of 64 x 64: tile B row br is, for wave
// column br / 64 and block (br / 32) % 2, the gate (block 0) or up (block 1)
// row 128 n + 32 (br / 64) + br % 32, so each lane holds gate and up of the
// same h element.  Two waves per SIMD: one's MFMAs run while the other
// decodes weights or waits.
constexpr int kGThreads1 = 512;
template <int FMT>
__global__ __launch_bounds__(kGThreads1, 1) void k_prefill_gateup(const uint16_t* __restrict__ x,
                                                                  int T, ExpertsDev routed,
                                                                  ExpertsDev shared,
                                                                  uint8_t* __restrict__ ws) {
  using Acc = TileAcc<kGBM, kGBN, 2, 4, kGBK1>;
  using G = GShape<kGBK1, kGThreads1>;
  using Slot = GSlot<FMT, G::EA, G::EB>;
  const PrefillLayout L = prefill_layout(T);
  int item, n;
  item_slice<kSlices1>(blockIdx.x, item, n);
  if (item >= wsp<int>(ws, L.nitems)[0]) return;
  const int2 it = wsp<int2>(ws, L.items)[item];
  const int e = it.x, m0 = it.y;
  const int rows = min(kGBM, wsp<int>(ws, L.cnt)[e] - m0);
  const int rbase = wsp<int>(ws, L.off)[e] + m0;       // first grouped row of the item
  const ExpertsDev X = e < kE ? routed : shared;
  const size_t ee = e < kE ? (size_t)e : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ __align__(16) __bf16 sA[2][kGBM * G::LR];
  __shared__ __align__(16) __bf16 sB[2][kGBN * G::LR];
  const int tok = wsp<int>(ws, L.perm)[rbase + min(tid / G::TA, rows - 1)];
  const uint4* ap = reinterpret_cast<const uint4*>(x + (size_t)tok * kH) + (tid % G::TA) * (G::EA / 8);
  const int brow = tid / G::TB, bcol = (tid % G::TB) * G::EB;
  const int bwn = brow / 64, bj = (brow / 32) % 2, brr = brow % 32;
  const size_t wrow = (ee * 2 + bj) * kI + 128 * n + 32 * bwn + brr;   // row of w13
  const uint8_t* bcodes = FMT == FMT_NVFP4 ? X.w13 + wrow * (kH / 2) + bcol / 2
                                           : X.w13 + (wrow * kH + bcol) * 2;
  const uint8_t* bscales = FMT == FMT_NVFP4 ? X.w13s + wrow * (kH / 16) + bcol / 16 : nullptr;
  // NVFP4: the tile's block scales (256 rows x 128 bytes) go to LDS once, in
  // full 16-byte loads (the two threads of a row take 64 bytes each); a
  // stage then reads its 2 bytes per thread from LDS.  Loaded per stage from
  // memory, each 2-byte load touched a cache line of its own and those loads
  // cost about a fifth of the kernel.
  // (row pitch 144 bytes: a wave's 32 rows spread over the banks)
  constexpr int kSP = kH / 16 + 16;
  __shared__ __align__(16) uint8_t sS[FMT == FMT_NVFP4 ? kGBN * kSP : 16];
  if constexpr (FMT == FMT_NVFP4) {
    const uint4* src = reinterpret_cast<const uint4*>(X.w13s + wrow * (kH / 16)) + (tid % G::TB) * 4;
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[i];
    uint4* dst = reinterpret_cast<uint4*>(sS + brow * kSP) + (tid % G::TB) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = v[i];
    __syncthreads();
  }
  const uint8_t* sscales = sS + brow * kSP + bcol / 16;
  Slot ring[kRingDepth<FMT>];
  auto gload = [&](Slot& sl, int kt) {
#pragma unroll
    for (int i = 0; i < G::EA / 8; ++i) sl.a[i] = ap[kt * (kGBK1 / 8) + i];
    if constexpr (FMT == FMT_NVFP4) {
      const uint4* cp = reinterpret_cast<const uint4*>(bcodes + (size_t)kt * (kGBK1 / 2));
#pragma unroll
      for (int i = 0; i < G::EB / 32; ++i) sl.c[i] = cp[i];
      sl.s = *reinterpret_cast<const decltype(sl.s)*>(sscales + kt * (kGBK1 / 16));
    } else {
      g_load_b<FMT, kGBK1>(sl, bcodes, bscales, kt);
    }
  };
  auto sstore = [&](const Slot& sl, int buf) {
    g_store<FMT, kGBK1, kGThreads1>(sl, sA[buf], sB[buf], tid);
  };
  Acc acc;
  acc.zero();
  kpipeline<kRingDepth<FMT>, kH / kGBK1>(ring, gload, sstore,
                                        [&](int buf) { acc.mma(sA[buf], sB[buf], wave, lane); });
  // epilogue: h = SiLU(g * sg) * (u * su) -> bf16
  float sg = 1.0f, su = 1.0f;
  if constexpr (FMT == FMT_NVFP4) {
    sg = X.glob[ee * 3 + 0];
    su = X.glob[ee * 3 + 1];
  }
  uint16_t* h = wsp<uint16_t>(ws, L.h);
  const int hcol = 128 * n + 32 * (wave % 4) + (lane & 31);
#pragma unroll
  for (int i = 0; i < Acc::MB; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = Acc::row_of(wave, lane, i, k);
      if (r < rows) {
        const float g = acc.c[i][0][k] * sg, u = acc.c[i][1][k] * su;
        h[(size_t)(rbase + r) * kI + hcol] = f32_to_bf16_rne(silu_mul(g, u));
      }
    }
}

// ------------------------------------------------------------------ P5 GEMM 2, bf16 weights
// Work item (expert e, row m0) x column slice n (256 of the 2048 outputs):
// partial[row][col] = w_row * global * (h_row . D_e[col]) as fp16.  512
// threads as 2 x 4 waves, like GEMM 1.
constexpr int kGThreads2 = 512;
template <int FMT>
__global__ __launch_bounds__(kGThreads2, 1) void k_prefill_down(int T, ExpertsDev routed,
                                                                ExpertsDev shared,
                                                                uint8_t* __restrict__ ws) {
  using Acc = TileAcc<kGBM, kGBN, 2, 4, kGBK2>;
  using G = GShape<kGBK2, kGThreads2>;
  using Slot = GSlot<FMT, G::EA, G::EB>;
  const PrefillLayout L = prefill_layout(T);
  int item, n;
  item_slice<kSlices2>(blockIdx.x, item, n);
  if (item >= wsp<int>(ws, L.nitems)[0]) return;
  const int2 it = wsp<int2>(ws, L.items)[item];
  const int e = it.x, m0 = it.y;
  const int rows = min(kGBM, wsp<int>(ws, L.cnt)[e] - m0);
  const int rbase = wsp<int>(ws, L.off)[e] + m0;
  const ExpertsDev X = e < kE ? routed : shared;
  const size_t ee = e < kE ? (size_t)e : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ __align__(16) __bf16 sA[2][kGBM * G::LR];
  __shared__ __align__(16) __bf16 sB[2][kGBN * G::LR];
  const uint16_t* hsrc = wsp<uint16_t>(ws, L.h);
  const uint4* ap =
      reinterpret_cast<const uint4*>(hsrc + (size_t)(rbase + min(tid / G::TA, rows - 1)) * kI) +
      (tid % G::TA) * (G::EA / 8);
  const int bcol = (tid % G::TB) * G::EB;
  const size_t wrow = ee * kH + (size_t)kGBN * n + tid / G::TB;   // output column = row of w2
  const uint8_t* bcodes = FMT == FMT_NVFP4 ? X.w2 + wrow * (kI / 2) + bcol / 2
                                           : X.w2 + (wrow * kI + bcol) * 2;
  const uint8_t* bscales = FMT == FMT_NVFP4 ? X.w2s + wrow * (kI / 16) + bcol / 16 : nullptr;
  Slot ring[kRingDepth<FMT>];
  auto gload = [&](Slot& sl, int kt) {
#pragma unroll
    for (int i = 0; i < G::EA / 8; ++i) sl.a[i] = ap[kt * (kGBK2 / 8) + i];
    g_load_b<FMT, kGBK2>(sl, bcodes, bscales, kt);
  };
  auto sstore = [&](const Slot& sl, int buf) {
    g_store<FMT, kGBK2, kGThreads2>(sl, sA[buf], sB[buf], tid);
  };
  Acc acc;
  acc.zero();
  kpipeline<kRingDepth<FMT>, kI / kGBK2>(ring, gload, sstore,
                                        [&](int buf) { acc.mma(sA[buf], sB[buf], wave, lane); });
  const float gl = FMT == FMT_NVFP4 ? X.glob[ee * 3 + 2] : 1.0f;
  __shared__ float s_wr[kGBM];                          // routing weight * global per row
  if (tid < kGBM) s_wr[tid] = tid < rows ? wsp<float>(ws, L.wpos)[rbase + tid] * gl : 0.0f;
  __syncthreads();
  f16* part = wsp<f16>(ws, L.part);
#pragma unroll
  for (int i = 0; i < Acc::MB; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = Acc::row_of(wave, lane, i, k);
      if (r < rows) {
        const float wr = s_wr[r];
#pragma unroll
        for (int j = 0; j < Acc::NB; ++j)
          part[(size_t)(rbase + r) * kH + kGBN * n + Acc::col_of(wave, lane, j)] =
              (f16)(acc.c[i][j][k] * wr);
      }
    }
}

// ------------------------------------------------------------------ P5 GEMM 2, NVFP4 weights in registers
// The down GEMM of NVFP4 experts takes the weight operand straight from
// memory into the MFMA operand registers (no LDS for it): only the gathered
// h rows go through LDS.  At K = 512 the LDS-tiled form spends a large share
// of its time filling and draining the weight tiles; here each weight byte
// is loaded once, by the wave that multiplies it.  A workgroup is 8 waves (two per SIMD, so one's matrix
// instructions run while the other waits); each wave owns a 128 x 64 tile
// of the 128-row item, i.e. 4 x 2 blocks of 32 x 32, so an A fragment read
// from LDS feeds two products and a dequantised weight fragment four.
//
// Weight fragment of v_mfma_f32_32x32x16_bf16: lane l supplies B[k][n] for
// n = l % 32 and k = 8 (l / 32) .. + 7 of the 16-deep k-step.  A weight row
// (output column n) keeps K contiguous, so a 64-deep stage of a row is 32
// code bytes (dwords d = 0..7, dword d holding k 8 d .. 8 d + 7): the lower
// half-wave needs dwords 0, 2, 4, 6 (one per k-step), the upper half 1, 3,
// 5, 7.  Lane l loads bytes 16 (l / 32) .. + 15 of its row's stage (dwords
// 0-3 low, 4-7 high) and two 32-lane swaps hand each half its dwords.  Each
// k-step lies inside one 16-element block, so one E4M3 scale (byte ks of the
// stage's scale word) applies to the whole fragment; e2m1 * e4m3 is exact in
// bf16, so the dequantised operand is exact.
constexpr int kW2BK = 64;                // K per pipeline stage
constexpr int kW2Waves = 8;              // waves per workgroup (two per SIMD)
constexpr int kW2Threads = 64 * kW2Waves;
constexpr int kW2N = 64 * kW2Waves;      // weight rows (output columns) per workgroup
constexpr int kW2Slices2 = kH / kW2N;    // column slices of the down GEMM
constexpr int kW2Ring = 2;               // stages of global loads in flight
constexpr int kW2TPR = kW2Threads / kGBM;   // threads per A row
constexpr int kW2EA = kW2BK / kW2TPR;       // A elements per thread per stage

// One stage of a thread's global loads: 16 activation elements of its A row
// share, and the lane's 16 code bytes and the stage's four block scales of
// each of its two weight rows.
struct W2Slot {
  uint4 a[kW2EA / 8];
  uint4 c[2];
  uint32_t s[2];
};
// The weight words of the stage being multiplied, after the exchange: d[j][ks]
// is the dword of row j for k-step ks of this lane's half.
struct W2Cur {
  uint32_t d[2][4];
  uint32_t s[2];
};

__device__ __forceinline__ void w2_take(const W2Slot& sl, W2Cur& cur) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float r0 = __builtin_bit_cast(float, sl.c[j].x), r1 = __builtin_bit_cast(float, sl.c[j].y);
    float r2 = __builtin_bit_cast(float, sl.c[j].z), r3 = __builtin_bit_cast(float, sl.c[j].w);
    swap32(r0, r1);   // r0: dword 0 (low half) / 1 (high half); r1: 4 / 5
    swap32(r2, r3);   // r2: dword 2 / 3;                        r3: 6 / 7
    cur.d[j][0] = __builtin_bit_cast(uint32_t, r0);
    cur.d[j][1] = __builtin_bit_cast(uint32_t, r2);
    cur.d[j][2] = __builtin_bit_cast(uint32_t, r1);
    cur.d[j][3] = __builtin_bit_cast(uint32_t, r3);
    cur.s[j] = sl.s[j];
  }
}

// The wave's 128 x 64 accumulator (4 row blocks x 2 column blocks).
struct W2Acc {
  f32x16 c[4][2];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) c[i][j][k] = 0.0f;
  }
  // one 64-deep stage: A from LDS (rows of the item, pitch LR), the weight
  // fragments dequantised from cur one k-step at a time
  template <int LR>
  __device__ __forceinline__ void mma(const __bf16* sA, const W2Cur& cur, int lane) {
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (32 * i + r) * LR + 16 * ks + kh);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = __builtin_bit_cast(bf16x8, dequant8(cur.d[j][ks], e4m3_sel(cur.s[j], ks)));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], c[i][j], 0, 0, 0);
    }
  }
  // row (within the item) of accumulator element k of row block i
  __device__ __forceinline__ static int row_of(int lane, int i, int k) {
    return 32 * i + (k % 4) + 8 * (k / 4) + 4 * (lane >> 5);
  }
};

// P5: work item x slice n: output columns [512 n, 512 n + 512); wave w owns
// columns 512 n + 64 w + 32 j + l % 32 (j = 0, 1); partial[row][col] =
// w_row * global * (h_row . D_e[col]) as fp16.
__global__ __launch_bounds__(kW2Threads, 1) void k_prefill_down_w(int T, ExpertsDev routed,
                                                                  ExpertsDev shared,
                                                                  uint8_t* __restrict__ ws) {
  constexpr int LR = kW2BK + kLdsPad;
  const PrefillLayout L = prefill_layout(T);
  int item, n;
  item_slice<kW2Slices2>(blockIdx.x, item, n);
  if (item >= wsp<int>(ws, L.nitems)[0]) return;
  const int2 it = wsp<int2>(ws, L.items)[item];
  const int e = it.x, m0 = it.y;
  const int rows = min(kGBM, wsp<int>(ws, L.cnt)[e] - m0);
  const int rbase = wsp<int>(ws, L.off)[e] + m0;
  const ExpertsDev X = e < kE ? routed : shared;
  const size_t ee = e < kE ? (size_t)e : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;

  __shared__ __align__(16) __bf16 sA[2][kGBM * LR];
  const uint16_t* hsrc = wsp<uint16_t>(ws, L.h);
  const uint4* ap =
      reinterpret_cast<const uint4*>(hsrc + (size_t)(rbase + min(tid / kW2TPR, rows - 1)) * kI) +
      (tid % kW2TPR) * (kW2EA / 8);
  __bf16* adst0 = sA[0] + (tid / kW2TPR) * LR + (tid % kW2TPR) * kW2EA;
  const uint8_t* wrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t row = ee * kH + (size_t)kW2N * n + 64 * wave + 32 * j + (lane & 31);
    wrow[j] = X.w2 + row * (kI / 2);
  }
  // the block scales of the workgroup's 512 weight rows (contiguous, 32 bytes
  // a row) go to LDS once in 16-byte loads, and each stage reads its words
  // there: loaded per stage from memory, every 4-byte scale load touched a
  // cache line of its own (row pitch 48 bytes: at most two rows of a wave's
  // 32 on a bank)
  constexpr int kSP2 = kI / 16 + 16;
  __shared__ __align__(16) uint8_t sS2[kW2N * kSP2];
  {
    const uint4* src =
        reinterpret_cast<const uint4*>(X.w2s + (ee * kH + (size_t)kW2N * n) * (kI / 16)) + 2 * tid;
    const uint4 v0 = src[0], v1 = src[1];
    uint4* dst = reinterpret_cast<uint4*>(sS2 + tid * kSP2);
    dst[0] = v0;
    dst[1] = v1;
    __syncthreads();
  }
  const uint8_t* ssc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ssc[j] = sS2 + (64 * wave + 32 * j + (lane & 31)) * kSP2;
  W2Slot ring[kW2Ring];
  W2Cur cur;
  auto gload = [&](W2Slot& sl, int kt) {
#pragma unroll
    for (int i = 0; i < kW2EA / 8; ++i) sl.a[i] = ap[kt * (kW2BK / 8) + i];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sl.c[j] = *reinterpret_cast<const uint4*>(wrow[j] + (size_t)kt * (kW2BK / 2) + 16 * half);
      sl.s[j] = *reinterpret_cast<const uint32_t*>(ssc[j] + kt * (kW2BK / 16));
    }
  };
  auto sstore = [&](const W2Slot& sl, int buf) {
    __bf16* d = adst0 + buf * (kGBM * LR);
#pragma unroll
    for (int i = 0; i < kW2EA / 8; ++i) st_lds16(d + 8 * i, sl.a[i]);
    w2_take(sl, cur);
  };
  W2Acc acc;
  acc.zero();
  kpipeline<kW2Ring, kI / kW2BK>(ring, gload, sstore,
                                 [&](int buf) { acc.mma<LR>(sA[buf], cur, lane); });
  const float gl = X.glob[ee * 3 + 2];
  __shared__ float s_wr[kGBM];                          // routing weight * global per row
  if (tid < kGBM) s_wr[tid] = tid < rows ? wsp<float>(ws, L.wpos)[rbase + tid] * gl : 0.0f;
  __syncthreads();
  f16* part = wsp<f16>(ws, L.part);
  const int col0 = kW2N * n + 64 * wave + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = W2Acc::row_of(lane, i, k);
      if (r < rows) {
        const float wr = s_wr[r];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          part[(size_t)(rbase + r) * kH + col0 + 32 * j] = (f16)(acc.c[i][j][k] * wr);
      }
    }
}

// ------------------------------------------------------------------ P0 RMSNorm
// One wave per token, lane l on elements 32 l .. 32 l + 31: the mean square
// is summed in the same order as in the decode kernel's fused norm, so a
// token normalises to the same bf16 values on both paths.
__global__ __launch_bounds__(kPThreads) void k_prefill_rmsnorm(int T, const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ nw,
                                                               float eps,
                                                               uint16_t* __restrict__ xn) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kPThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)t * kH + 32 * lane);
  const uint4* q = reinterpret_cast<const uint4*>(nw + 32 * lane);
  uint4 a[4], w[4];
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = p[i];
    w[i] = q[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i] = a[i].x; v[4 * i + 1] = a[i].y; v[4 * i + 2] = a[i].z; v[4 * i + 3] = a[i].w;
  }
  const float r = row_rms_inv(v, eps);
  uint4* o = reinterpret_cast<uint4*>(xn + (size_t)t * kH + 32 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = rmsnorm8(a[i], w[i], r);
}

// ------------------------------------------------------------------ P6 combine
// Thread -> (token, 8 columns); routed rows in ascending expert id, then shared,
// then the residual when one is fused in.
__global__ __launch_bounds__(kPThreads) void k_prefill_combine(int T, uint8_t* __restrict__ ws,
                                                               const uint16_t* resid,
                                                               uint16_t* out) {
  const PrefillLayout L = prefill_layout(T);
  const int gid = blockIdx.x * kPThreads + threadIdx.x;
  const int t = gid / (kH / 8), c8 = (gid % (kH / 8)) * 8;
  if (t >= T) return;
  const int* ids = wsp<int>(ws, L.ids);
  const int* pos = wsp<int>(ws, L.pos);
  const f16* part = wsp<f16>(ws, L.part);
  // the token's six (expert, partial row) pairs in registers, sorted by
  // expert id (distinct within a token) with compare-exchanges on values
  int eid[kK], prow[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    eid[j] = ids[(size_t)t * kK + j];
    prow[j] = pos[(size_t)t * kK + j];
  }
#pragma unroll
  for (int a = 1; a < kK; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = eid[b] < eid[b - 1];
      const int e0 = eid[b - 1], e1 = eid[b], p0 = prow[b - 1], p1 = prow[b];
      eid[b - 1] = sw ? e1 : e0;
      eid[b] = sw ? e0 : e1;
      prow[b - 1] = sw ? p1 : p0;
      prow[b] = sw ? p0 : p1;
    }
  float y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add_row = [&](int p) {
    const uint4 v = *reinterpret_cast<const uint4*>(part + (size_t)p * kH + c8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] += (float)__builtin_bit_cast(f16, (uint16_t)(u[q] & 0xFFFF));
      y[2 * q + 1] += (float)__builtin_bit_cast(f16, (uint16_t)(u[q] >> 16));
    }
  };
#pragma unroll
  for (int j = 0; j < kK; ++j) add_row(prow[j]);
  add_row(T * kK + t);
  if (resid) {
    const uint4 v = *reinterpret_cast<const uint4*>(resid + (size_t)t * kH + c8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] += bf16_lo(u[q]);
      y[2 * q + 1] += bf16_hi(u[q]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (uint32_t)f32_to_bf16_rne(y[2 * q]) | ((uint32_t)f32_to_bf16_rne(y[2 * q + 1]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * kH + c8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ------------------------------------------------------------------ launcher
hipError_t launch_prefill(int T, int fmt, const uint16_t* x, const uint16_t* rw,
                          const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                          int32_t* ids, float* w, uint8_t* ws, hipStream_t st,
                          const FuseDev& fz) {
  const PrefillLayout L = prefill_layout(T);
  if (fz.norm_w) {
    uint16_t* xn = fz.xn_out ? fz.xn_out : reinterpret_cast<uint16_t*>(ws + L.xn);
    hipLaunchKernelGGL(k_prefill_rmsnorm, dim3((T + kPThreads / 64 - 1) / (kPThreads / 64)),
                       dim3(kPThreads), 0, st, T, x, fz.norm_w, fz.eps, xn);
    x = xn;
  }
  hipLaunchKernelGGL(k_prefill_route, dim3(L.ntiles), dim3(kRThreads), 0, st, x, rw, T, ws, ids, w);
  hipLaunchKernelGGL(k_prefill_scan, dim3(1), dim3(kScanThreads), 0, st, T, ws);
  hipLaunchKernelGGL(k_prefill_positions, dim3(L.ntiles), dim3(kPThreads), 0, st, T, ws);
  const int items8 = (L.max_items + 7) / 8 * 8;
  if (fmt == FMT_NVFP4) {
    hipLaunchKernelGGL(k_prefill_gateup<FMT_NVFP4>, dim3(items8 * kSlices1), dim3(kGThreads1), 0, st,
                       x, T, routed, shared, ws);
    hipLaunchKernelGGL(k_prefill_down_w, dim3(items8 * kW2Slices2), dim3(kW2Threads), 0, st, T,
                       routed, shared, ws);
  } else {
    hipLaunchKernelGGL(k_prefill_gateup<FMT_BF16>, dim3(items8 * kSlices1), dim3(kGThreads1), 0, st,
                       x, T, routed, shared, ws);
    hipLaunchKernelGGL(k_prefill_down<FMT_BF16>, dim3(items8 * kSlices2), dim3(kGThreads2), 0, st,
                       T, routed, shared, ws);
  }
  const int nthr = T * (kH / 8);
  hipLaunchKernelGGL(k_prefill_combine, dim3((nthr + kPThreads - 1) / kPThreads), dim3(kPThreads),
                     0, st, T, ws, fz.resid, out);
  return hipGetLastError();
}

}  // namespace moe
