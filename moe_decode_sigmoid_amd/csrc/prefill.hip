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
//   P4 GEMM 1       per work item and 64-column slice: [gate; up] rows of the
//      expert, NVFP4 decoded to bf16 in LDS, times the gathered x rows;
//      SiLU(g) * u in registers -> h (bf16) [T*7][512].
//   P5 GEMM 2       h rows . D_e^T, times the routing weight -> fp16 partial
//      rows [T*7][2048].
//   P6 combine      y[t] = sum over the token's six routed rows (ascending
//      expert id) + its shared row, fp32, rounded once to bf16.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Lane l supplies A[row l%32][k 8(l/32)..+7]
// and B[k 8(l/32)..+7][col l%32]; result element i of lane l is
// C[(i%4) + 8(i/4) + 4(l/32)][l%32].  The weight matrices are stored
// output-major with K contiguous, so B rows come straight from memory.
#include "common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16;

constexpr int kBK = 64;                  // K per pipeline stage
constexpr int kLdsPad = 8;               // bf16 elements of padding per LDS row
constexpr int kLdsRow = kBK + kLdsPad;   // LDS row pitch (bf16 elements)
constexpr int kPTile = 32;               // router tile (tokens)
constexpr int kGBM = 128;                // grouped GEMM rows per work item
constexpr int kGBN = 128;                // grouped GEMM B rows per tile
constexpr int kPThreads = 256;

// ------------------------------------------------------------------ workspace
struct PrefillLayout {
  size_t ids, w, hist, base, cnt, off, nitems, items, perm, pos, wpos, h, part, total;
  int T, ntiles, max_items;
};

__host__ __device__ inline size_t al256(size_t v) { return (v + 255) / 256 * 256; }

__host__ __device__ inline PrefillLayout prefill_layout(int T) {
  PrefillLayout L;
  L.T = T;
  L.ntiles = (T + kPTile - 1) / kPTile;
  L.max_items = (T * kK + kGBM - 1) / kGBM + kE + (T + kGBM - 1) / kGBM;
  size_t o = 0;
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
// LDS as bf16 [rows][kLdsRow].  WM x WN waves; wave tile (BM/WM) x (BN/WN)
// made of 32x32 blocks.
template <int BM, int BN, int WM, int WN>
struct TileAcc {
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
  // one kBK stage from LDS
  __device__ __forceinline__ void mma(const __bf16* sA, const __bf16* sB, int wave, int lane) {
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * (BM / WM) + 32 * i + r) * kLdsRow + ks + kh);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(sB + (wn * (BN / WN) + 32 * j + r) * kLdsRow + ks + kh);
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

// 32 NVFP4 codes + their two block scales -> 32 exact bf16 values in LDS.
// e2m1 (exact in fp32) * e4m3 (exact) is exact in fp32 and, having at most
// six significant bits, in bf16 too.
__device__ __forceinline__ void dequant32_to_lds(__bf16* dst, uint4 c, uint32_t sc) {
  const float s0 = e4m3_to_f32<0>(sc), s1 = e4m3_to_f32<1>(sc);
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float s = d < 2 ? s0 : s1;
    f32x2 p[4] = {fp4x2_to_f32<0>(w[d]), fp4x2_to_f32<1>(w[d]), fp4x2_to_f32<2>(w[d]),
                  fp4x2_to_f32<3>(w[d])};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = __builtin_bit_cast(uint32_t, p[q].x * s) >> 16;
      const uint32_t hi = __builtin_bit_cast(uint32_t, p[q].y * s) & 0xFFFF0000u;
      o[4 * d + q] = lo | hi;
    }
  }
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d4[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

// ------------------------------------------------------------------ P1 router + top-6
// Tile of kPTile tokens x 256 experts; waves 1 x 4, each 32 tokens x 64 experts.
__global__ __launch_bounds__(kPThreads) void k_prefill_route(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ rw, int T,
                                                             uint8_t* __restrict__ ws,
                                                             int32_t* __restrict__ ids_out,
                                                             float* __restrict__ w_out) {
  using Acc = TileAcc<kPTile, kE, 1, 4>;
  const PrefillLayout L = prefill_layout(T);
  const int tile = blockIdx.x, t0 = tile * kPTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ __align__(16) __bf16 sA[2][kPTile * kLdsRow];
  __shared__ __align__(16) __bf16 sB[2][kE * kLdsRow];
  // loaders: A 32 rows x 128 B -> one uint4 per thread; B 256 rows x 128 B -> 8 per thread
  const int ar = tid >> 3, aseg = tid & 7;
  const int at = min(t0 + ar, T - 1);
  const uint4* ap = reinterpret_cast<const uint4*>(x + (size_t)at * kH) + aseg;
  uint4 av, bv[8];
  auto gload = [&](int kt) {
    av = ap[kt * 8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + kPThreads * i, row = idx >> 3, seg = idx & 7;
      bv[i] = reinterpret_cast<const uint4*>(rw + (size_t)row * kH)[kt * 8 + seg];
    }
  };
  auto sstore = [&](int st) {
    st_lds16(&sA[st][ar * kLdsRow + aseg * 8], av);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + kPThreads * i, row = idx >> 3, seg = idx & 7;
      st_lds16(&sB[st][row * kLdsRow + seg * 8], bv[i]);
    }
  };
  Acc acc;
  acc.zero();
  constexpr int NK = kH / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < NK; ++kt) {
    if (kt + 1 < NK) gload(kt + 1);
    acc.mma(sA[kt & 1], sB[kt & 1], wave, lane);
    if (kt + 1 < NK) sstore((kt + 1) & 1);
    __syncthreads();
  }
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
  for (int r = wave; r < kPTile; r += 4) {
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
  {
    int c = 0;
    for (int i = 0; i < kPTile * kK; ++i) c += (s_ids[i / kK][i % kK] == tid) ? 1 : 0;
    wsp<int>(ws, L.hist)[(size_t)tile * kE + tid] = c;
  }
}

// ------------------------------------------------------------------ P2 scan
// One workgroup: thread e owns expert e.  Stable order: tiles in order, and
// inside a tile tokens in order (positions kernel).  Work items of kGBM rows
// per expert, then the shared expert's.
__global__ __launch_bounds__(kPThreads) void k_prefill_scan(int T, uint8_t* __restrict__ ws) {
  const PrefillLayout L = prefill_layout(T);
  const int e = threadIdx.x;
  const int* hist = wsp<int>(ws, L.hist);
  int* base = wsp<int>(ws, L.base);
  int run = 0;
  for (int tile = 0; tile < L.ntiles; ++tile) {
    base[(size_t)tile * kE + e] = run;
    run += hist[(size_t)tile * kE + e];
  }
  __shared__ int s_cnt[kE], s_tiles[kE];
  s_cnt[e] = run;
  s_tiles[e] = (run + kGBM - 1) / kGBM;
  wsp<int>(ws, L.cnt)[e] = run;
  __syncthreads();
  if (e == 0) {
    int* off = wsp<int>(ws, L.off);
    int2* items = wsp<int2>(ws, L.items);
    int o = 0, n = 0;
    for (int x = 0; x < kE; ++x) {
      off[x] = o;
      for (int m = 0; m < s_tiles[x]; ++m) items[n++] = make_int2(x, m * kGBM);
      o += s_cnt[x];
    }
    off[kE] = o;                                       // = T * 6: shared rows start here
    off[kE + 1] = o + T;
    wsp<int>(ws, L.cnt)[kE] = T;
    for (int m = 0; m < (T + kGBM - 1) / kGBM; ++m) items[n++] = make_int2(kE, m * kGBM);
    wsp<int>(ws, L.nitems)[0] = n;
  }
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

// ------------------------------------------------------------------ grouped GEMM loaders
// B rows of a grouped GEMM tile: NVFP4 (one 32-element chunk per thread and
// stage: 128 rows x 2 chunks) or bf16 (4 uint4 per thread).
template <int FMT>
struct BLoad;

template <>
struct BLoad<FMT_NVFP4> {
  uint4 c;
  uint32_t s;
  // row pointer to codes / scales of the B row; K chunk kt
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int K, int kt,
                                       int chunk) {
    c = *reinterpret_cast<const uint4*>(codes + (size_t)kt * (kBK / 2) + 16 * chunk);
    s = *reinterpret_cast<const uint16_t*>(scales + (size_t)kt * (kBK / 16) + 2 * chunk);
    (void)K;
  }
  __device__ __forceinline__ void store(__bf16* sB, int row, int chunk) const {
    dequant32_to_lds(sB + row * kLdsRow + 32 * chunk, c, s);
  }
};

template <>
struct BLoad<FMT_BF16> {
  uint4 v[2];
  __device__ __forceinline__ void load(const uint8_t* rowp, const uint8_t*, int K, int kt, int chunk) {
    (void)K;
    const uint4* p = reinterpret_cast<const uint4*>(rowp) + (size_t)kt * (kBK / 8) + 2 * chunk;
    v[0] = p[0];
    v[1] = p[1];
  }
  __device__ __forceinline__ void store(__bf16* sB, int row, int chunk) const {
    // chunk c of BF16 rows covers 16 elements [16c, 16c + 16) of the 64
    st_lds16(sB + row * kLdsRow + 16 * chunk, v[0]);
    st_lds16(sB + row * kLdsRow + 16 * chunk + 8, v[1]);
  }
};

// ------------------------------------------------------------------ P4 GEMM 1
// Work item (expert e, row m0) x column slice n: the tile's 128 B rows are,
// for wave column wn and block j, gate (j = 0) or up (j = 1) row
// 64 n + 32 wn + r, so each lane holds gate and up of the same h element.
template <int FMT>
__global__ __launch_bounds__(kPThreads) void k_prefill_gateup(const uint16_t* __restrict__ x, int T,
                                                              ExpertsDev routed, ExpertsDev shared,
                                                              uint8_t* __restrict__ ws) {
  using Acc = TileAcc<kGBM, kGBN, 2, 2>;
  const PrefillLayout L = prefill_layout(T);
  const int n = blockIdx.x % (kI / 64), item = blockIdx.x / (kI / 64);
  if (item >= wsp<int>(ws, L.nitems)[0]) return;
  const int2 it = wsp<int2>(ws, L.items)[item];
  const int e = it.x, m0 = it.y;
  const int rows = min(kGBM, wsp<int>(ws, L.cnt)[e] - m0);
  const int rbase = wsp<int>(ws, L.off)[e] + m0;       // first grouped row of the item
  const ExpertsDev X = e < kE ? routed : shared;
  const size_t ee = e < kE ? (size_t)e : 0;
  const int* perm = wsp<int>(ws, L.perm);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ __align__(16) __bf16 sA[2][kGBM * kLdsRow];
  __shared__ __align__(16) __bf16 sB[2][kGBN * kLdsRow];
  // A: 128 rows x 128 B: thread -> row tid / 2, half (64 B) tid % 2
  const int ar = tid >> 1, ah = tid & 1;
  const int tok = perm[rbase + min(ar, rows - 1)];
  const uint4* ap = reinterpret_cast<const uint4*>(x + (size_t)tok * kH) + 4 * ah;
  // B: tile row br = tid / 2 (0..127), chunk tid % 2
  const int br = tid >> 1, bch = tid & 1;
  const int bwn = br / 64, bj = (br / 32) % 2, brr = br % 32;
  const int wrow = 64 * n + 32 * bwn + brr;              // row within gate / up
  const int mat = bj;                                    // 0 gate, 1 up
  const uint8_t* bcodes;
  const uint8_t* bscales = nullptr;
  if constexpr (FMT == FMT_NVFP4) {
    bcodes = X.w13 + ((ee * 2 + mat) * kI + wrow) * (size_t)(kH / 2);
    bscales = X.w13s + ((ee * 2 + mat) * kI + wrow) * (size_t)(kH / 16);
  } else {
    bcodes = X.w13 + ((ee * 2 + mat) * kI + wrow) * (size_t)kH * 2;
  }
  uint4 av[4];
  BLoad<FMT> bl;
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = ap[kt * 8 + i];
    if constexpr (FMT == FMT_NVFP4) bl.load(bcodes, bscales, kH, kt, bch);
  };
  BLoad<FMT> bl2;
  auto gload_bf = [&](int kt) {                          // BF16 B needs 4 chunks of 16 per row
    if constexpr (FMT == FMT_BF16) {
      bl.load(bcodes, nullptr, kH, kt, 2 * bch);
      bl2.load(bcodes, nullptr, kH, kt, 2 * bch + 1);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st_lds16(&sA[st][ar * kLdsRow + ah * 32 + 8 * i], av[i]);
    if constexpr (FMT == FMT_NVFP4) {
      bl.store(sB[st], br, bch);
    } else {
      bl.store(sB[st], br, 2 * bch);
      bl2.store(sB[st], br, 2 * bch + 1);
    }
  };
  Acc acc;
  acc.zero();
  constexpr int NK = kH / kBK;
  gload(0);
  gload_bf(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < NK; ++kt) {
    if (kt + 1 < NK) {
      gload(kt + 1);
      gload_bf(kt + 1);
    }
    acc.mma(sA[kt & 1], sB[kt & 1], wave, lane);
    if (kt + 1 < NK) sstore((kt + 1) & 1);
    __syncthreads();
  }
  // epilogue: h = SiLU(g * sg) * (u * su) -> bf16
  float sg = 1.0f, su = 1.0f;
  if constexpr (FMT == FMT_NVFP4) {
    sg = X.glob[ee * 3 + 0];
    su = X.glob[ee * 3 + 1];
  }
  uint16_t* h = wsp<uint16_t>(ws, L.h);
  const int hcol = 64 * n + 32 * (wave % 2) + (lane & 31);
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

// ------------------------------------------------------------------ P5 GEMM 2
// Work item (expert e, row m0) x column slice n (128 of the 2048 outputs):
// partial[row][col] = w_row * global * (h_row . D_e[col]) as fp16.
template <int FMT>
__global__ __launch_bounds__(kPThreads) void k_prefill_down(int T, ExpertsDev routed,
                                                            ExpertsDev shared,
                                                            uint8_t* __restrict__ ws) {
  using Acc = TileAcc<kGBM, kGBN, 2, 2>;
  const PrefillLayout L = prefill_layout(T);
  const int n = blockIdx.x % (kH / kGBN), item = blockIdx.x / (kH / kGBN);
  if (item >= wsp<int>(ws, L.nitems)[0]) return;
  const int2 it = wsp<int2>(ws, L.items)[item];
  const int e = it.x, m0 = it.y;
  const int rows = min(kGBM, wsp<int>(ws, L.cnt)[e] - m0);
  const int rbase = wsp<int>(ws, L.off)[e] + m0;
  const ExpertsDev X = e < kE ? routed : shared;
  const size_t ee = e < kE ? (size_t)e : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ __align__(16) __bf16 sA[2][kGBM * kLdsRow];
  __shared__ __align__(16) __bf16 sB[2][kGBN * kLdsRow];
  const uint16_t* hsrc = wsp<uint16_t>(ws, L.h);
  const int ar = tid >> 1, ah = tid & 1;
  const uint4* ap = reinterpret_cast<const uint4*>(hsrc + (size_t)(rbase + min(ar, rows - 1)) * kI) + 4 * ah;
  const int br = tid >> 1, bch = tid & 1;
  const int wrow = kGBN * n + br;                        // output column = D row
  const uint8_t* bcodes;
  const uint8_t* bscales = nullptr;
  if constexpr (FMT == FMT_NVFP4) {
    bcodes = X.w2 + (ee * kH + wrow) * (size_t)(kI / 2);
    bscales = X.w2s + (ee * kH + wrow) * (size_t)(kI / 16);
  } else {
    bcodes = X.w2 + (ee * kH + wrow) * (size_t)kI * 2;
  }
  uint4 av[4];
  BLoad<FMT> bl, bl2;
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = ap[kt * 8 + i];
    if constexpr (FMT == FMT_NVFP4) {
      bl.load(bcodes, bscales, kI, kt, bch);
    } else {
      bl.load(bcodes, nullptr, kI, kt, 2 * bch);
      bl2.load(bcodes, nullptr, kI, kt, 2 * bch + 1);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st_lds16(&sA[st][ar * kLdsRow + ah * 32 + 8 * i], av[i]);
    if constexpr (FMT == FMT_NVFP4) {
      bl.store(sB[st], br, bch);
    } else {
      bl.store(sB[st], br, 2 * bch);
      bl2.store(sB[st], br, 2 * bch + 1);
    }
  };
  Acc acc;
  acc.zero();
  constexpr int NK = kI / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < NK; ++kt) {
    if (kt + 1 < NK) gload(kt + 1);
    acc.mma(sA[kt & 1], sB[kt & 1], wave, lane);
    if (kt + 1 < NK) sstore((kt + 1) & 1);
    __syncthreads();
  }
  const float gl = FMT == FMT_NVFP4 ? X.glob[ee * 3 + 2] : 1.0f;
  const float* wpos = wsp<float>(ws, L.wpos);
  f16* part = wsp<f16>(ws, L.part);
#pragma unroll
  for (int i = 0; i < Acc::MB; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = Acc::row_of(wave, lane, i, k);
      if (r < rows) {
        const float wr = wpos[rbase + r] * gl;
#pragma unroll
        for (int j = 0; j < Acc::NB; ++j)
          part[(size_t)(rbase + r) * kH + kGBN * n + Acc::col_of(wave, lane, j)] =
              (f16)(acc.c[i][j][k] * wr);
      }
    }
}

// ------------------------------------------------------------------ P6 combine
// Thread -> (token, 8 columns); routed rows in ascending expert id, then shared.
__global__ __launch_bounds__(kPThreads) void k_prefill_combine(int T, uint8_t* __restrict__ ws,
                                                               uint16_t* __restrict__ out) {
  const PrefillLayout L = prefill_layout(T);
  const int gid = blockIdx.x * kPThreads + threadIdx.x;
  const int t = gid / (kH / 8), c8 = (gid % (kH / 8)) * 8;
  if (t >= T) return;
  const int* ids = wsp<int>(ws, L.ids);
  const int* pos = wsp<int>(ws, L.pos);
  const f16* part = wsp<f16>(ws, L.part);
  int order[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) order[j] = j;
#pragma unroll
  for (int a = 1; a < kK; ++a)                            // sort slots by expert id
#pragma unroll
    for (int b = a; b > 0; --b) {
      const int ea = ids[(size_t)t * kK + order[b]], eb = ids[(size_t)t * kK + order[b - 1]];
      if (ea < eb) {
        const int tmp = order[b];
        order[b] = order[b - 1];
        order[b - 1] = tmp;
      }
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
  for (int j = 0; j < kK; ++j) add_row(pos[(size_t)t * kK + order[j]]);
  add_row(T * kK + t);
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (uint32_t)f32_to_bf16_rne(y[2 * q]) | ((uint32_t)f32_to_bf16_rne(y[2 * q + 1]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * kH + c8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ------------------------------------------------------------------ launcher
hipError_t launch_prefill(int T, int fmt, const uint16_t* x, const uint16_t* rw,
                          const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                          int32_t* ids, float* w, uint8_t* ws, hipStream_t st) {
  const PrefillLayout L = prefill_layout(T);
  hipLaunchKernelGGL(k_prefill_route, dim3(L.ntiles), dim3(kPThreads), 0, st, x, rw, T, ws, ids, w);
  hipLaunchKernelGGL(k_prefill_scan, dim3(1), dim3(kPThreads), 0, st, T, ws);
  hipLaunchKernelGGL(k_prefill_positions, dim3(L.ntiles), dim3(kPThreads), 0, st, T, ws);
  if (fmt == FMT_NVFP4) {
    hipLaunchKernelGGL(k_prefill_gateup<FMT_NVFP4>, dim3(L.max_items * (kI / 64)), dim3(kPThreads),
                       0, st, x, T, routed, shared, ws);
    hipLaunchKernelGGL(k_prefill_down<FMT_NVFP4>, dim3(L.max_items * (kH / kGBN)),
                       dim3(kPThreads), 0, st, T, routed, shared, ws);
  } else {
    hipLaunchKernelGGL(k_prefill_gateup<FMT_BF16>, dim3(L.max_items * (kI / 64)), dim3(kPThreads),
                       0, st, x, T, routed, shared, ws);
    hipLaunchKernelGGL(k_prefill_down<FMT_BF16>, dim3(L.max_items * (kH / kGBN)),
                       dim3(kPThreads), 0, st, T, routed, shared, ws);
  }
  const int nthr = T * (kH / 8);
  hipLaunchKernelGGL(k_prefill_combine, dim3((nthr + kPThreads - 1) / kPThreads), dim3(kPThreads),
                     0, st, T, ws, out);
  return hipGetLastError();
}

}  // namespace moe
