/*
 * Seeded synthetic inputs for the Flint-style MoE decode layer.
 *
 * This module produces inputs only: activations x, router weights and expert
 * weights, the latter either kept as bf16 or packed to NVFP4.  It holds none
 * of the layer's arithmetic (no decode of packed values, no GEMV, no routing),
 * so that the fp64 oracle and the HIP kernels, which both consume its output,
 * stay independent of each other.
 *
 * Random stream.  splitmix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: output n
 * of a stream with state `key` is mix(key + n * 0x9E3779B97F4A7C15).  A stream
 * key is derived from (seed, layer, expert, tensor) by chaining the mixer.
 * Element i of a tensor consumes outputs 3i+1, 3i+2, 3i+3.
 *
 * Normal draws.  Irwin-Hall with twelve 16-bit uniforms (four per 64-bit
 * output): z = (sum - 12 * 32767.5) / 65536, which has mean 0 and standard
 * deviation 1 up to a 2^-32 relative term.  All integer until the last,
 * exact, division, so the value depends on nothing but the counter.  The
 * standard deviation sigma is applied in fp32 and the result is rounded to
 * bf16 (round to nearest, ties to even).
 *
 * NVFP4 packing (the format the Flint pages name for their checkpoint:
 * "Day-0 Support for Flint on vLLM", section "Model architecture"; 16-element
 * blocks whose FP4 maximum is 6, as the Inkling-2-Small article describes in
 * its 48-layer MoE section).  Per tensor [rows][cols], blocks of 16 along cols:
 *   global = fp32(tensor_amax / 2688)                  (2688 = 6 * 448)
 *   s      = fp32(fp32(block_amax / 6) / global), rounded to E4M3FN (RNE,
 *            saturating at 448) -> byte and value q
 *   code   = E2M1 rounding (RNE, saturating at 6) of fp32(w / fp32(q*global))
 * Codes are packed two per byte, element 2j in bits 0-3 of byte j and
 * element 2j+1 in bits 4-7.  An all-zero tensor gets global 0, scale bytes 0
 * and codes 0; an all-zero block gets scale byte 0 and codes 0.
 *
 * Tensor ids: 0 router, 1 gate, 2 up, 3 down, 4 activations x.
 * Expert ids: 0..E-1 routed, E = the shared expert (for E = 256 that is 256).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TG_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t tg_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* n-th output (n >= 1) of the splitmix64 stream whose state starts at key. */
uint64_t tg_splitmix_at(uint64_t key, uint64_t n) { return tg_mix(key + n * TG_GAMMA); }

uint64_t tg_stream_key(uint64_t seed, int32_t layer, int32_t expert, int32_t tensor) {
  uint64_t k = tg_mix(seed + TG_GAMMA);
  k = tg_mix((k ^ (uint64_t)(uint32_t)layer) + TG_GAMMA);
  k = tg_mix((k ^ (uint64_t)(uint32_t)expert) + TG_GAMMA);
  k = tg_mix((k ^ (uint64_t)(uint32_t)tensor) + TG_GAMMA);
  return k;
}

static inline float tg_normal_at(uint64_t key, uint64_t i) {
  int64_t s = 0;
  for (int j = 1; j <= 3; ++j) {
    uint64_t r = tg_mix(key + (3 * i + (uint64_t)j) * TG_GAMMA);
    s += (int64_t)(r & 0xFFFF) + (int64_t)((r >> 16) & 0xFFFF) +
         (int64_t)((r >> 32) & 0xFFFF) + (int64_t)(r >> 48);
  }
  /* 12 * 32767.5 = 393210; the difference is an integer of magnitude < 2^20. */
  return (float)(s - 393210) / 65536.0f;
}

/* fp32 -> bf16 bits, round to nearest even.  NaN is kept quiet. */
uint16_t tg_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static inline float tg_bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Standard normal draws, times sigma in fp32, rounded to bf16. */
void tg_normal_bf16(uint64_t seed, int32_t layer, int32_t expert, int32_t tensor, float sigma,
                    int64_t n, uint16_t* out) {
  uint64_t key = tg_stream_key(seed, layer, expert, tensor);
  for (int64_t i = 0; i < n; ++i) out[i] = tg_bf16_rne(tg_normal_at(key, (uint64_t)i) * sigma);
}

/* The raw fp32 normal draws (before sigma and bf16), for distribution tests. */
void tg_normal_f32(uint64_t seed, int32_t layer, int32_t expert, int32_t tensor, int64_t n,
                   float* out) {
  uint64_t key = tg_stream_key(seed, layer, expert, tensor);
  for (int64_t i = 0; i < n; ++i) out[i] = tg_normal_at(key, (uint64_t)i);
}

/* Round a positive finite s to E4M3FN (bias 7, 3 mantissa bits, largest
 * finite 448, subnormal step 2^-9), ties to even, saturating at 448.
 * Returns the byte and writes the rounded value to *q. */
uint8_t tg_e4m3_encode(float s, float* q) {
  if (!(s > 0.0f)) { *q = 0.0f; return 0; }
  if (s >= 448.0f) { *q = 448.0f; return 0x7E; }
  if (s < 0.015625f) {                      /* below 2^-6: subnormal grid of 2^-9 */
    float m = rintf(ldexpf(s, 9));          /* exact scaling, then RNE to an integer */
    if (m >= 8.0f) { *q = 0.015625f; return 0x08; }
    *q = ldexpf(m, -9);
    return (uint8_t)m;
  }
  int k;
  float f = frexpf(s, &k);                  /* s = f * 2^k, f in [0.5, 1) */
  int e = k - 1;                            /* s = (2f) * 2^e, 2f in [1, 2) */
  float m = rintf((2.0f * f - 1.0f) * 8.0f);/* 3 fractional bits, RNE */
  if (m >= 8.0f) { m = 0.0f; e += 1; }
  if (e > 8 || (e == 8 && m > 6.0f)) { *q = 448.0f; return 0x7E; }
  *q = ldexpf(1.0f + m / 8.0f, e);
  return (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Round v to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} (RNE, saturating at
 * 6) and return the 4-bit code: bit 3 the sign of v, bits 0-2 the grid index.
 * The grid index is the number of decision points below |v|; a point that is
 * a tie between two grid values counts only when |v| is strictly above it if
 * the lower neighbour has the even (zero) mantissa bit, else from it on. */
static inline uint8_t tg_e2m1_code(float v) {
  float a = fabsf(v);
  int m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
          (a >= 3.5f) + (a > 5.0f);
  return (uint8_t)((signbit(v) ? 8 : 0) | m);
}

uint8_t tg_e2m1_encode(float v) { return tg_e2m1_code(v); }

/* Pack one bf16 tensor [rows][cols] (cols a multiple of 16) to NVFP4. */
void tg_quantize_nvfp4(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* codes,
                       uint8_t* scales, float* global_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < rows * cols; ++i) {
    float a = fabsf(tg_bf16_to_float(w[i]));
    if (a > amax) amax = a;
  }
  float global = amax / 2688.0f;
  *global_out = global;
  int64_t nb = cols / 16;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* blk = w + r * cols + b * 16;
      uint8_t* cb = codes + r * (cols / 2) + b * 8;
      float bmax = 0.0f;
      for (int j = 0; j < 16; ++j) {
        float a = fabsf(tg_bf16_to_float(blk[j]));
        if (a > bmax) bmax = a;
      }
      float q = 0.0f;
      uint8_t sb = 0;
      if (global > 0.0f && bmax > 0.0f) sb = tg_e4m3_encode((bmax / 6.0f) / global, &q);
      scales[r * nb + b] = sb;
      if (q == 0.0f) { memset(cb, 0, 8); continue; }
      float denom = q * global;
      float v[16];
      for (int j = 0; j < 16; ++j) v[j] = tg_bf16_to_float(blk[j]) / denom;
      for (int j = 0; j < 8; ++j)
        cb[j] = (uint8_t)(tg_e2m1_code(v[2 * j]) | (tg_e2m1_code(v[2 * j + 1]) << 4));
    }
  }
}

/* One expert tensor drawn from its stream and packed; tmp holds rows*cols bf16. */
static void tg_make_tensor_nvfp4(uint64_t seed, int32_t layer, int32_t expert, int32_t tensor,
                                 float sigma, int64_t rows, int64_t cols, uint16_t* tmp,
                                 uint8_t* codes, uint8_t* scales, float* global) {
  tg_normal_bf16(seed, layer, expert, tensor, sigma, rows * cols, tmp);
  tg_quantize_nvfp4(tmp, rows, cols, codes, scales, global);
}

/*
 * Expert set of n experts starting at expert id e0, NVFP4.  Layout:
 *   w13   u8  [n][2][I][H/2]   (gate, up)      w13s u8 [n][2][I][H/16]
 *   w2    u8  [n][H][I/2]                      w2s  u8 [n][H][I/16]
 *   glob  f32 [n][3]           (gate, up, down)
 * Work is split over (expert, tensor) pairs with OpenMP.
 */
void tg_make_experts_nvfp4(uint64_t seed, int32_t layer, int32_t e0, int32_t n, int32_t H,
                           int32_t I, float sigma, uint8_t* w13, uint8_t* w13s, uint8_t* w2,
                           uint8_t* w2s, float* glob) {
  int64_t mat = (int64_t)H * I;
  #pragma omp parallel
  {
    uint16_t* tmp = (uint16_t*)malloc((size_t)mat * sizeof(uint16_t));
    #pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < (int64_t)n * 3; ++task) {
      int64_t e = task / 3;
      int t = (int)(task % 3);
      if (t < 2) {
        tg_make_tensor_nvfp4(seed, layer, e0 + (int32_t)e, 1 + t, sigma, I, H, tmp,
                             w13 + (e * 2 + t) * (mat / 2), w13s + (e * 2 + t) * (mat / 16),
                             glob + e * 3 + t);
      } else {
        tg_make_tensor_nvfp4(seed, layer, e0 + (int32_t)e, 3, sigma, H, I, tmp,
                             w2 + e * (mat / 2), w2s + e * (mat / 16), glob + e * 3 + 2);
      }
    }
    free(tmp);
  }
}

/* Expert set kept in bf16: w13 [n][2][I][H], w2 [n][H][I]. */
void tg_make_experts_bf16(uint64_t seed, int32_t layer, int32_t e0, int32_t n, int32_t H,
                          int32_t I, float sigma, uint16_t* w13, uint16_t* w2) {
  int64_t mat = (int64_t)H * I;
  #pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < (int64_t)n * 3; ++task) {
    int64_t e = task / 3;
    int t = (int)(task % 3);
    uint16_t* dst = t < 2 ? w13 + (e * 2 + t) * mat : w2 + e * mat;
    tg_normal_bf16(seed, layer, e0 + (int32_t)e, 1 + t, sigma, mat, dst);
  }
}

/*
 * MXFP8 packing (OCP Microscaling Formats v1.0, conversion to an MX format):
 * per block of 32 consecutive values, shared exponent
 *   X = 2^(floor(log2(amax)) - 8)      (8 = exponent of E4M3's largest normal)
 * clamped to the E8M0 range [-127, 127], stored as the byte 127 + log2 X; each
 * element is v / X rounded to E4M3FN (nearest-even, saturating at +-448).  An
 * all-zero block gets the byte 0 and zero elements.
 */
static uint8_t tg_e4m3_signed(float v) {
  float q;
  uint8_t b = tg_e4m3_encode(fabsf(v), &q);
  return (uint8_t)(b | (signbit(v) ? 0x80 : 0));
}

void tg_quantize_mxfp8(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* el,
                       uint8_t* scales) {
  int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* blk = w + r * cols + b * 32;
      uint8_t* eb = el + r * cols + b * 32;
      float amax = 0.0f;
      for (int j = 0; j < 32; ++j) {
        float a = fabsf(tg_bf16_to_float(blk[j]));
        if (a > amax) amax = a;
      }
      if (amax == 0.0f) {
        scales[r * nb + b] = 0;
        memset(eb, 0, 32);
        continue;
      }
      int k;
      (void)frexpf(amax, &k);                   /* amax in [2^(k-1), 2^k) */
      int xe = (k - 1) - 8;
      if (xe < -127) xe = -127;
      if (xe > 127) xe = 127;
      scales[r * nb + b] = (uint8_t)(xe + 127);
      for (int j = 0; j < 32; ++j) eb[j] = tg_e4m3_signed(ldexpf(tg_bf16_to_float(blk[j]), -xe));
    }
}

/* Expert set in MXFP8: w13 u8 [n][2][I][H], w13s u8 [n][2][I][H/32],
 * w2 u8 [n][H][I], w2s u8 [n][H][I/32]. */
void tg_make_experts_mxfp8(uint64_t seed, int32_t layer, int32_t e0, int32_t n, int32_t H,
                           int32_t I, float sigma, uint8_t* w13, uint8_t* w13s, uint8_t* w2,
                           uint8_t* w2s) {
  int64_t mat = (int64_t)H * I;
  #pragma omp parallel
  {
    uint16_t* tmp = (uint16_t*)malloc((size_t)mat * sizeof(uint16_t));
    #pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < (int64_t)n * 3; ++task) {
      int64_t e = task / 3;
      int t = (int)(task % 3);
      tg_normal_bf16(seed, layer, e0 + (int32_t)e, 1 + t, sigma, mat, tmp);
      if (t < 2)
        tg_quantize_mxfp8(tmp, I, H, w13 + (e * 2 + t) * mat, w13s + (e * 2 + t) * (mat / 32));
      else
        tg_quantize_mxfp8(tmp, H, I, w2 + e * mat, w2s + e * (mat / 32));
    }
    free(tmp);
  }
}

/* Router [E][H] bf16, split over rows with OpenMP (row r uses elements r*H..). */
void tg_make_router(uint64_t seed, int32_t layer, int32_t E, int32_t H, float sigma,
                    uint16_t* out) {
  uint64_t key = tg_stream_key(seed, layer, 0, 0);
  #pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < E; ++r)
    for (int64_t c = 0; c < H; ++c)
      out[r * H + c] = tg_bf16_rne(tg_normal_at(key, (uint64_t)(r * H + c)) * sigma);
}

/* Activations x [T][H] bf16, standard normal; one stream per seed. */
void tg_make_x(uint64_t seed, int32_t T, int32_t H, uint16_t* out) {
  uint64_t key = tg_stream_key(seed, 0, 0, 4);
  #pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < H; ++c)
      out[t * H + c] = tg_bf16_rne(tg_normal_at(key, (uint64_t)(t * H + c)));
}

int tg_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
