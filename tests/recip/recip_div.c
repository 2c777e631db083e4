/* Host check of the W4A4 quantiser's division through a correctly rounded
 * reciprocal: q = RN(v y), r = RN(v - d q) by FMA, q' = RN(q + r y), with
 * y = RN(1 / d), against IEEE division v / d (x86-64 SSE division and libm's
 * fmaf are correctly rounded, as gfx950's v_mul_f32 / v_fma_f32 are).
 *
 *  part 1: every bf16 significand of v (128) against every fp32 significand
 *          of d (2^23), exponents 0 (quotients in (1/2, 2)): q' == v / d bit
 *          for bit.  Every step scales exactly with the exponents while the
 *          values stay normal, so this covers the normal range.
 *  part 2: every bf16 value of v (subnormals, zeros, both signs) against
 *          divisors spread over [2^-64, 2^64], for the quotients the
 *          quantiser can meet (|v / d| <= 16: v is at most the block
 *          maximum bmax and d is the E4M3 scale of bmax / M times the global,
 *          which rounds down by at most a factor 1.5 (among the subnormal
 *          scales), so |v / d| <= 1.5 M = 9; a saturated scale leaves it at
 *          most 2688 / 448 = 6): the E2M1 code of q' equals
 *          the code of v / d, and q' == v / d bit for bit wherever
 *          |v / d| >= 1/8.
 *  part 3: every bf16 value of v (the block maxima) divided by 6 through
 *          the reciprocal RN(1 / 6) = 0x1.555556p-3: bit for bit, subnormal
 *          quotients included.
 * Prints "mismatches 0 0 0" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float div_by_recip(float v, float d, float y) {
  const float q = v * y;
  const float r = fmaf(-d, q, v);
  return copysignf(fmaf(r, y, q), v);
}

/* E2M1 nearest-even with saturation at 6, by the definition's comparisons */
static float e2m1(float x) {
  const float a = fabsf(x);
  float c;
  if (a <= 0.25f) c = 0.0f;
  else if (a < 0.75f) c = 0.5f;
  else if (a <= 1.25f) c = 1.0f;
  else if (a < 1.75f) c = 1.5f;
  else if (a <= 2.5f) c = 2.0f;
  else if (a < 3.5f) c = 3.0f;
  else if (a <= 5.0f) c = 4.0f;
  else c = 6.0f;
  return copysignf(c, x);
}

int main(void) {
  long bad1 = 0, bad2 = 0;
#pragma omp parallel for reduction(+ : bad1) schedule(static)
  for (uint32_t dm = 0; dm < (1u << 23); ++dm) {
    const float d = fb((127u << 23) | dm);
    const float y = 1.0f / d;
    for (uint32_t vm = 0; vm < 256; ++vm) {   /* both signs */
      const float v = fb(((vm >> 7) << 31) | (127u << 23) | ((vm & 127u) << 16));
      if (bf(div_by_recip(v, d, y)) != bf(v / d)) bad1++;
    }
  }
  /* divisors: 2^e (1 + k / 61) for e = -64 .. 63, k = 0 .. 60, plus 2^64 */
#pragma omp parallel for reduction(+ : bad2) schedule(dynamic)
  for (int e = -64; e <= 64; ++e) {
    for (int k = 0; k < (e == 64 ? 1 : 61); ++k) {
      const float d = ldexpf(1.0f + (float)k / 61.0f, e);
      const float y = 1.0f / d;
      for (uint32_t b = 0; b < 65536u; ++b) {
        const float v = fb(b << 16);
        if (isnan(v) || isinf(v)) continue;
        const float ref = v / d, got = div_by_recip(v, d, y);
        if (!(fabsf(ref) <= 16.0f)) continue;
        if (bf(e2m1(got)) != bf(e2m1(ref))) bad2++;
        else if (fabsf(ref) >= 0.125f && bf(got) != bf(ref)) bad2++;
      }
    }
  }
  long bad3 = 0;
  const float y6 = 0x1.555556p-3f;
  if (bf(y6) != bf(1.0f / 6.0f)) bad3++;
  for (uint32_t b = 0; b < 65536u; ++b) {
    const float v = fb(b << 16);
    if (isnan(v) || isinf(v)) continue;
    if (bf(div_by_recip(v, 6.0f, y6)) != bf(v / 6.0f)) bad3++;
  }
  printf("mismatches %ld %ld %ld\n", bad1, bad2, bad3);
  return (bad1 || bad2 || bad3) ? 1 : 0;
}
