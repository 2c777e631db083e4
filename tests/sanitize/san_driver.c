/*
 * Drives every exported routine of the fp64 oracle and of the seeded input
 * generator on small shapes, for an AddressSanitizer + UndefinedBehavior-
 * Sanitizer build (CPU only; compiled and run by tests/test_sanitize.py).
 * Every buffer is allocated at exactly the size the routine's contract
 * states, so any read or write past it is reported.  A few cheap invariants
 * are checked as well (top-k ids distinct and ordered, routing weights
 * summing to 1, the sparse forward equal to the dense masked sum).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const void* w13;
  const uint8_t* w13s;
  const void* w2;
  const uint8_t* w2s;
  const float* glob;
  int32_t fmt;
} or_experts;
typedef struct {
  int32_t hidden, inter, n_experts, top_k, n_shared;
} or_shape;

double or_e2m1(uint8_t);
double or_e4m3(uint8_t);
double or_e8m0(uint8_t);
double or_bf16(uint16_t);
uint16_t or_bf16_rne(double);
void or_bf16_rne_array(const double*, int64_t, uint16_t*);
void or_dequant_f32(const uint8_t*, const uint8_t*, float, int64_t, int64_t, float*);
void or_dequant_f64(const uint8_t*, const uint8_t*, float, int64_t, int64_t, double*);
void or_router_logits(const uint16_t*, const uint16_t*, int32_t, int32_t, double*);
double or_sigmoid(double);
void or_topk(const double*, int32_t, int32_t, int32_t*, double*);
void or_route(const or_shape*, const uint16_t*, int32_t, const uint16_t*, int32_t*, double*,
              double*, double*);
void or_expert(const or_shape*, const or_experts*, int32_t, const double*, double*);
void or_forward(const or_shape*, const uint16_t*, int32_t, const uint16_t*, const or_experts*,
                const or_experts*, const int32_t*, double*, int32_t*, double*, double*);
void or_forward_dense(const or_shape*, const uint16_t*, int32_t, const uint16_t*,
                      const or_experts*, const or_experts*, double*);
void or_gemv_nvfp4(const uint16_t*, int32_t, int32_t, int32_t, const uint8_t*, const uint8_t*,
                   float, double*);
void or_rmsnorm_bf16(const uint16_t*, int32_t, int32_t, const uint16_t*, double, uint16_t*);
void or_quant_fp4_46(const float*, int64_t, uint8_t*, uint8_t*, float*, double*);
void or_forward_w4a4(const or_shape*, const uint16_t*, int32_t, const uint16_t*,
                     const or_experts*, const or_experts*, const int32_t*, const uint16_t*,
                     double*, int32_t*, double*, double*, uint16_t*);
int or_num_threads(void);
void or_set_num_threads(int);

uint64_t tg_splitmix_at(uint64_t, uint64_t);
uint64_t tg_stream_key(uint64_t, int32_t, int32_t, int32_t);
uint16_t tg_bf16_rne(float);
void tg_normal_bf16(uint64_t, int32_t, int32_t, int32_t, float, int64_t, uint16_t*);
void tg_normal_f32(uint64_t, int32_t, int32_t, int32_t, int64_t, float*);
uint8_t tg_e4m3_encode(float, float*);
uint8_t tg_e2m1_encode(float);
void tg_quantize_nvfp4(const uint16_t*, int64_t, int64_t, uint8_t*, uint8_t*, float*);
void tg_make_experts_nvfp4(uint64_t, int32_t, int32_t, int32_t, int32_t, int32_t, float,
                           uint8_t*, uint8_t*, uint8_t*, uint8_t*, float*);
void tg_make_experts_bf16(uint64_t, int32_t, int32_t, int32_t, int32_t, int32_t, float,
                          uint16_t*, uint16_t*);
void tg_quantize_mxfp8(const uint16_t*, int64_t, int64_t, uint8_t*, uint8_t*);
void tg_make_experts_mxfp8(uint64_t, int32_t, int32_t, int32_t, int32_t, int32_t, float,
                           uint8_t*, uint8_t*, uint8_t*, uint8_t*);
void tg_make_router(uint64_t, int32_t, int32_t, int32_t, float, uint16_t*);
void tg_make_x(uint64_t, int32_t, int32_t, uint16_t*);
int tg_num_threads(void);

static int g_fail = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      fprintf(stderr, "check failed: " __VA_ARGS__);    \
      fprintf(stderr, "\n");                            \
      g_fail = 1;                                       \
    }                                                   \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}

typedef struct {
  void *w13, *w2;
  uint8_t *w13s, *w2s;
  float* glob;
  or_experts X;
} experts_buf;

/* n experts of format fmt (0 NVFP4, 1 BF16, 2 MXFP8) at exact sizes */
static experts_buf make_experts(int fmt, int32_t layer, int32_t e0, int32_t n, int32_t H,
                                int32_t I) {
  experts_buf b;
  memset(&b, 0, sizeof(b));
  const int64_t mat = (int64_t)H * I;
  if (fmt == 0) {
    b.w13 = xmalloc((size_t)(n * 2 * mat / 2));
    b.w13s = xmalloc((size_t)(n * 2 * mat / 16));
    b.w2 = xmalloc((size_t)(n * mat / 2));
    b.w2s = xmalloc((size_t)(n * mat / 16));
    b.glob = xmalloc(sizeof(float) * (size_t)(n * 3));
    tg_make_experts_nvfp4(7, layer, e0, n, H, I, 0.05f, b.w13, b.w13s, b.w2, b.w2s, b.glob);
  } else if (fmt == 1) {
    b.w13 = xmalloc(2 * (size_t)(n * 2 * mat));
    b.w2 = xmalloc(2 * (size_t)(n * mat));
    tg_make_experts_bf16(7, layer, e0, n, H, I, 0.05f, b.w13, b.w2);
  } else {
    b.w13 = xmalloc((size_t)(n * 2 * mat));
    b.w13s = xmalloc((size_t)(n * 2 * mat / 32));
    b.w2 = xmalloc((size_t)(n * mat));
    b.w2s = xmalloc((size_t)(n * mat / 32));
    tg_make_experts_mxfp8(7, layer, e0, n, H, I, 0.05f, b.w13, b.w13s, b.w2, b.w2s);
  }
  b.X.w13 = b.w13; b.X.w13s = b.w13s; b.X.w2 = b.w2; b.X.w2s = b.w2s; b.X.glob = b.glob;
  b.X.fmt = fmt;
  return b;
}
static void free_experts(experts_buf* b) {
  free(b->w13); free(b->w2); free(b->w13s); free(b->w2s); free(b->glob);
}

static void check_route(const or_shape* S, int32_t B, const int32_t* ids, const double* w) {
  for (int32_t t = 0; t < B; ++t) {
    double sum = 0.0;
    for (int32_t j = 0; j < S->top_k; ++j) {
      const int32_t e = ids[t * S->top_k + j];
      CHECK(e >= 0 && e < S->n_experts, "id %d out of range", e);
      for (int32_t q = 0; q < j; ++q) CHECK(ids[t * S->top_k + q] != e, "id %d repeated", e);
      sum += w[t * S->top_k + j];
    }
    CHECK(fabs(sum - 1.0) < 1e-12, "weights of token %d sum to %.17g", t, sum);
  }
}

/* one MoE shape through route / forward / dense / W4A4 in one format */
static void run_shape(int fmt, int32_t H, int32_t I, int32_t E, int32_t K, int32_t NS,
                      int32_t B) {
  const or_shape S = {H, I, E, K, NS};
  experts_buf R = make_experts(fmt, 0, 0, E, H, I), Sh = make_experts(fmt, 0, E, NS, H, I);
  uint16_t* router = xmalloc(2 * (size_t)E * H);
  uint16_t* x = xmalloc(2 * (size_t)B * H);
  tg_make_router(7, 0, E, H, 0.02f, router);
  tg_make_x(11, B, H, x);
  int32_t* ids = xmalloc(sizeof(int32_t) * (size_t)B * K);
  double* w = xmalloc(sizeof(double) * (size_t)B * K);
  double* gap = xmalloc(sizeof(double) * (size_t)B);
  double* scores = xmalloc(sizeof(double) * (size_t)B * E);
  or_route(&S, x, B, router, ids, w, gap, scores);
  check_route(&S, B, ids, w);
  double* y = xmalloc(sizeof(double) * (size_t)B * H);
  double* yd = xmalloc(sizeof(double) * (size_t)B * H);
  or_forward(&S, x, B, router, &R.X, &Sh.X, NULL, y, ids, w, gap);
  check_route(&S, B, ids, w);
  or_forward_dense(&S, x, B, router, &R.X, &Sh.X, yd);
  double err = 0.0, ref = 0.0;
  for (int64_t i = 0; i < (int64_t)B * H; ++i) {
    err = fmax(err, fabs(y[i] - yd[i]));
    ref = fmax(ref, fabs(yd[i]));
  }
  CHECK(err <= 1e-12 * (ref + 1.0), "sparse vs dense forward differ by %.3g (fmt %d)", err, fmt);
  /* forced ids: reversed order of the chosen ones */
  int32_t* forced = xmalloc(sizeof(int32_t) * (size_t)B * K);
  for (int32_t t = 0; t < B; ++t)
    for (int32_t j = 0; j < K; ++j) forced[t * K + j] = ids[t * K + (K - 1 - j)];
  or_forward(&S, x, B, router, &R.X, &Sh.X, forced, y, ids, w, gap);
  check_route(&S, B, ids, w);
  double* d = xmalloc(sizeof(double) * (size_t)H);
  double* xe = xmalloc(sizeof(double) * (size_t)H);
  for (int32_t c = 0; c < H; ++c) xe[c] = or_bf16(x[c]);
  or_expert(&S, &R.X, E - 1, xe, d);
  or_expert(&S, &Sh.X, 0, xe, d);
  if (fmt == 0) {
    const int32_t nslot = K + NS;
    uint16_t* h = xmalloc(2 * (size_t)B * nslot * I);
    or_forward_w4a4(&S, x, B, router, &R.X, &Sh.X, NULL, NULL, y, ids, w, gap, h);
    check_route(&S, B, ids, w);
    or_forward_w4a4(&S, x, B, router, &R.X, &Sh.X, forced, h, y, ids, w, gap, NULL);
    free(h);
  }
  free(forced); free(d); free(xe); free(y); free(yd); free(ids); free(w); free(gap); free(scores);
  free(router); free(x);
  free_experts(&R);
  free_experts(&Sh);
}

int main(void) {
  /* formats: every byte / nibble, and RNE round trips */
  for (int i = 0; i < 16; ++i) CHECK(or_e2m1((uint8_t)i) == or_e2m1((uint8_t)i), "e2m1 %d", i);
  for (int i = 0; i < 256; ++i) (void)or_e4m3((uint8_t)i);
  for (int i = 0; i < 256; ++i) (void)or_e8m0((uint8_t)i);
  for (int i = 0; i < 65536; ++i) {
    const double v = or_bf16((uint16_t)i);
    if (v == v && v != 0.0) CHECK(or_bf16_rne(v) == (uint16_t)i, "bf16 round trip %04x", i);
  }
  {
    double v[5] = {1.0, -2.5, 1e-40, 3.0e38, 0.0};
    uint16_t o[5];
    or_bf16_rne_array(v, 5, o);
    float q;
    for (int i = 0; i < 100; ++i) (void)tg_e4m3_encode((float)i * 0.37f, &q);
    for (int i = -8; i <= 8; ++i) (void)tg_e2m1_encode((float)i * 0.75f);
    (void)tg_bf16_rne(1.5f);
    (void)tg_splitmix_at(tg_stream_key(1, 2, 3, 4), 5);
  }
  /* generator streams */
  {
    uint16_t* a = xmalloc(2 * 1000);
    float* f = xmalloc(4 * 1000);
    tg_normal_bf16(3, 1, 2, 3, 0.5f, 1000, a);
    tg_normal_f32(3, 1, 2, 3, 1000, f);
    free(a); free(f);
  }
  /* NVFP4 / MXFP8 packing and dequantisation of one [48][96] tensor */
  {
    const int64_t rows = 48, cols = 96;
    uint16_t* wt = xmalloc(2 * (size_t)(rows * cols));
    tg_normal_bf16(5, 0, 0, 1, 0.1f, rows * cols, wt);
    uint8_t* codes = xmalloc((size_t)(rows * cols / 2));
    uint8_t* sc = xmalloc((size_t)(rows * cols / 16));
    float g;
    tg_quantize_nvfp4(wt, rows, cols, codes, sc, &g);
    float* o32 = xmalloc(sizeof(float) * (size_t)(rows * cols));
    double* o64 = xmalloc(sizeof(double) * (size_t)(rows * cols));
    or_dequant_f32(codes, sc, g, rows, cols, o32);
    or_dequant_f64(codes, sc, g, rows, cols, o64);
    for (int64_t i = 0; i < rows * cols; ++i)
      CHECK(fabs((double)o32[i] - o64[i]) <= ldexp(fabs(o64[i]), -24),
            "f32 dequant is not o64 rounded once to fp32 at %ld", (long)i);
    uint8_t* el = xmalloc((size_t)(rows * cols));
    uint8_t* msc = xmalloc((size_t)(rows * cols / 32));
    tg_quantize_mxfp8(wt, rows, cols, el, msc);
    /* dense NVFP4 GEMV, B = 3 */
    uint16_t* xg = xmalloc(2 * 3 * (size_t)cols);
    tg_make_x(9, 3, (int32_t)cols, xg);
    double* yg = xmalloc(sizeof(double) * 3 * (size_t)rows);
    or_gemv_nvfp4(xg, 3, (int32_t)cols, (int32_t)rows, codes, sc, g, yg);
    /* RMSNorm of 3 rows */
    uint16_t* nw = xmalloc(2 * (size_t)cols);
    uint16_t* xn = xmalloc(2 * 3 * (size_t)cols);
    tg_normal_bf16(5, 0, 0, 9, 1.0f, cols, nw);
    or_rmsnorm_bf16(xg, 3, (int32_t)cols, nw, 1e-6, xn);
    /* four-over-six FP4 quantiser, including an all-zero block */
    float* v = xmalloc(sizeof(float) * 64);
    for (int i = 0; i < 64; ++i) v[i] = i < 16 ? 0.0f : sinf((float)i) * (float)i;
    uint8_t* qc = xmalloc(64);
    uint8_t* qs = xmalloc(64 / 16);
    double* qv = xmalloc(sizeof(double) * 64);
    float qg;
    or_quant_fp4_46(v, 64, qc, qs, &qg, qv);
    free(wt); free(codes); free(sc); free(o32); free(o64); free(el); free(msc); free(xg);
    free(yg); free(nw); free(xn); free(v); free(qc); free(qs); free(qv);
  }
  /* top-k with ties (lowest index first) */
  {
    double s[8] = {0.5, 0.9, 0.5, 0.9, 0.1, 0.5, 0.2, 0.9};
    int32_t ids[4];
    double gap;
    or_topk(s, 8, 4, ids, &gap);
    CHECK(ids[0] == 1 && ids[1] == 3 && ids[2] == 7 && ids[3] == 0, "top-k tie order");
    (void)or_sigmoid(-3.0);
  }
  /* MoE shapes: NVFP4 (with W4A4), BF16, MXFP8; B = 1 and a ragged B = 5 */
  or_set_num_threads(2);
  run_shape(0, 64, 32, 16, 4, 1, 1);
  run_shape(0, 64, 32, 16, 4, 2, 5);
  run_shape(1, 64, 32, 12, 3, 1, 5);
  run_shape(2, 64, 32, 12, 3, 1, 2);
  (void)or_num_threads();
  (void)tg_num_threads();
  if (g_fail) return 1;
  printf("sanitized oracle and generator: OK\n");
  return 0;
}
