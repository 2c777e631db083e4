/*
 * fp64 CPU oracle for the Flint-style small-batch MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no code,
 * header, table or helper with the HIP library; it reads the same packed
 * input bytes and computes the layer from its definition, slowly, in fp64.
 *
 * What it follows (pages: "Day-0 Support for Flint on vLLM", the vLLM blog on
 * Recursive's Flint, in its zh / ja / fr / ko renderings; and the AREX article
 * on vLLM's Day-0 support for Inkling-2-Small, cited only where marked):
 *  - Model architecture section: 256 experts chosen by a sigmoid top-6, plus
 *    one shared expert that every token uses.
 *  - Model architecture section: the NVFP4 checkpoint runs weight-only
 *    (W4A16) with BF16 activations.
 *  - Optimization section, Fig. 2 change list: the router and the expert
 *    GEMVs read only the selected experts' weights, i.e. the layer is the
 *    sparse evaluation of the dense masked sum (pinned by or_forward_dense).
 *  - Optimization section: the SiLU kernels (SiLU-gated expert FFN).
 *  - Optimization section, low-latency path: routing and the expert combine.
 *  - Optimization section, low-latency path: the pre-MoE RMSNorm and the
 *    residual add fused into the adjacent GEMVs (or_rmsnorm_bf16; the
 *    residual is a plain fp64 addition done by the Python wrapper).
 *  - Inkling-2-Small article, 48-layer MoE section: NVFP4 blocks of 16 with
 *    an FP4 maximum of 6; accuracy section: the router is kept in FP32 (the
 *    oracle keeps it in fp64).
 * Readings where the pages are silent (no router bias or scaling factor,
 * ties to the lower expert index, renormalisation w = s / sum s, shared
 * expert with weight 1, element 2j in the low nibble) are the plainest ones;
 * the repository's design notes list each.
 *
 * Formats decoded from their published closed forms:
 *  - E2M1 (OCP Microscaling Formats v1.0, FP4): bit 3 sign, bits 2..1
 *    exponent with bias 1, bit 0 mantissa; exponent 0 is subnormal m * 0.5.
 *  - E4M3FN (OCP 8-bit Floating Point v1.0): bit 7 sign, bits 6..3 exponent
 *    with bias 7, bits 2..0 mantissa; exponent 0 is subnormal m/8 * 2^-6;
 *    S.1111.111 is NaN (never produced by the input generator).
 *  - bf16: the upper 16 bits of an IEEE binary32.
 *
 * Numerics: every weight is used at its exact fp64 value
 * e2m1 * e4m3 * global (at most 30 significant bits, so exact in fp64);
 * every sum runs sequentially in index order; OpenMP only splits independent
 * rows or tokens, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#else
static int omp_in_parallel(void) { return 0; }
#endif

/* ------------------------------------------------------------------ formats */

double or_e2m1(uint8_t nib) {
  int sign = (nib >> 3) & 1;
  int ex = (nib >> 1) & 3;
  int man = nib & 1;
  double mag = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
  return sign ? -mag : mag;
}

double or_e4m3(uint8_t byte) {
  int sign = (byte >> 7) & 1;
  int ex = (byte >> 3) & 15;
  int man = byte & 7;
  double mag;
  if (ex == 15 && man == 7) return NAN;
  if (ex == 0) mag = ldexp(man / 8.0, -6);
  else mag = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -mag : mag;
}

/* E8M0 (OCP Microscaling Formats v1.0, the shared block scale of the MX
 * formats): an unsigned biased exponent, 2^(b - 127); 0xFF is NaN. */
double or_e8m0(uint8_t byte) {
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

double or_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Lookup tables filled from the closed forms above on first use.  The ready
 * flag is read with acquire and set with release ordering (GCC's __atomic
 * builtins), so a thread that sees it set also sees the filled tables. */
static double g_e2m1[16], g_e4m3[256];
static int g_tables_ready = 0;
static void or_tables(void) {
  if (__atomic_load_n(&g_tables_ready, __ATOMIC_ACQUIRE)) return;
  #pragma omp critical(or_tables_init)
  {
    if (!__atomic_load_n(&g_tables_ready, __ATOMIC_RELAXED)) {
      for (int i = 0; i < 16; ++i) g_e2m1[i] = or_e2m1((uint8_t)i);
      for (int i = 0; i < 256; ++i) g_e4m3[i] = or_e4m3((uint8_t)i);
      __atomic_store_n(&g_tables_ready, 1, __ATOMIC_RELEASE);
    }
  }
}

/* ------------------------------------------------------------ weight access */

enum { OR_NVFP4 = 0, OR_BF16 = 1, OR_MXFP8 = 2 };

/* One expert set (n experts).  NVFP4: w13 u8 [n][2][I][H/2], w13s u8
 * [n][2][I][H/16], w2 u8 [n][H][I/2], w2s u8 [n][H][I/16], glob f32 [n][3].
 * BF16: w13 u16 [n][2][I][H], w2 u16 [n][H][I]; w13s, w2s, glob unused.
 * MXFP8 (OCP MX, the expert format of the Inkling-2-Small article's last 8
 * layers, 48-layer MoE section): E4M3 elements w13 u8 [n][2][I][H], w2 u8
 * [n][H][I], one E8M0 scale per 32 consecutive inputs w13s u8 [n][2][I][H/32],
 * w2s u8 [n][H][I/32]; no tensor scale (glob unused). */
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

/* Row r of matrix t (0 gate, 1 up, 2 down) of expert e, dequantised to fp64.
 * gate/up rows have H columns; down rows have I columns. */
static void or_row(const or_experts* X, int64_t e, int t, int64_t r, int64_t H, int64_t I,
                   double* out) {
  int64_t rows = t < 2 ? I : H;
  int64_t cols = t < 2 ? H : I;
  if (X->fmt == OR_BF16) {
    const uint16_t* base = t < 2 ? (const uint16_t*)X->w13 + ((e * 2 + t) * rows) * cols
                                 : (const uint16_t*)X->w2 + (e * rows) * cols;
    for (int64_t c = 0; c < cols; ++c) out[c] = or_bf16(base[r * cols + c]);
    return;
  }
  if (X->fmt == OR_MXFP8) {
    const uint8_t* el = t < 2 ? (const uint8_t*)X->w13 + ((e * 2 + t) * rows) * cols
                              : (const uint8_t*)X->w2 + (e * rows) * cols;
    const uint8_t* sc = t < 2 ? X->w13s + ((e * 2 + t) * rows) * (cols / 32)
                              : X->w2s + (e * rows) * (cols / 32);
    for (int64_t c = 0; c < cols; ++c)
      out[c] = g_e4m3[el[r * cols + c]] * or_e8m0(sc[r * (cols / 32) + c / 32]);
    return;
  }
  const uint8_t* codes = t < 2 ? (const uint8_t*)X->w13 + ((e * 2 + t) * rows) * (cols / 2)
                               : (const uint8_t*)X->w2 + (e * rows) * (cols / 2);
  const uint8_t* scales = t < 2 ? X->w13s + ((e * 2 + t) * rows) * (cols / 16)
                                : X->w2s + (e * rows) * (cols / 16);
  double global = (double)X->glob[e * 3 + t];
  for (int64_t c = 0; c < cols; ++c) {
    uint8_t byte = codes[r * (cols / 2) + c / 2];
    uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
    out[c] = g_e2m1[nib] * g_e4m3[scales[r * (cols / 16) + c / 16]] * global;
  }
}

/* Dequantise one NVFP4 tensor [rows][cols] to fp32 with a single rounding:
 * fp32(e2m1 * e4m3 * global), the product being exact in fp64. */
void or_dequant_f32(const uint8_t* codes, const uint8_t* scales, float global, int64_t rows,
                    int64_t cols, float* out) {
  or_tables();
  #pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t byte = codes[r * (cols / 2) + c / 2];
      uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * cols + c] = (float)(g_e2m1[nib] * g_e4m3[scales[r * (cols / 16) + c / 16]] *
                                  (double)global);
    }
}

/* The same tensor at its exact fp64 value. */
void or_dequant_f64(const uint8_t* codes, const uint8_t* scales, float global, int64_t rows,
                    int64_t cols, double* out) {
  or_tables();
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t byte = codes[r * (cols / 2) + c / 2];
      uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * cols + c] = g_e2m1[nib] * g_e4m3[scales[r * (cols / 16) + c / 16]] * (double)global;
    }
}

/* ------------------------------------------------------------------ routing */

/* logits[e] = sum_k W_r[e][k] * x[k], fp64, k ascending. */
void or_router_logits(const uint16_t* x, const uint16_t* router, int32_t E, int32_t H,
                      double* logits) {
  #pragma omp parallel for schedule(static) if (!omp_in_parallel())
  for (int64_t e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int64_t k = 0; k < H; ++k) acc += or_bf16(router[e * H + k]) * or_bf16(x[k]);
    logits[e] = acc;
  }
}

double or_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* The k largest scores, ordered by (score descending, expert index ascending).
 * gap = s_(k) - s_(k+1), the distance between the last chosen and the first
 * rejected score (+inf when every expert is chosen). */
void or_topk(const double* scores, int32_t E, int32_t k, int32_t* ids, double* gap) {
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int32_t i = 0; i < E; ++i) order[i] = i;
  /* insertion sort on (score desc, index asc) */
  for (int32_t i = 1; i < E; ++i) {
    int32_t v = order[i];
    int32_t j = i - 1;
    while (j >= 0 && (scores[order[j]] < scores[v] ||
                      (scores[order[j]] == scores[v] && order[j] > v))) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = v;
  }
  for (int32_t i = 0; i < k; ++i) ids[i] = order[i];
  *gap = k < E ? scores[order[k - 1]] - scores[order[k]] : INFINITY;
  free(order);
}

/* Routing of one token: ids [k] (score descending), weights w [k] = s / sum s,
 * gap as in or_topk; scores_out [E] (nullable) receives every sigmoid score.
 * When forced is non-null its k ids are used instead of the top-k. */
static void or_route_token(const or_shape* S, const uint16_t* x, const uint16_t* router,
                           const int32_t* forced, int32_t* ids, double* w, double* gap,
                           double* scores_out) {
  int32_t E = S->n_experts, k = S->top_k;
  double* logits = (double*)malloc(sizeof(double) * (size_t)E);
  double* scores = (double*)malloc(sizeof(double) * (size_t)E);
  or_router_logits(x, router, E, S->hidden, logits);
  for (int32_t e = 0; e < E; ++e) scores[e] = or_sigmoid(logits[e]);
  or_topk(scores, E, k, ids, gap);
  if (forced) for (int32_t j = 0; j < k; ++j) ids[j] = forced[j];
  double sum = 0.0;
  for (int32_t j = 0; j < k; ++j) sum += scores[ids[j]];
  for (int32_t j = 0; j < k; ++j) w[j] = scores[ids[j]] / sum;
  if (scores_out) memcpy(scores_out, scores, sizeof(double) * (size_t)E);
  free(logits);
  free(scores);
}

void or_route(const or_shape* S, const uint16_t* x, int32_t B, const uint16_t* router,
              int32_t* ids, double* w, double* gap, double* scores) {
  #pragma omp parallel for schedule(static) if (B > 1)
  for (int32_t t = 0; t < B; ++t)
    or_route_token(S, x + (int64_t)t * S->hidden, router, NULL, ids + (int64_t)t * S->top_k,
                   w + (int64_t)t * S->top_k, gap + t,
                   scores ? scores + (int64_t)t * S->n_experts : NULL);
}

/* ------------------------------------------------------------------ experts */

/* d = D_e (SiLU(G_e x) * (U_e x)) for one token x (fp64, length H). */
void or_expert(const or_shape* S, const or_experts* X, int32_t e, const double* x, double* d) {
  int64_t H = S->hidden, I = S->inter;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  or_tables();
  #pragma omp parallel if (!omp_in_parallel())
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    #pragma omp for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
      double g = 0.0, u = 0.0;
      or_row(X, e, 0, i, H, I, row);
      for (int64_t k = 0; k < H; ++k) g += row[k] * x[k];
      or_row(X, e, 1, i, H, I, row);
      for (int64_t k = 0; k < H; ++k) u += row[k] * x[k];
      h[i] = g * or_sigmoid(g) * u;
    }
    #pragma omp for schedule(static)
    for (int64_t j = 0; j < H; ++j) {
      double acc = 0.0;
      or_row(X, e, 2, j, H, I, row);
      for (int64_t i = 0; i < I; ++i) acc += row[i] * h[i];
      d[j] = acc;
    }
    free(row);
  }
  free(h);
}

static int or_cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* One token of the layer: y = sum_j w_j d_{e_j} (ascending expert id), then
 * + d_s of each shared expert s = 0 .. n_shared - 1 in turn (weight 1; the
 * Flint page has one shared expert, the Inkling article's earlier model two,
 * Inkling-2-Small none). */
static void or_forward_token(const or_shape* S, const uint16_t* xb, const uint16_t* router,
                             const or_experts* routed, const or_experts* shared,
                             const int32_t* forced, double* y, int32_t* ids, double* w,
                             double* gap) {
  int64_t H = S->hidden;
  int32_t k = S->top_k;
  double* x = (double*)malloc(sizeof(double) * (size_t)H);
  double* d = (double*)malloc(sizeof(double) * (size_t)H);
  int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  for (int64_t c = 0; c < H; ++c) x[c] = or_bf16(xb[c]);
  or_route_token(S, xb, router, forced, ids, w, gap, NULL);
  memcpy(sorted, ids, sizeof(int32_t) * (size_t)k);
  qsort(sorted, (size_t)k, sizeof(int32_t), or_cmp_i32);
  for (int64_t c = 0; c < H; ++c) y[c] = 0.0;
  for (int32_t s = 0; s < k; ++s) {
    double wj = 0.0;
    for (int32_t j = 0; j < k; ++j) if (ids[j] == sorted[s]) wj = w[j];
    or_expert(S, routed, sorted[s], x, d);
    for (int64_t c = 0; c < H; ++c) y[c] += wj * d[c];
  }
  for (int32_t s = 0; shared && s < S->n_shared; ++s) {
    or_expert(S, shared, s, x, d);
    for (int64_t c = 0; c < H; ++c) y[c] += d[c];
  }
  free(x);
  free(d);
  free(sorted);
}

/* The layer for B tokens.  y [B][H] fp64; ids [B][k]; w [B][k]; gap [B].
 * forced (nullable) [B][k]: use these expert ids instead of the top-k. */
void or_forward(const or_shape* S, const uint16_t* x, int32_t B, const uint16_t* router,
                const or_experts* routed, const or_experts* shared, const int32_t* forced,
                double* y, int32_t* ids, double* w, double* gap) {
  or_tables();
  int64_t H = S->hidden, k = S->top_k;
  #pragma omp parallel for schedule(dynamic, 1) if (B > 1)
  for (int32_t t = 0; t < B; ++t)
    or_forward_token(S, x + t * H, router, routed, shared, forced ? forced + t * k : NULL,
                     y + t * H, ids + t * k, w + t * k, gap + t);
}

/* Dense evaluation with masked weights: every routed expert is computed and
 * scaled by m_e = w_e if e was selected and 0 otherwise, summed in ascending
 * expert id, then the shared expert is added.  Equal to or_forward bit for bit. */
void or_forward_dense(const or_shape* S, const uint16_t* xb, int32_t B, const uint16_t* router,
                      const or_experts* routed, const or_experts* shared, double* y) {
  or_tables();
  int64_t H = S->hidden;
  int32_t E = S->n_experts, k = S->top_k;
  double* x = (double*)malloc(sizeof(double) * (size_t)H);
  double* d = (double*)malloc(sizeof(double) * (size_t)H);
  double* m = (double*)malloc(sizeof(double) * (size_t)E);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* w = (double*)malloc(sizeof(double) * (size_t)k);
  for (int32_t t = 0; t < B; ++t) {
    double gap;
    for (int64_t c = 0; c < H; ++c) x[c] = or_bf16(xb[t * H + c]);
    or_route_token(S, xb + t * H, router, NULL, ids, w, &gap, NULL);
    for (int32_t e = 0; e < E; ++e) m[e] = 0.0;
    for (int32_t j = 0; j < k; ++j) m[ids[j]] = w[j];
    double* yt = y + t * H;
    for (int64_t c = 0; c < H; ++c) yt[c] = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      or_expert(S, routed, e, x, d);
      for (int64_t c = 0; c < H; ++c) yt[c] += m[e] * d[c];
    }
    for (int32_t s = 0; shared && s < S->n_shared; ++s) {
      or_expert(S, shared, s, x, d);
      for (int64_t c = 0; c < H; ++c) yt[c] += d[c];
    }
  }
  free(x);
  free(d);
  free(m);
  free(ids);
  free(w);
}

/* ------------------------------------------------------------------ dense GEMV */

/* Small-batch dense GEMV on packed NVFP4 weights, the kernel the pages list
 * for the non-expert projections ("Day-0 Support for Flint on vLLM",
 * Optimization section, Fig. 2 change list): y[t][n] = sum_k W[n][k] x[t][k]
 * with W at its exact fp64 value e2m1 * e4m3 * global, k ascending.
 * x bf16 [B][K]; codes u8 [N][K/2]; scales u8 [N][K/16]; y fp64 [B][N]. */
void or_gemv_nvfp4(const uint16_t* x, int32_t B, int32_t K, int32_t N, const uint8_t* codes,
                   const uint8_t* scales, float global, double* y) {
  or_tables();
  #pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t t = 0; t < B; ++t) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        uint8_t byte = codes[n * (K / 2) + k / 2];
        uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
        double w = g_e2m1[nib] * g_e4m3[scales[n * (K / 16) + k / 16]] * (double)global;
        acc += w * or_bf16(x[t * K + k]);
      }
      y[t * N + n] = acc;
    }
}

/* ------------------------------------------------------------------ RMSNorm */

/* Round an fp64 value once to bf16 (round to nearest, ties to even), from the
 * format's definition: bf16 keeps 8 significant bits (7 stored) with fp32's
 * exponent range, so the value is snapped to the grid 2^(e - 7) of its
 * binade (2^-133 below the smallest normal 2^-126) with rint() in the default
 * ties-to-even mode; the snapped value has at most 9 significant bits, so it
 * converts to fp32 exactly and bf16 is its upper half.  Overflow gives inf. */
uint16_t or_bf16_rne(double v) {
  if (v != v) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int e = 0;
  (void)frexp(a, &e);                              /* a = m 2^e, m in [0.5, 1) */
  const int lead = e - 1;                          /* exponent of the leading bit */
  const int qexp = lead >= -126 ? lead - 7 : -133; /* grid spacing 2^qexp */
  const double r = ldexp(rint(ldexp(a, -qexp)), qexp);
  const float f = (float)r;                        /* exact, or inf on overflow */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

void or_bf16_rne_array(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_rne(v[i]);
}

/* The pre-MoE RMSNorm that the pages' low-latency path fuses into the
 * adjacent GEMVs ("Day-0 Support for Flint on vLLM", Optimization section,
 * low-latency MoE path and Fig. 3; the norm kernels are one of the Fig. 2
 * steps): xn[k] = x[k] * w[k] / sqrt(mean_j x[j]^2 + eps), in fp64 with the
 * sum over j in index order, then rounded once to bf16, since the router and
 * the experts take bf16 activations (Model architecture section, W4A16).
 * x bf16 [T][H]; w bf16 [H]; xn bf16 [T][H]. */
void or_rmsnorm_bf16(const uint16_t* x, int32_t T, int32_t H, const uint16_t* w, double eps,
                     uint16_t* xn) {
  #pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t k = 0; k < H; ++k) {
      const double v = or_bf16(x[t * H + k]);
      ss += v * v;
    }
    const double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t k = 0; k < H; ++k)
      xn[t * H + k] = or_bf16_rne(or_bf16(x[t * H + k]) * or_bf16(w[k]) * r);
  }
}

/* ------------------------------------------------------------------ W4A4 */

/* NVFP4 activations with the Four Over Six block scale (the AREX article on
 * vLLM's Day-0 support for Inkling-2-Small, 48-layer MoE section: a
 * per-token global scale, and for each 16-element block the scale that maps
 * the block maximum to 6 or the one that maps it to 4, whichever leaves the
 * smaller reconstruction error, MAE).  Readings (the article gives no
 * formula): the global is amax / (6 * 448) like the weights'; a candidate's
 * scale is fp32(fp32(bmax / M) / g) rounded to E4M3 (nearest-even,
 * saturating at 448); codes are v / fp32(e4m3 * g) rounded to E2M1; the MAE
 * is summed in fp32 in element order over |v - fp32(e2m1 * q)|; a tie keeps
 * the max->6 candidate.  Every step is an fp32 operation in the order
 * written, so that another implementation can take the same decisions. */

/* nearest-even onto the E4M3FN grid of a finite s >= 0, saturating at 448 */
static uint8_t or_e4m3_rne(float s) {
  if (!(s > 0.0f)) return 0;
  if (s >= 448.0f) return 0x7E;
  if (s < 0.015625f) {                          /* subnormal: multiples of 2^-9 */
    const float m = rintf(ldexpf(s, 9));
    return m >= 8.0f ? 0x08 : (uint8_t)m;
  }
  int k;
  (void)frexpf(s, &k);                          /* s in [2^(k-1), 2^k) */
  int e = k - 1;
  float m = rintf((ldexpf(s, -e) - 1.0f) * 8.0f);
  if (m >= 8.0f) { m = 0.0f; e += 1; }
  if (e > 8 || (e == 8 && m > 6.0f)) return 0x7E;
  return (uint8_t)(((e + 7) << 3) | (int)m);
}

/* nearest-even onto the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating:
 * the 4-bit code (bit 3 = sign).  Midpoints go to the neighbour with the even
 * mantissa bit: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
 * 3.5 -> 4, 5 -> 4. */
static uint8_t or_e2m1_rne(float v) {
  static const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float a = fabsf(v);
  int best = 0;
  for (int i = 1; i < 8; ++i) {
    const float dn = a - grid[best], di = fabsf(a - grid[i]);
    if (di < fabsf(dn) || (di == fabsf(dn) && (i & 1) == 0)) best = i;
  }
  return (uint8_t)((signbit(v) ? 8 : 0) | best);
}

/* One 16-block with scale candidate M: the E4M3 byte, the codes and the MAE. */
static float or_fp4_candidate(const float* v, float bmax, float g, float M, uint8_t* sbyte,
                              uint8_t* codes) {
  *sbyte = or_e4m3_rne((bmax / M) / g);
  const float q = (float)or_e4m3(*sbyte) * g;
  float mae = 0.0f;
  for (int i = 0; i < 16; ++i) {
    codes[i] = q > 0.0f ? or_e2m1_rne(v[i] / q) : 0;
    const float d = (float)or_e2m1(codes[i]) * q;
    mae += fabsf(v[i] - d);
  }
  return mae;
}

/* Quantise v[n] (n a multiple of 16, one token's vector): codes u8 [n] (one
 * 4-bit code per byte), scales u8 [n / 16], *g_out the global, out[n] the
 * exact fp64 values e2m1 * e4m3 * g. */
void or_quant_fp4_46(const float* v, int64_t n, uint8_t* codes, uint8_t* scales, float* g_out,
                     double* out) {
  or_tables();
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float g = amax / 2688.0f;
  *g_out = g;
  for (int64_t b = 0; b < n / 16; ++b) {
    const float* vb = v + 16 * b;
    uint8_t* cb = codes + 16 * b;
    float bmax = 0.0f;
    for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(vb[i]));
    if (g == 0.0f || bmax == 0.0f) {
      scales[b] = 0;
      memset(cb, 0, 16);
    } else {
      uint8_t s6, s4, c6[16], c4[16];
      const float m6 = or_fp4_candidate(vb, bmax, g, 6.0f, &s6, c6);
      const float m4 = or_fp4_candidate(vb, bmax, g, 4.0f, &s4, c4);
      const int four = m4 < m6;
      scales[b] = four ? s4 : s6;
      memcpy(cb, four ? c4 : c6, 16);
    }
    for (int i = 0; i < 16; ++i)
      out[16 * b + i] = g_e2m1[cb[i]] * g_e4m3[scales[b]] * (double)g;
  }
}

/* h = SiLU(G_e x) * (U_e x) of one expert for an fp64 input (I values). */
static void or_expert_h(const or_shape* S, const or_experts* X, int32_t e, const double* x,
                        double* h) {
  int64_t H = S->hidden, I = S->inter;
  double* row = (double*)malloc(sizeof(double) * (size_t)H);
  for (int64_t i = 0; i < I; ++i) {
    double gg = 0.0, u = 0.0;
    or_row(X, e, 0, i, H, I, row);
    for (int64_t k = 0; k < H; ++k) gg += row[k] * x[k];
    or_row(X, e, 1, i, H, I, row);
    for (int64_t k = 0; k < H; ++k) u += row[k] * x[k];
    h[i] = gg * or_sigmoid(gg) * u;
  }
  free(row);
}

/* d = D_e h (H values). */
static void or_expert_down(const or_shape* S, const or_experts* X, int32_t e, const double* h,
                           double* d) {
  int64_t H = S->hidden, I = S->inter;
  double* row = (double*)malloc(sizeof(double) * (size_t)I);
  for (int64_t j = 0; j < H; ++j) {
    double acc = 0.0;
    or_row(X, e, 2, j, H, I, row);
    for (int64_t i = 0; i < I; ++i) acc += row[i] * h[i];
    d[j] = acc;
  }
  free(row);
}

/* The W4A4 layer for B tokens: routing on x itself (the router stays in high
 * precision); each expert's input is the Four-Over-Six quantisation of x,
 * its h = SiLU(g) * u is rounded to bf16 (the activation type between the
 * GEMVs) and quantised the same way before the down GEMV; combine as
 * or_forward.  h slots [B][k + n_shared][I] bf16, in the order routed ids
 * ascending then shared: h_out (nullable) receives this oracle's, and h_in
 * (nullable) replaces them, so that the second quantisation can be taken on
 * another implementation's h. */
void or_forward_w4a4(const or_shape* S, const uint16_t* x, int32_t B, const uint16_t* router,
                     const or_experts* routed, const or_experts* shared, const int32_t* forced,
                     const uint16_t* h_in, double* y, int32_t* ids, double* w, double* gap,
                     uint16_t* h_out) {
  or_tables();
  const int64_t H = S->hidden, I = S->inter;
  const int32_t k = S->top_k, ns = S->n_shared, nslot = k + ns;
  #pragma omp parallel for schedule(dynamic, 1) if (B > 1)
  for (int32_t t = 0; t < B; ++t) {
    const uint16_t* xb = x + t * H;
    int32_t* it = ids + (int64_t)t * k;
    double* wt = w + (int64_t)t * k;
    or_route_token(S, xb, router, forced ? forced + (int64_t)t * k : NULL, it, wt, gap + t, NULL);
    float* xf = (float*)malloc(sizeof(float) * (size_t)(H > I ? H : I));
    double* xq = (double*)malloc(sizeof(double) * (size_t)H);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* hq = (double*)malloc(sizeof(double) * (size_t)I);
    double* d = (double*)malloc(sizeof(double) * (size_t)H);
    uint8_t* codes = (uint8_t*)malloc((size_t)(H > I ? H : I));
    uint8_t* sc = (uint8_t*)malloc((size_t)(H > I ? H : I) / 16);
    float gq;
    for (int64_t c = 0; c < H; ++c) xf[c] = (float)or_bf16(xb[c]);
    or_quant_fp4_46(xf, H, codes, sc, &gq, xq);
    int32_t sorted[16];
    memcpy(sorted, it, sizeof(int32_t) * (size_t)k);
    qsort(sorted, (size_t)k, sizeof(int32_t), or_cmp_i32);
    double* yt = y + t * H;
    for (int64_t c = 0; c < H; ++c) yt[c] = 0.0;
    for (int32_t sl = 0; sl < nslot; ++sl) {
      const int is_sh = sl >= k;
      const or_experts* X = is_sh ? shared : routed;
      const int32_t e = is_sh ? sl - k : sorted[sl];
      double wj = 1.0;
      if (!is_sh)
        for (int32_t j = 0; j < k; ++j) if (it[j] == e) wj = wt[j];
      const int64_t off = ((int64_t)t * nslot + sl) * I;
      or_expert_h(S, X, e, xq, h);
      for (int64_t i = 0; i < I; ++i) {
        const uint16_t hb = or_bf16_rne(h[i]);
        if (h_out) h_out[off + i] = hb;
        xf[i] = (float)or_bf16(h_in ? h_in[off + i] : hb);
      }
      or_quant_fp4_46(xf, I, codes, sc, &gq, hq);
      or_expert_down(S, X, e, hq, d);
      for (int64_t c = 0; c < H; ++c) yt[c] += wj * d[c];
    }
    free(xf); free(xq); free(h); free(hq); free(d); free(codes); free(sc);
  }
}

int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void or_set_num_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n);
#else
  (void)n;
#endif
}
