/*
 * Calls every function of oracle/fp8_oracle.c on small ragged and strided
 * inputs held in heap buffers of exactly the size each call may touch, so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer reports
 * any access outside them or any undefined operation.  Built and run by
 * tests/test_oracle_sanitizers.py; exits 0 when every call returned.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_decode(int fmt, int code);
void orc_decode_table(int fmt, double* out256);
double orc_fmax(int fmt);
int orc_encode_rne(int fmt, double c);
uint16_t orc_double_to_bf16(double x);
void orc_double_to_bf16_array(const double* x, int64_t n, uint16_t* out);
float orc_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld);
float orc_scale_from_amax(float amax, int fmt);
void orc_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float s, int fmt, uint8_t* q,
              int64_t ldq);
void orc_cast_f32(const float* x, int64_t n, float s, int fmt, uint8_t* q);
void orc_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int fmt, uint8_t* q, int64_t ldq,
               float* scale, float* amax_out);
void orc_gemm_nt(const uint8_t* a, int64_t lda, int fa, float sa, const uint8_t* b, int64_t ldb, int fb,
                 float sb, int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy, const int64_t* row_idx,
                 int64_t n_rows);
void orc_gemm_nn(const uint8_t* a, int64_t lda, int fa, float sa, const uint8_t* b, int64_t ldb, int fb,
                 float sb, int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy, const int64_t* row_idx,
                 int64_t n_rows);
void orc_gemm_tn(const uint8_t* a, int64_t lda, int fa, float sa, const uint8_t* b, int64_t ldb, int fb,
                 float sb, int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy, const int64_t* row_idx,
                 int64_t n_rows);
void orc_gemm_tn_acc(const uint8_t* a, int64_t lda, int fa, float sa, const uint8_t* b, int64_t ldb, int fb,
                     float sb, int64_t M, int64_t N, int64_t K, double* acc, int64_t ldacc);
void orc_gemm_nn_acc(const uint8_t* a, int64_t lda, int fa, float sa, const uint8_t* b, int64_t ldb, int fb,
                     float sb, int64_t M, int64_t N, int64_t K, double* acc, int64_t ldacc,
                     const int64_t* row_idx, int64_t n_rows);
void orc_rmsnorm(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const uint16_t* g, float eps,
                 uint16_t* out, float* rstd);
void orc_relu2(const uint16_t* h, int64_t n, uint16_t* a);
void orc_relu2_bwd(const uint16_t* h, const uint16_t* da, int64_t n, uint16_t* dh);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* a [rows, cols] matrix with leading dimension ld, allocated to its last
   element exactly; finite bf16 values (exponent field below 0xFF) */
static uint16_t* bf16_matrix(int64_t rows, int64_t cols, int64_t ld) {
  const int64_t n = rows > 0 && cols > 0 ? (rows - 1) * ld + cols : 0;
  uint16_t* p = (uint16_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) {
    uint16_t v = (uint16_t)(next_u32() & 0xFFFFu);
    if (((v >> 7) & 0xFF) >= 0x86) v = (uint16_t)((v & 0x807Fu) | (0x70u << 7)); /* |v| < 2^7: keep it tame */
    p[i] = v;
  }
  return p;
}

/* FP8 codes without NaN encodings */
static uint8_t* code_matrix(int64_t rows, int64_t cols, int64_t ld, int fmt) {
  const int64_t n = rows > 0 && cols > 0 ? (rows - 1) * ld + cols : 0;
  uint8_t* p = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) {
    uint8_t c = (uint8_t)(next_u32() & 0xFFu);
    if (fmt == 0 && (c & 0x7F) == 0x7F) c ^= 1; /* E4M3 NaN */
    if (fmt == 1 && (c & 0x7C) == 0x7C) c &= 0xF3; /* E5M2 inf/NaN */
    p[i] = c;
  }
  return p;
}

static void quant_cases(void) {
  const int64_t shapes[][3] = {{5, 7, 9}, {1, 1, 1}, {3, 16, 16}, {0, 4, 4}, {4, 0, 1}};
  for (int fmt = 0; fmt < 2; ++fmt)
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
      const int64_t r = shapes[s][0], c = shapes[s][1], ld = shapes[s][2], ldq = c + 3;
      uint16_t* x = bf16_matrix(r, c, ld);
      const int64_t nq = r > 0 && c > 0 ? (r - 1) * ldq + c : 1;
      uint8_t* q = (uint8_t*)malloc((size_t)nq);
      float sc = 0.f, am = 0.f;
      orc_quant(x, r, c, ld, fmt, q, ldq, &sc, &am);
      orc_quant(x, r, c, ld, fmt, q, ldq, &sc, NULL);
      const float a2 = orc_amax(x, r, c, ld);
      orc_cast(x, r, c, ld, orc_scale_from_amax(a2, fmt), fmt, q, ldq);
      if (a2 != am) { fprintf(stderr, "amax mismatch\n"); exit(2); }
      free(x);
      free(q);
    }
  float* xf = (float*)malloc(11 * sizeof(float));
  uint8_t* qf = (uint8_t*)malloc(11);
  for (int i = 0; i < 11; ++i) xf[i] = (float)(i - 5) * 0.37f;
  orc_cast_f32(xf, 11, 0.01f, 0, qf);
  orc_cast_f32(xf, 11, 0.01f, 1, qf);
  free(xf);
  free(qf);
}

static void gemm_cases(void) {
  const int64_t M = 7, N = 5, K = 9, pad = 3;
  for (int fa = 0; fa < 2; ++fa)
    for (int fb = 0; fb < 2; ++fb) {
      /* NT: a [M,K], b [N,K], y [M,N] */
      uint8_t* a = code_matrix(M, K, K + pad, fa);
      uint8_t* b = code_matrix(N, K, K + pad, fb);
      uint16_t* y = (uint16_t*)malloc((size_t)((M - 1) * (N + pad) + N) * sizeof(uint16_t));
      orc_gemm_nt(a, K + pad, fa, 0.5f, b, K + pad, fb, 2.0f, M, N, K, y, N + pad, NULL, 0);
      const int64_t rows[3] = {M - 1, 0, 3};
      uint16_t* ys = (uint16_t*)malloc((size_t)(3 * N) * sizeof(uint16_t));
      orc_gemm_nt(a, K + pad, fa, 0.5f, b, K + pad, fb, 2.0f, M, N, K, ys, N, rows, 3);
      free(a); free(b); free(y); free(ys);
      /* NN: a [M,N], b [N,K], y [M,K] */
      a = code_matrix(M, N, N + pad, fa);
      b = code_matrix(N, K, K, fb);
      y = (uint16_t*)malloc((size_t)(M * K) * sizeof(uint16_t));
      orc_gemm_nn(a, N + pad, fa, 0.25f, b, K, fb, 3.0f, M, N, K, y, K, NULL, 0);
      ys = (uint16_t*)malloc((size_t)(3 * K) * sizeof(uint16_t));
      orc_gemm_nn(a, N + pad, fa, 0.25f, b, K, fb, 3.0f, M, N, K, ys, K, rows, 3);
      double* acc = (double*)calloc((size_t)(3 * K), sizeof(double));
      orc_gemm_nn_acc(a, N + pad, fa, 0.25f, b, K, fb, 3.0f, M, N, K, acc, K, rows, 3);
      double* accf = (double*)calloc((size_t)(M * K), sizeof(double));
      orc_gemm_nn_acc(a, N + pad, fa, 0.25f, b, K, fb, 3.0f, M, N, K, accf, K, NULL, 0);
      free(a); free(b); free(y); free(ys); free(acc); free(accf);
      /* TN: a [M,N], b [M,K], y [N,K] */
      a = code_matrix(M, N, N, fa);
      b = code_matrix(M, K, K + pad, fb);
      y = (uint16_t*)malloc((size_t)((N - 1) * (K + pad) + K) * sizeof(uint16_t));
      orc_gemm_tn(a, N, fa, 1.5f, b, K + pad, fb, 0.75f, M, N, K, y, K + pad, NULL, 0);
      const int64_t nrows[2] = {N - 1, 1};
      ys = (uint16_t*)malloc((size_t)(2 * K) * sizeof(uint16_t));
      orc_gemm_tn(a, N, fa, 1.5f, b, K + pad, fb, 0.75f, M, N, K, ys, K, nrows, 2);
      acc = (double*)calloc((size_t)(N * K), sizeof(double));
      orc_gemm_tn_acc(a, N, fa, 1.5f, b, K + pad, fb, 0.75f, M, N, K, acc, K);
      free(a); free(b); free(y); free(ys); free(acc);
    }
  /* empty reductions and outputs */
  uint8_t* a = code_matrix(1, 1, 1, 0);
  uint8_t* b2 = code_matrix(2, 1, 1, 0); /* [N=2, K=1] */
  uint16_t* y = (uint16_t*)malloc(4 * sizeof(uint16_t));
  orc_gemm_nt(a, 1, 0, 1.f, a, 1, 0, 1.f, 2, 2, 0, y, 2, NULL, 0);   /* K = 0 */
  orc_gemm_nt(a, 1, 0, 1.f, b2, 1, 0, 1.f, 0, 2, 1, y, 2, NULL, 0);  /* M = 0 */
  orc_gemm_tn(a, 1, 0, 1.f, a, 1, 0, 1.f, 0, 2, 2, y, 2, NULL, 0);   /* M = 0 reduction */
  free(a);
  free(b2);
  free(y);
}

static void elementwise_cases(void) {
  double tab[256];
  for (int fmt = 0; fmt < 2; ++fmt) {
    orc_decode_table(fmt, tab);
    for (int c = 0; c < 256; ++c) {
      const double v = orc_decode(fmt, c);
      if (!isnan(v) && !isinf(v)) (void)orc_encode_rne(fmt, v);
    }
    const double fm = orc_fmax(fmt);
    const double probes[] = {0.0, -0.0, fm, -fm, fm * 0.999, 1e-12, -1e-12, 3.0e-5, 0.5};
    for (size_t i = 0; i < sizeof probes / sizeof probes[0]; ++i) (void)orc_encode_rne(fmt, probes[i]);
  }
  const double vals[] = {0.0, -0.0, 1.0, -1.5, 1e-40, 3.0e38, -3.3e38, 1e300, 65504.0, 1.00390625};
  uint16_t out[sizeof vals / sizeof vals[0]];
  for (size_t i = 0; i < sizeof vals / sizeof vals[0]; ++i) (void)orc_double_to_bf16(vals[i]);
  orc_double_to_bf16_array(vals, (int64_t)(sizeof vals / sizeof vals[0]), out);

  const int64_t n = 37;
  uint16_t* h = bf16_matrix(1, n, n);
  uint16_t* da = bf16_matrix(1, n, n);
  uint16_t* o = (uint16_t*)malloc((size_t)n * sizeof(uint16_t));
  orc_relu2(h, n, o);
  orc_relu2_bwd(h, da, n, o);
  free(h); free(da); free(o);

  const int64_t r = 6, c = 13, ld = 17;
  uint16_t* x = bf16_matrix(r, c, ld);
  uint16_t* g = bf16_matrix(1, c, c);
  uint16_t* xo = (uint16_t*)malloc((size_t)(r * c) * sizeof(uint16_t));
  float* rs = (float*)malloc((size_t)r * sizeof(float));
  orc_rmsnorm(x, r, c, ld, g, 1e-6f, xo, rs);
  orc_rmsnorm(x, r, c, ld, NULL, 0.0f, xo, rs);
  free(x); free(g); free(xo); free(rs);
}

int main(void) {
  quant_cases();
  gemm_cases();
  elementwise_cases();
  puts("oracle sanitizer run: ok");
  return 0;
}
