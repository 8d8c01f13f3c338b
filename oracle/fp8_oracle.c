/*
 * CPU oracle for the FP8 tensorwise-scaled linear layer and the non-gated
 * relu^2 MLP block.  TEST INFRASTRUCTURE ONLY: it is called by the test
 * suite, by the smoke check and by the CPU-baseline leg of the benchmark,
 * never by the library's product path.  It shares no source with the HIP
 * kernels.
 *
 * What it follows:
 *  - "Het trainen van een 3.8B LLM tot 0.384 CORE voor $998" (decomputer.nl),
 *    section "Vroege experimenten", item 4, and section "Doorvoer verhogen",
 *    first bullet: every linear layer runs its three GEMMs (one forward, two
 *    backward) in FP8 with dynamic tensorwise scaling, i.e. one scale per
 *    tensor recomputed from that tensor on every call.
 *  - The same page's appendix configuration (hidden_act relu2, gated_mlp
 *    false, intermediate 4x hidden, dtype bf16): the block is
 *    Y = relu(X W_up^T)^2 W_down^T with bf16 tensors.
 *  - The pages leave the numeric details open.  Readings used here:
 *    OCP E4M3 (fn) for activations/weights, OCP E5M2 for gradients;
 *    scale s = RN32(amax / fmax) (s = 1 when amax == 0) used as the
 *    dequantisation scale; codes q = RNE_fp8(clamp(RN32(x / s), +-fmax));
 *    GEMMs accumulate exact products and write RN_bf16(RN32(sa*sb) * sum).
 *
 * Arithmetic: fp64 unless a step is defined in another precision (the fp32
 * division of the cast, the fp32 scale product, the bf16 outputs).
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math:
 * every rounding here is meant to be IEEE).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_E4M3 0
#define ORC_E5M2 1

/* ---------------------------------------------------------------------- */
/* Format definitions (OCP 8-bit floating point).                          */
/*   E4M3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no infs;   */
/*           exponent 15 with mantissa 7 is NaN; largest finite 448.       */
/*   E5M2:   1 sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent  */
/*           31 is inf (mantissa 0) or NaN; largest finite 57344.          */
/* ---------------------------------------------------------------------- */
static int fmt_ebits(int fmt) { return fmt == ORC_E4M3 ? 4 : 5; }
static int fmt_mbits(int fmt) { return fmt == ORC_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == ORC_E4M3 ? 7 : 15; }

/* Decode one code from the bit fields.  Returns NaN for NaN codes and
 * +-INFINITY for the E5M2 infinities. */
double orc_decode(int fmt, int code) {
  int ebits = fmt_ebits(fmt), mbits = fmt_mbits(fmt), bias = fmt_bias(fmt);
  int sign = (code >> 7) & 1;
  int e = (code >> mbits) & ((1 << ebits) - 1);
  int m = code & ((1 << mbits) - 1);
  int emax_field = (1 << ebits) - 1;
  double v;
  if (fmt == ORC_E4M3 && e == emax_field && m == (1 << mbits) - 1) return NAN;
  if (fmt == ORC_E5M2 && e == emax_field) {
    if (m != 0) return NAN;
    return sign ? -INFINITY : INFINITY;
  }
  if (e == 0) /* subnormal: 0.m x 2^(1-bias) */
    v = ldexp((double)m, 1 - bias - mbits);
  else /* normal: 1.m x 2^(e-bias) */
    v = ldexp((double)((1 << mbits) + m), e - bias - mbits);
  return sign ? -v : v;
}

void orc_decode_table(int fmt, double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = orc_decode(fmt, c);
}

double orc_fmax(int fmt) { return fmt == ORC_E4M3 ? 448.0 : 57344.0; }

/* Largest positive finite code: 0x7E for E4M3, 0x7B for E5M2. */
static int fmt_max_code(int fmt) { return fmt == ORC_E4M3 ? 0x7E : 0x7B; }

/* Round a finite value c with |c| <= fmax to the nearest code; ties go to
 * the code with the even significand (code bit 0 clear, since positive codes
 * are ordered by magnitude and bit 0 is the last mantissa bit).  The sign of
 * c (including -0) is kept.  Search is over the table of positive finite
 * values, which is sorted by code. */
int orc_encode_rne(int fmt, double c) {
  int neg = signbit(c) ? 1 : 0;
  double a = fabs(c);
  int top = fmt_max_code(fmt);
  int lo = 0, hi = top, code;
  /* find largest code with decode(code) <= a (decode(0) = 0 <= a) */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (orc_decode(fmt, mid) <= a) lo = mid; else hi = mid - 1;
  }
  code = lo;
  if (code < top) {
    double below = orc_decode(fmt, code), above = orc_decode(fmt, code + 1);
    double midpoint = 0.5 * (below + above); /* exact in fp64 */
    if (a > midpoint) code = code + 1;
    else if (a == midpoint && (code & 1)) code = code + 1;
  }
  return neg ? (code | 0x80) : code;
}

/* bf16 bits -> value (exact). */
static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double to the nearest bf16 (8 significant bits, exponent range of
 * binary32, gradual underflow with quantum 2^-133), ties to even.  The
 * result is produced in one rounding step from the double. */
uint16_t orc_double_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  int neg = signbit(x) ? 1 : 0;
  double a = fabs(x);
  uint16_t sign = neg ? 0x8000 : 0;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);     /* a = f * 2^e with f in [0.5, 1) -> floor(log2 a) = e-1 */
  int ex = e - 1;
  if (ex < -126) ex = -126;          /* subnormal range shares the quantum 2^-133 */
  double quantum = ldexp(1.0, ex - 7);
  double r = nearbyint(a / quantum) * quantum; /* a/quantum exact (power of 2) */
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow -> inf */
  float f = (float)r; /* exact: r has <= 8 significant bits inside binary32 range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* ---------------------------------------------------------------------- */
/* Quantisation: amax, scale, cast.                                        */
/* ---------------------------------------------------------------------- */

/* amax = max_i |x_i| over a rows x cols bf16 matrix with leading dim ld. */
float orc_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld) {
  float amax = 0.0f;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      float v = fabsf(bf16_to_float(x[r * ld + c]));
      if (v > amax) amax = v;
    }
  return amax;
}

/* s = RN32(amax / fmax); 1 when amax is zero. */
float orc_scale_from_amax(float amax, int fmt) {
  if (amax == 0.0f) return 1.0f;
  volatile float fm = (float)orc_fmax(fmt);
  volatile float q = amax / fm; /* binary32 division, correctly rounded */
  return q;
}

/* q_i = RNE_fp8(clamp(RN32(x_i / s), -fmax, fmax)) for a given scale. */
void orc_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float s,
              int fmt, uint8_t* q, int64_t ldq) {
  float fm = (float)orc_fmax(fmt);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      volatile float v = bf16_to_float(x[r * ld + c]) / s; /* RN32 */
      float cl = v;
      if (cl > fm) cl = fm;
      if (cl < -fm) cl = -fm;
      q[r * ldq + c] = (uint8_t)orc_encode_rne(fmt, (double)cl);
    }
}

/* Same as orc_cast but x is given as binary32 values (used by the pins,
 * which probe rounding boundaries that bf16 cannot express). */
void orc_cast_f32(const float* x, int64_t n, float s, int fmt, uint8_t* q) {
  float fm = (float)orc_fmax(fmt);
  for (int64_t i = 0; i < n; ++i) {
    volatile float v = x[i] / s;
    float cl = v;
    if (cl > fm) cl = fm;
    if (cl < -fm) cl = -fm;
    q[i] = (uint8_t)orc_encode_rne(fmt, (double)cl);
  }
}

/* Full dynamic tensorwise quantisation of one tensor. */
void orc_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int fmt,
               uint8_t* q, int64_t ldq, float* scale, float* amax_out) {
  float amax = orc_amax(x, rows, cols, ld);
  float s = orc_scale_from_amax(amax, fmt);
  orc_cast(x, rows, cols, ld, s, fmt, q, ldq);
  *scale = s;
  if (amax_out) *amax_out = amax;
}

/* ---------------------------------------------------------------------- */
/* GEMMs on fp8 codes.  All matrices row-major with explicit leading dims.  */
/*   out = RN_bf16( RN32(sa*sb) * sum dec(a)*dec(b) ), sum in fp64.         */
/* row_idx (may be NULL) restricts the computation to the listed output     */
/* rows; out then holds those rows densely, one after another.              */
/* ---------------------------------------------------------------------- */
static float scale_product(float sa, float sb) {
  volatile float p = sa * sb; /* RN32 */
  return p;
}

static void decode_matrix(const uint8_t* a, int64_t rows, int64_t cols, int64_t ld, int fmt,
                          double* out) {
  double tab[256];
  orc_decode_table(fmt, tab);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = tab[a[r * ld + c]];
}

/* NT: y[m,n] = sum_k a[m,k] b[n,k];  a [M,K], b [N,K]  (forward) */
void orc_gemm_nt(const uint8_t* a, int64_t lda, int fa, float sa,
                 const uint8_t* b, int64_t ldb, int fb, float sb,
                 int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                 const int64_t* row_idx, int64_t n_rows) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K));
  double ta[256];
  orc_decode_table(fa, ta);
  decode_matrix(b, N, K, ldb, fb, bd);
  double p = (double)scale_product(sa, sb);
  int64_t R = row_idx ? n_rows : M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < R; ++i) {
    int64_t m = row_idx ? row_idx[i] : i;
    double* arow = (double*)malloc(sizeof(double) * (size_t)K);
    for (int64_t k = 0; k < K; ++k) arow[k] = ta[a[m * lda + k]];
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      const double* brow = bd + n * K;
      for (int64_t k = 0; k < K; ++k) acc += arow[k] * brow[k];
      y[i * ldy + n] = orc_double_to_bf16(acc * p);
    }
    free(arow);
  }
  free(bd);
  (void)M;
}

/* NN: y[m,k] = sum_n a[m,n] b[n,k];  a [M,N], b [N,K]  (grad-input) */
void orc_gemm_nn(const uint8_t* a, int64_t lda, int fa, float sa,
                 const uint8_t* b, int64_t ldb, int fb, float sb,
                 int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                 const int64_t* row_idx, int64_t n_rows) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K));
  double ta[256];
  orc_decode_table(fa, ta);
  decode_matrix(b, N, K, ldb, fb, bd);
  double p = (double)scale_product(sa, sb);
  int64_t R = row_idx ? n_rows : M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < R; ++i) {
    int64_t m = row_idx ? row_idx[i] : i;
    double* acc = (double*)calloc((size_t)K, sizeof(double));
    for (int64_t n = 0; n < N; ++n) {
      double av = ta[a[m * lda + n]];
      const double* brow = bd + n * K;
      for (int64_t k = 0; k < K; ++k) acc[k] += av * brow[k];
    }
    for (int64_t k = 0; k < K; ++k) y[i * ldy + k] = orc_double_to_bf16(acc[k] * p);
    free(acc);
  }
  free(bd);
  (void)M;
}

/* TN: y[n,k] = sum_m a[m,n] b[m,k];  a [M,N], b [M,K]  (grad-weight) */
void orc_gemm_tn(const uint8_t* a, int64_t lda, int fa, float sa,
                 const uint8_t* b, int64_t ldb, int fb, float sb,
                 int64_t M, int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                 const int64_t* row_idx, int64_t n_rows) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  double ta[256];
  orc_decode_table(fa, ta);
  decode_matrix(b, M, K, ldb, fb, bd);
  double p = (double)scale_product(sa, sb);
  int64_t R = row_idx ? n_rows : N;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < R; ++i) {
    int64_t n = row_idx ? row_idx[i] : i;
    double* acc = (double*)calloc((size_t)K, sizeof(double));
    for (int64_t m = 0; m < M; ++m) {
      double av = ta[a[m * lda + n]];
      const double* brow = bd + m * K;
      for (int64_t k = 0; k < K; ++k) acc[k] += av * brow[k];
    }
    for (int64_t k = 0; k < K; ++k) y[i * ldy + k] = orc_double_to_bf16(acc[k] * p);
    free(acc);
  }
  free(bd);
}

/* TN product added to an fp64 accumulator, without any rounding:          */
/*   acc[n,k] += RN32(sa*sb) * sum_m dec(a[m,n]) dec(b[m,k])               */
/* for a gradient summed over several chunks of rows before its single     */
/* rounding to bf16 (the chunked LM-head cross-entropy's weight gradient). */
void orc_gemm_tn_acc(const uint8_t* a, int64_t lda, int fa, float sa,
                     const uint8_t* b, int64_t ldb, int fb, float sb,
                     int64_t M, int64_t N, int64_t K, double* acc, int64_t ldacc) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
  double ta[256];
  orc_decode_table(fa, ta);
  decode_matrix(b, M, K, ldb, fb, bd);
  double p = (double)scale_product(sa, sb);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < N; ++n) {
    double* s = (double*)calloc((size_t)K + 1, sizeof(double));
    for (int64_t m = 0; m < M; ++m) {
      double av = ta[a[m * lda + n]];
      const double* brow = bd + m * K;
      for (int64_t k = 0; k < K; ++k) s[k] += av * brow[k];
    }
    for (int64_t k = 0; k < K; ++k) acc[n * ldacc + k] += s[k] * p;
    free(s);
  }
  free(bd);
}

/* NN product added to an fp64 accumulator, without rounding:              */
/*   acc[i,k] += RN32(sa*sb) * sum_n dec(a[m,n]) dec(b[n,k]),  m = rows[i]  */
/* for a grad-input that is the sum of two products (the gated MLP's dX    */
/* through the gate and the up projection) rounded once to bf16.  row_idx  */
/* may be NULL (all M rows).                                               */
void orc_gemm_nn_acc(const uint8_t* a, int64_t lda, int fa, float sa,
                     const uint8_t* b, int64_t ldb, int fb, float sb,
                     int64_t M, int64_t N, int64_t K, double* acc, int64_t ldacc,
                     const int64_t* row_idx, int64_t n_rows) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
  double ta[256];
  orc_decode_table(fa, ta);
  decode_matrix(b, N, K, ldb, fb, bd);
  double p = (double)scale_product(sa, sb);
  int64_t R = row_idx ? n_rows : M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < R; ++i) {
    int64_t m = row_idx ? row_idx[i] : i;
    double* s = (double*)calloc((size_t)K + 1, sizeof(double));
    for (int64_t n = 0; n < N; ++n) {
      double av = ta[a[m * lda + n]];
      const double* brow = bd + n * K;
      for (int64_t k = 0; k < K; ++k) s[k] += av * brow[k];
    }
    for (int64_t k = 0; k < K; ++k) acc[i * ldacc + k] += s[k] * p;
    free(s);
  }
  free(bd);
}

/* ---------------------------------------------------------------------- */
/* RMSNorm of bf16 rows (decomputer.nl, appendix: Llama-style RMSNorm,     */
/* rms_norm_eps 1.0e-6), the step before the MLP's input quantisation:     */
/*   ms = RN32(sum_j x_j^2 / d)       (sum in fp64)                         */
/*   r  = RN32(1 / RN32(sqrt(RN32(ms + eps))))                              */
/*   X_j = RN_bf16(RN32(RN32(x_j r) g_j))   (g NULL: RN_bf16(RN32(x_j r)))   */
/* out [rows, cols] bf16 bits (dense), rstd [rows] = r.                    */
/* ---------------------------------------------------------------------- */
static uint16_t f32_to_bf16_bits(float f) { return orc_double_to_bf16((double)f); }

void orc_rmsnorm(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const uint16_t* g,
                 float eps, uint16_t* out, float* rstd) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < rows; ++i) {
    double ss = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      const double v = (double)bf16_to_float(x[i * ld + j]);
      ss += v * v;
    }
    volatile float ms = (float)(ss / (double)cols);
    volatile float t = ms + eps;
    volatile float sq = sqrtf(t);
    volatile float r = 1.0f / sq;
    rstd[i] = r;
    for (int64_t j = 0; j < cols; ++j) {
      volatile float y = bf16_to_float(x[i * ld + j]) * r;
      if (g) y = y * bf16_to_float(g[j]);
      out[i * cols + j] = f32_to_bf16_bits(y);
    }
  }
}

/* ---------------------------------------------------------------------- */
/* relu^2 and its derivative on bf16 tensors.                              */
/*   A  = RN_bf16( relu(H)^2 )             (exact square before rounding)  */
/*   dH = RN_bf16( 2 * relu(H) * dA )      (exact product before rounding) */
/* ---------------------------------------------------------------------- */
void orc_relu2(const uint16_t* h, int64_t n, uint16_t* a) {
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)bf16_to_float(h[i]);
    double r = v > 0.0 ? v : 0.0;
    a[i] = orc_double_to_bf16(r * r);
  }
}

void orc_relu2_bwd(const uint16_t* h, const uint16_t* da, int64_t n, uint16_t* dh) {
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)bf16_to_float(h[i]);
    double r = v > 0.0 ? v : 0.0;
    dh[i] = orc_double_to_bf16(2.0 * r * (double)bf16_to_float(da[i]));
  }
}

void orc_double_to_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_bf16(x[i]);
}
