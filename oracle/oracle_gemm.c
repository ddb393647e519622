/*
 * oracle_gemm.c -- the CPU oracle for dense GEMM.  TEST INFRASTRUCTURE ONLY:
 * only tests/, the smoke check and the CPU-baseline leg of the benchmark load
 * this file's library.  It shares no code, header or table with the GPU
 * library and must never be used as a fallback for it.
 *
 * What it computes is the plain definition, with no blocking or reordering:
 *
 *   C[i][j] = alpha * sum_{k=0}^{K-1} op(A)[i][k] * op(B)[k][j] + beta * C[i][j]
 *
 *  - "SGEMM CUDA代码学习" (leetCUDA 15-sgemm), section 问题定义与记号: C = A x B,
 *    all row-major, A[m][k] at m*K+k, one output is one K-long dot product.
 *  - "CUDA GEMM：从基础写法到工程优化", opening definition and section 1 (the
 *    one-thread-per-output kernel): C = alpha*A*B + beta*C with A M x K,
 *    B K x N, C M x N, row-major.
 *  - "如何优化一个 CUDA Matmul Kernel ... 一份 Worklog", Kernel 1 (naive):
 *    the same alpha/beta update.
 *  - TN layout ("HGEMM SMEM Swizzle 代码学习" kernel comment; "Warp
 *    Specialization HGEMM", section 6 on B's (N,K) layout): A row-major M x K,
 *    B stored N x K row-major.  Here that is op(A)=A, op(B)=transpose of the
 *    stored N x K matrix.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - leading dimensions: element (r,c) of a stored row-major matrix sits at
 *    base + r*ld + c;
 *  - op(X) is X or its transpose; a transposed A is stored K x M, a
 *    transposed B is stored N x K;
 *  - beta == 0: C_in is not read (NaN in C_in does not propagate);
 *    alpha == 0 or K == 0: C = beta*C_in and A, B are not read;
 *  - the accumulator is fp64, k ascending, one accumulator per output;
 *  - inputs in fp16/bf16/fp32 are widened exactly to fp64, so the oracle sees
 *    the same quantised values as any implementation.
 *
 * Output is fp64 (row-major M x N, leading dimension N).  Rounding helpers
 * give the correctly rounded (round-to-nearest-even) fp32/fp16/bf16 value of
 * an fp64 number, for bit-exact comparisons on integer-valued data.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 };

/* ---- exact widening of the stored formats (IEEE 754 binary16 / bfloat16) -- */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(f + 1024), e - 25); /* (1 + f/2^10) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an fp32 (1 sign, 8 exponent, 7 fraction). */
double oracle_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* subnormal: f * 2^-126 * 2^-7 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(f + 128), e - 134); /* (1 + f/2^7) * 2^(e-127) */
  return sign ? -v : v;
}

static double widen(int dtype, const void *p, int64_t idx) {
  switch (dtype) {
  case OR_F32: return (double)((const float *)p)[idx];
  case OR_F16: return oracle_f16_to_f64(((const uint16_t *)p)[idx]);
  case OR_BF16: return oracle_bf16_to_f64(((const uint16_t *)p)[idx]);
  default: return ((const double *)p)[idx];
  }
}

/* ---- correctly rounded narrowing (one rounding, ties to even) ------------- */

/* Round x to a binary format with `p` significand bits (implicit bit
 * included), minimum normal exponent `emin` and largest exponent `emax`.
 * Returns the rounded value as fp64 (+-inf on overflow).  Division and
 * multiplication by the power-of-two quantum are exact in fp64 for every
 * value reached here; nearbyint rounds to nearest-even in the default mode. */
static double round_to_format(double x, int p, int emin, int emax) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int E;
  frexp(x, &E);             /* |x| in [2^(E-1), 2^E) */
  int lead = E - 1;         /* exponent of the leading bit */
  if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
  double q = ldexp(1.0, lead - (p - 1));
  double r = nearbyint(x / q) * q;
  double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (fabs(r) > maxfin) return x > 0 ? INFINITY : -INFINITY;
  return r;
}

static uint16_t encode16(double r, int ebits, int fbits) {
  /* r is exactly representable in the target format (or +-inf / NaN). */
  int bias = (1 << (ebits - 1)) - 1;
  uint16_t sign = signbit(r) ? (uint16_t)(1u << 15) : 0;
  uint16_t emask = (uint16_t)((1u << ebits) - 1);
  if (isnan(r)) return (uint16_t)(sign | (emask << fbits) | (1u << (fbits - 1)));
  if (isinf(r)) return (uint16_t)(sign | (emask << fbits));
  double a = fabs(r);
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E);
  int lead = E - 1;
  int emin = 1 - bias;
  if (lead < emin) { /* subnormal: a = f * 2^(emin - fbits) */
    uint32_t f = (uint32_t)ldexp(a, fbits - emin);
    return (uint16_t)(sign | f);
  }
  uint32_t sig = (uint32_t)ldexp(a, fbits - lead); /* in [2^fbits, 2^(fbits+1)) */
  uint32_t f = sig - (1u << fbits);
  return (uint16_t)(sign | ((uint32_t)(lead + bias) << fbits) | f);
}

/* binary16: p = 11, emin = -14, emax = 15. */
uint16_t oracle_f64_to_f16(double x) { return encode16(round_to_format(x, 11, -14, 15), 5, 10); }
/* bfloat16: p = 8, emin = -126, emax = 127. */
uint16_t oracle_f64_to_bf16(double x) { return encode16(round_to_format(x, 8, -126, 127), 8, 7); }
/* binary32: the C conversion is round-to-nearest-even in the default mode. */
float oracle_f64_to_f32(double x) { return (float)x; }

/* Array forms for the Python wrapper. */
void oracle_round_array(const double *x, int64_t n, int out_dtype, void *out) {
  for (int64_t i = 0; i < n; ++i) {
    if (out_dtype == OR_F32) ((float *)out)[i] = oracle_f64_to_f32(x[i]);
    else if (out_dtype == OR_F16) ((uint16_t *)out)[i] = oracle_f64_to_f16(x[i]);
    else if (out_dtype == OR_BF16) ((uint16_t *)out)[i] = oracle_f64_to_bf16(x[i]);
    else ((double *)out)[i] = x[i];
  }
}
void oracle_widen_array(const void *x, int64_t n, int in_dtype, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen(in_dtype, x, i);
}

/* ---- the GEMM definition ------------------------------------------------- */

typedef struct {
  int64_t M, N, K;
  double alpha, beta;
  const double *opA;  /* M x K, row-major, exact copy of op(A) */
  const double *opBt; /* N x K, row-major: opBt[j][k] = op(B)[k][j] */
  const void *Cin;
  int c_dtype;
  int64_t ldc;
  double *out;        /* M x N, leading dimension N */
  int64_t row0, row1;
} job_t;

static void *run_rows(void *arg) {
  job_t *j = (job_t *)arg;
  for (int64_t i = j->row0; i < j->row1; ++i) {
    for (int64_t c = 0; c < j->N; ++c) {
      double s = 0.0;
      if (j->alpha != 0.0) {
        const double *a = j->opA + i * j->K;
        const double *b = j->opBt + c * j->K;
        for (int64_t k = 0; k < j->K; ++k) s += a[k] * b[k];
      }
      double r = (j->alpha != 0.0) ? j->alpha * s : 0.0;
      if (j->beta != 0.0) r += j->beta * widen(j->c_dtype, j->Cin, i * j->ldc + c);
      j->out[i * j->N + c] = r;
    }
  }
  return NULL;
}

/* ta/tb: 0 = op(X) is X, 1 = op(X) is the transpose of the stored matrix.
 * Rows [row0, row1) of the M x N result are computed (the benchmark's CPU
 * leg evaluates a slab; tests use row0 = 0, row1 = M).  `out` receives
 * (row1 - row0) x N values.  Returns 0, or -1 on a bad argument, -2 when
 * memory runs out. */
int oracle_gemm_rows(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha,
                     const void *A, int a_dtype, int64_t lda, const void *B, int b_dtype,
                     int64_t ldb, double beta, const void *Cin, int c_dtype, int64_t ldc,
                     double *out, int64_t row0, int64_t row1, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || row0 < 0 || row1 > M || row0 > row1) return -1;
  int64_t rows = row1 - row0;
  if (rows == 0 || N == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  int need_ab = (alpha != 0.0 && K > 0);
  double *opA = NULL, *opBt = NULL;
  if (need_ab) {
    opA = (double *)malloc(sizeof(double) * (size_t)(rows * K));
    opBt = (double *)malloc(sizeof(double) * (size_t)(N * K));
    if (!opA || !opBt) { free(opA); free(opBt); return -2; }
    /* op(A)[i][k]: A[i][k] if not transposed, else A[k][i]. */
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t k = 0; k < K; ++k)
        opA[i * K + k] = ta ? widen(a_dtype, A, k * lda + (i + row0))
                            : widen(a_dtype, A, (i + row0) * lda + k);
    /* op(B)[k][j]: B[k][j] if not transposed, else B[j][k]. */
    for (int64_t jj = 0; jj < N; ++jj)
      for (int64_t k = 0; k < K; ++k)
        opBt[jj * K + k] = tb ? widen(b_dtype, B, jj * ldb + k) : widen(b_dtype, B, k * ldb + jj);
  }
  double eff_alpha = need_ab ? alpha : 0.0;
  /* The C_in pointer is shifted to row0 so job rows index from 0. */
  const void *cin = Cin;
  int64_t cbytes = (c_dtype == OR_F32) ? 4 : (c_dtype == OR_F64 ? 8 : 2);
  if (beta != 0.0) cin = (const char *)Cin + row0 * ldc * cbytes;
  if (nthreads > rows) nthreads = (int)rows;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
  if (!th || !jobs) { free(th); free(jobs); free(opA); free(opBt); return -2; }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (job_t){rows, N, K, eff_alpha, beta, opA, opBt, cin, c_dtype, ldc, out,
                      rows * t / nthreads, rows * (t + 1) / nthreads};
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_rows, &jobs[t]);
  run_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th); free(jobs); free(opA); free(opBt);
  return 0;
}

int oracle_gemm(int ta, int tb, int64_t M, int64_t N, int64_t K, double alpha, const void *A,
                int a_dtype, int64_t lda, const void *B, int b_dtype, int64_t ldb, double beta,
                const void *Cin, int c_dtype, int64_t ldc, double *out, int nthreads) {
  return oracle_gemm_rows(ta, tb, M, N, K, alpha, A, a_dtype, lda, B, b_dtype, ldb, beta, Cin,
                          c_dtype, ldc, out, 0, M, nthreads);
}

/* One output element, for sampled checks at sizes where the full oracle is
 * too slow.  Same arithmetic as oracle_gemm_rows. */
double oracle_gemm_element(int ta, int tb, int64_t K, double alpha, const void *A, int a_dtype,
                           int64_t lda, const void *B, int b_dtype, int64_t ldb, double beta,
                           const void *Cin, int c_dtype, int64_t ldc, int64_t i, int64_t j) {
  double s = 0.0;
  if (alpha != 0.0)
    for (int64_t k = 0; k < K; ++k) {
      double a = ta ? widen(a_dtype, A, k * lda + i) : widen(a_dtype, A, i * lda + k);
      double b = tb ? widen(b_dtype, B, j * ldb + k) : widen(b_dtype, B, k * ldb + j);
      s += a * b;
    }
  double r = (alpha != 0.0) ? alpha * s : 0.0;
  if (beta != 0.0) r += beta * widen(c_dtype, Cin, i * ldc + j);
  return r;
}
