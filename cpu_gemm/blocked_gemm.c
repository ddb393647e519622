/*
 * Cache-blocked CPU GEMM with fp32 accumulation: a reported CPU baseline for
 * the GPU library, next to the fp64 oracle (which it does not share code
 * with).  C = alpha * op(A) * op(B) + beta * C on rows [row0, row1) of C,
 * the same operation as the GPU path ("SGEMM CUDA代码学习", section
 * 问题定义与记号, with the alpha/beta update of "CUDA GEMM：从基础写法到工程优化").
 *
 * The blocking follows the hierarchy those pages build on the GPU, restated
 * for CPU caches: op(B) is widened once to an fp32 K x N copy; each thread
 * owns a range of NC-wide column stripes and, per KC-deep block of k, packs
 * the rows' MR-row panels of op(A) k-major; an MR x NR register tile (6 x 32
 * floats, which the compiler maps onto vector FMAs under -march=native) runs
 * each panel against the L2-resident KC x NC block of the packed op(B).  fp16 / bf16 inputs are
 * widened exactly to fp32; the output is fp32.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { BT_F32 = 0, BT_F16 = 1, BT_BF16 = 2 };
enum { MR = 6, NR = 32, KC = 256, NC = 512 };

static float widen(const void *base, int type, int64_t idx) {
  if (type == BT_F32) return ((const float *)base)[idx];
  const uint16_t h = ((const uint16_t *)base)[idx];
  if (type == BT_BF16) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  const uint32_t s = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 31, m = h & 1023;
  if (e == 0) {
    const float f = ldexpf((float)m, -24);  /* zero or subnormal: m * 2^-24 */
    return s ? -f : f;
  }
  const uint32_t u = e == 31 ? (s | 0x7f800000u | (m << 13)) : (s | ((e + 112) << 23) | (m << 13));
  float f;
  memcpy(&f, &u, 4);
  return f;
}

typedef struct {
  int ta, M, N, K;
  float alpha, beta;
  const void *A;
  int a_type;
  int64_t lda;
  const float *Bp;  /* op(B) as fp32, K x N row-major */
  const float *Cin;
  int64_t ldcin;
  float *C;
  int64_t ldc;
  int r0, r1, c0, c1;
} Job;

/* op(A)[m][k] */
static float a_at(const Job *j, int m, int k) {
  return j->ta ? widen(j->A, j->a_type, (int64_t)k * j->lda + m) : widen(j->A, j->a_type, (int64_t)m * j->lda + k);
}

/* out (MR x NR) = Ap (kc x MR, k-major) * Bs (kc rows of NR, pitch N) */
static void tile_full(int kc, const float *restrict ap, const float *restrict bs, int64_t pitch,
                      float *restrict out) {
  float acc[MR][NR] = {{0}};
  for (int k = 0; k < kc; ++k) {
    const float *restrict b = bs + (int64_t)k * pitch;
    const float *restrict a = ap + k * MR;
#pragma GCC unroll 6
    for (int r = 0; r < MR; ++r) {
      const float av = a[r];
#pragma GCC unroll 32
      for (int c = 0; c < NR; ++c) acc[r][c] += av * b[c];
    }
  }
  memcpy(out, acc, sizeof acc);
}

/* One thread: every row of [r0, r1) for the columns [c0, c1) (whole NC
 * stripes).  The fp32 sums accumulate in C itself, then the epilogue
 * applies alpha and beta. */
static void *worker(void *arg) {
  const Job *j = (const Job *)arg;
  const int rows = j->r1 - j->r0;
  if (rows <= 0 || j->c0 >= j->c1) return NULL;
  const int panels = (rows + MR - 1) / MR;
  float *ap = (float *)malloc(sizeof(float) * (size_t)panels * MR * KC);
  if (!ap) return (void *)1;
  for (int r = 0; r < rows; ++r)
    memset(j->C + (int64_t)(j->r0 + r) * j->ldc + j->c0, 0, sizeof(float) * (j->c1 - j->c0));
  for (int k0 = 0; k0 < j->K; k0 += KC) {
    const int kc = j->K - k0 < KC ? j->K - k0 : KC;
    for (int p = 0; p < panels; ++p)  /* pack op(A) rows, k-major per panel, zero rows past r1 */
      for (int k = 0; k < kc; ++k)
        for (int r = 0; r < MR; ++r) {
          const int m = j->r0 + p * MR + r;
          ap[((size_t)p * KC + k) * MR + r] = m < j->r1 ? a_at(j, m, k0 + k) : 0.0f;
        }
    for (int n0 = j->c0; n0 < j->c1; n0 += NC) {
      const int nc = j->c1 - n0 < NC ? j->c1 - n0 : NC;
      for (int p = 0; p < panels; ++p) {
        const int mr = rows - p * MR < MR ? rows - p * MR : MR;
        for (int c0 = 0; c0 < nc; c0 += NR) {
          const int nr = nc - c0 < NR ? nc - c0 : NR;
          const float *bs = j->Bp + (int64_t)k0 * j->N + n0 + c0;
          float acc[MR][NR];
          if (nr == NR) {
            tile_full(kc, ap + (size_t)p * KC * MR, bs, j->N, &acc[0][0]);
          } else {
            memset(acc, 0, sizeof acc);
            for (int k = 0; k < kc; ++k)
              for (int r = 0; r < MR; ++r)
                for (int c = 0; c < nr; ++c)
                  acc[r][c] += ap[((size_t)p * KC + k) * MR + r] * bs[(int64_t)k * j->N + c];
          }
          for (int r = 0; r < mr; ++r) {
            float *dst = j->C + (int64_t)(j->r0 + p * MR + r) * j->ldc + n0 + c0;
            for (int c = 0; c < nr; ++c) dst[c] += acc[r][c];
          }
        }
      }
    }
  }
  for (int r = 0; r < rows; ++r) {
    const int m = j->r0 + r;
    float *dst = j->C + (int64_t)m * j->ldc;
    for (int n = j->c0; n < j->c1; ++n) {
      float v = j->alpha * dst[n];
      if (j->beta != 0.0f) v = fmaf(j->beta, j->Cin[(int64_t)m * j->ldcin + n], v);
      dst[n] = v;
    }
  }
  free(ap);
  return NULL;
}

typedef struct {
  const void *B;
  int b_type, tb;
  int64_t ldb;
  int N, K;
  float *Bp;
  int k0, k1;
} PackJob;

static void *pack_b(void *arg) {
  const PackJob *p = (const PackJob *)arg;
  for (int k = p->k0; k < p->k1; ++k) {
    float *dst = p->Bp + (int64_t)k * p->N;
    if (!p->tb && p->b_type == BT_F32) {
      memcpy(dst, (const float *)p->B + (int64_t)k * p->ldb, sizeof(float) * p->N);
    } else if (!p->tb && p->b_type == BT_BF16) {
      const uint16_t *src = (const uint16_t *)p->B + (int64_t)k * p->ldb;
      for (int n = 0; n < p->N; ++n) {
        const uint32_t u = (uint32_t)src[n] << 16;
        memcpy(&dst[n], &u, 4);
      }
    } else {
      for (int n = 0; n < p->N; ++n)
        dst[n] = p->tb ? widen(p->B, p->b_type, (int64_t)n * p->ldb + k)
                       : widen(p->B, p->b_type, (int64_t)k * p->ldb + n);
    }
  }
  return NULL;
}

/* Rows [row0, row1) of C (fp32, pitch ldc); Cin (fp32, pitch ldcin) is read
 * only when beta != 0.  Returns 0, or -1 on an allocation failure. */
int blocked_gemm(int ta, int tb, int M, int N, int K, float alpha, const void *A, int a_type, int64_t lda,
                 const void *B, int b_type, int64_t ldb, float beta, const float *Cin, int64_t ldcin,
                 float *C, int64_t ldc, int row0, int row1, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (row1 > M) row1 = M;
  if (row0 >= row1 || N <= 0) return 0;
  float *Bp = (float *)malloc(sizeof(float) * (size_t)K * N + 64);
  if (!Bp) return -1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  PackJob *pj = (PackJob *)malloc(sizeof(PackJob) * nthreads);
  Job *jobs = (Job *)malloc(sizeof(Job) * nthreads);
  if (!th || !pj || !jobs) {
    free(Bp); free(th); free(pj); free(jobs);
    return -1;
  }
  for (int t = 0; t < nthreads; ++t) {
    pj[t] = (PackJob){B, b_type, tb, ldb, N, K, Bp, (int)((int64_t)K * t / nthreads),
                      (int)((int64_t)K * (t + 1) / nthreads)};
    pthread_create(&th[t], NULL, pack_b, &pj[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  int status = 0;
  for (int t = 0; t < nthreads; ++t) {
    /* contiguous column ranges in whole NC stripes (the last may be partial) */
    const int stripes = (N + NC - 1) / NC;
    const int s0 = (int)((int64_t)stripes * t / nthreads), s1 = (int)((int64_t)stripes * (t + 1) / nthreads);
    const int c0 = s0 * NC < N ? s0 * NC : N, c1 = s1 * NC < N ? s1 * NC : N;
    jobs[t] = (Job){ta, M, N, K, alpha, beta, A, a_type, lda, Bp, Cin, ldcin, C, ldc, row0, row1, c0, c1};
    pthread_create(&th[t], NULL, worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) {
    void *ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) status = -1;
  }
  free(Bp); free(th); free(pj); free(jobs);
  return status;
}
