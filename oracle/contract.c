/*
 * The GEMM contraction written as the plain triple loop, in float64 --
 * test infrastructure, not product code.
 *
 * The DeepGEMM page (zwxr.cn/news/240083) keeps the naive triple loop as the
 * golden reference its optimised kernels are checked against (section 3.2,
 * the baseline that indexes A[m*K + k] and B[k*N + n]).  This file is that
 * loop over operands already decoded to float64 by the Python side of the
 * oracle:
 *
 *     y[i][j] = sum_{k = 0 .. K-1} a[i][k] * b[k][j]
 *     d[i][j] = sum_{k = 0 .. K-1} |a[i][k] * b[k][j]|
 *
 * d is the magnitude sum the error metric divides by.  The loops run in
 * i-k-j order: for every output element the terms are added one at a time
 * with k ascending, the same order as the textbook i-j-k loop; only the
 * innermost index walks along a row of b, and every j is independent of
 * every other.  Each product is rounded once and added with one rounding
 * (no fused multiply-add: built with -ffp-contract=off).  Rows i are shared
 * out to POSIX threads in contiguous blocks; a row is computed by exactly
 * one thread, so the thread count never changes a result bit.
 *
 * Strides are in elements; the inner stride is 1.  Returns 0 on success,
 * -1 on a bad argument or when a thread cannot be started.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const double* a;
  const double* b;
  double* y;
  double* d;
  int64_t lda, ldb, ldy;
  int64_t row0, row1, N, K;
} rows_job;

static void contract_rows(const rows_job* jb) {
  for (int64_t i = jb->row0; i < jb->row1; ++i) {
    double* yi = jb->y + i * jb->ldy;
    double* di = jb->d + i * jb->ldy;
    memset(yi, 0, (size_t)jb->N * sizeof(double));
    memset(di, 0, (size_t)jb->N * sizeof(double));
    for (int64_t k = 0; k < jb->K; ++k) {
      const double aik = jb->a[i * jb->lda + k];
      const double* bk = jb->b + k * jb->ldb;
      for (int64_t j = 0; j < jb->N; ++j) {
        const double t = aik * bk[j];
        yi[j] += t;
        di[j] += fabs(t);
      }
    }
  }
}

static void* contract_thread(void* arg) {
  contract_rows((const rows_job*)arg);
  return NULL;
}

int oracle_contract_f64(const double* a, int64_t lda, const double* b, int64_t ldb, double* y,
                        double* d, int64_t ldy, int64_t M, int64_t N, int64_t K, int threads) {
  if (M < 0 || N < 0 || K < 0 || y == NULL || d == NULL || ldy < N) return -1;
  if (M > 0 && K > 0 && (a == NULL || lda < K)) return -1;
  if (K > 0 && N > 0 && (b == NULL || ldb < N)) return -1;
  if (M == 0 || N == 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > M) threads = (int)M;
  rows_job* jobs = (rows_job*)calloc((size_t)threads, sizeof(rows_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
  if (jobs == NULL || tids == NULL) {
    free(jobs);
    free(tids);
    return -1;
  }
  for (int t = 0; t < threads; ++t) {
    rows_job* jb = &jobs[t];
    jb->a = a;
    jb->b = b;
    jb->y = y;
    jb->d = d;
    jb->lda = lda;
    jb->ldb = ldb;
    jb->ldy = ldy;
    jb->row0 = M * t / threads;
    jb->row1 = M * (t + 1) / threads;
    jb->N = N;
    jb->K = K;
  }
  int started = 0, rc = 0;
  for (int t = 1; t < threads; ++t) {
    if (pthread_create(&tids[t], NULL, contract_thread, &jobs[t]) != 0) {
      rc = -1;
      break;
    }
    started = t;
  }
  contract_rows(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
  /* Rows of threads that could not be started are done here, serially. */
  for (int t = started + 1; rc != 0 && t < threads; ++t) contract_rows(&jobs[t]);
  free(jobs);
  free(tids);
  return 0;
}
