/*
 * Plain CPU reference for single-precision GEMM.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the CPU-baseline leg of the benchmark call
 * it; the product path never does.  It shares no code, header or table with
 * the HIP library.
 *
 * What it computes (the plain definition of the product):
 *   C = A x B, A is M x K, B is K x N, C is M x N, all row-major
 *   ("4.1 CUDA GEMM operator performance optimization", section 1.1 "What
 *   GEMM computes"; row-major indexing as in its section 3.1 naive kernel).
 *   For every checked (i, j):
 *     ref[i][j]  = sum_{k=0..K-1} (double)A[i*lda+k] * (double)B[k*ldb+j]
 *     absb[i][j] = sum_{k=0..K-1} |(double)A[i*lda+k] * (double)B[k*ldb+j]|
 *   The sums run over k in ascending order, in double precision, following
 *   the lab of Module 14 in the DD2360 workbook "Applied GPU Programming"
 *   (section 14.3, "Lab: tiled matmul, square case": a CPU reference that
 *   accumulates in double).  absb is the scale of the acceptance bound
 *   |C - ref| <= 1e-4 * absb.
 *
 * Why the result is well defined: a product of two binary32 values has at
 * most 48 significant bits, so it is exact in binary64; only the additions
 * round.  Each element therefore sees one fixed sequence of roundings no
 * matter how the loops over i and j are nested, and whether the compiler
 * fuses a multiply into an add cannot change a value.  The full routine walks
 * k in the middle loop (i, k, j) with a row of double accumulators; each
 * element still receives its products in ascending k.  Build without
 * -ffast-math / -Ofast (they allow reassociation).
 *
 * Threads split the output rows (full routine) or the sample list (sampled
 * routine); each output is written by exactly one thread, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2
#define ORACLE_ETHREAD 3

typedef struct {
    int64_t M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    double *ref;
    double *absb;
    int64_t ldr;
    /* full routine: rows [lo, hi); sampled routine: samples [lo, hi) */
    int64_t lo, hi;
    const int64_t *rows;
    const int64_t *cols;
} job_t;

static void *full_rows(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t i = j->lo; i < j->hi; ++i) {
        double *r = j->ref + i * j->ldr;
        double *s = j->absb + i * j->ldr;
        for (int64_t c = 0; c < j->N; ++c) {
            r[c] = 0.0;
            s[c] = 0.0;
        }
        const float *arow = j->A + i * j->lda;
        for (int64_t k = 0; k < j->K; ++k) {
            const double a = (double)arow[k];
            const float *brow = j->B + k * j->ldb;
            for (int64_t c = 0; c < j->N; ++c) {
                const double p = a * (double)brow[c];
                r[c] += p;
                s[c] += fabs(p);
            }
        }
    }
    return NULL;
}

static void *sampled_elems(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t t = j->lo; t < j->hi; ++t) {
        const int64_t i = j->rows[t];
        const int64_t c = j->cols[t];
        const float *arow = j->A + i * j->lda;
        double sum = 0.0, sabs = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            const double p = (double)arow[k] * (double)j->B[k * j->ldb + c];
            sum += p;
            sabs += fabs(p);
        }
        j->ref[t] = sum;
        j->absb[t] = sabs;
    }
    return NULL;
}

/* Split [0, count) into nthreads contiguous chunks and run fn on each. */
static int run_split(job_t proto, int64_t count, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1)
        nthreads = 1;
    if ((int64_t)nthreads > count)
        nthreads = count > 0 ? (int)count : 1;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return ORACLE_ENOMEM;
    }
    int started = 0, rc = ORACLE_OK;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].lo = count * t / nthreads;
        jobs[t].hi = count * (t + 1) / nthreads;
        if (t == nthreads - 1)
            break; /* the calling thread takes the last chunk */
        if (pthread_create(&tids[t], NULL, fn, &jobs[t]) != 0) {
            rc = ORACLE_ETHREAD;
            break;
        }
        ++started;
    }
    if (rc == ORACLE_OK)
        fn(&jobs[nthreads - 1]);
    for (int t = 0; t < started; ++t)
        pthread_join(tids[t], NULL);
    free(jobs);
    free(tids);
    return rc;
}

/* Every output of rows [0, M): ref and absb are M x N with row stride ldr. */
int oracle_sgemm_full(int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda,
                      const float *B, int64_t ldb,
                      double *ref, double *absb, int64_t ldr,
                      int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || ldr < N || (K > 0 && lda < K) || (N > 0 && ldb < N))
        return ORACLE_EINVAL;
    if (M == 0 || N == 0)
        return ORACLE_OK;
    if (!ref || !absb || (K > 0 && (!A || !B)))
        return ORACLE_EINVAL;
    job_t proto;
    memset(&proto, 0, sizeof proto);
    proto.M = M; proto.N = N; proto.K = K;
    proto.A = A; proto.lda = lda; proto.B = B; proto.ldb = ldb;
    proto.ref = ref; proto.absb = absb; proto.ldr = ldr;
    return run_split(proto, M, nthreads, full_rows);
}

/* The outputs (rows[t], cols[t]) for t < count, into ref[t] and absb[t]. */
int oracle_sgemm_sampled(int64_t M, int64_t N, int64_t K,
                         const float *A, int64_t lda,
                         const float *B, int64_t ldb,
                         int64_t count, const int64_t *rows, const int64_t *cols,
                         double *ref, double *absb, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0 || (K > 0 && lda < K) || (N > 0 && ldb < N))
        return ORACLE_EINVAL;
    if (count == 0)
        return ORACLE_OK;
    if (!rows || !cols || !ref || !absb || (K > 0 && (!A || !B)))
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return ORACLE_EINVAL;
    job_t proto;
    memset(&proto, 0, sizeof proto);
    proto.M = M; proto.N = N; proto.K = K;
    proto.A = A; proto.lda = lda; proto.B = B; proto.ldb = ldb;
    proto.ref = ref; proto.absb = absb;
    proto.rows = rows; proto.cols = cols;
    return run_split(proto, count, nthreads, sampled_elems);
}
