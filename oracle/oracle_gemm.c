/*
 * oracle_gemm.c -- plain fp64 CPU reference for C = A @ B (fp32 operands).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes (the plain definition, with no blocking or reordering):
 *
 *   C[i][j]   = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *   Den[i][j] = sum_{k=0}^{K-1} |A[i][k]| * |B[k][j]|
 *
 * "My Triton From Scratch, Part 14: Shared-Memory Tiles" defines the
 * operation as dot(block<BMxBK>, block<BKxBN>) -> block<BMxBN> (opening
 * section), applied per output tile and accumulated over a runtime K loop
 * (section "Staging inside a runtime K loop").  Masked loads with zero fill
 * (section "Matching the safety mask") make a partial tile contribute exactly
 * the in-range terms, so the tiled computation equals the plain sum above.
 *
 * Arithmetic: every fp32 operand is widened to double; the product of two
 * fp32 values is exact in double (24 + 24 < 53 significand bits), so the only
 * rounding is in the fp64 additions, done for each element by one thread in
 * ascending k.  The result therefore does not depend on the thread count.
 * Built with -O2 -ffp-contract=off and without -ffast-math.
 *
 * Layout: A is row-major with leading dimension lda (element (i,k) at
 * A[i*lda + k]), B likewise with ldb.  Elements in the gap between the
 * logical width and the leading dimension are never read.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t N, K, lda, ldb;
    const float *A, *B;
    const int64_t *rows; /* output row r is matrix row rows[r] */
    int64_t r_begin, r_end;
    double *C, *Den; /* nrows x N, packed */
} rows_job;

/* One output row i: ascending k outer, j inner; each (i,j) accumulator still
 * sees its terms in ascending k. */
static void *rows_worker(void *p) {
    rows_job *job = (rows_job *)p;
    for (int64_t r = job->r_begin; r < job->r_end; ++r) {
        const int64_t i = job->rows[r];
        double *c = job->C + r * job->N;
        double *d = job->Den + r * job->N;
        for (int64_t j = 0; j < job->N; ++j) {
            c[j] = 0.0;
            d[j] = 0.0;
        }
        const float *arow = job->A + i * job->lda;
        for (int64_t k = 0; k < job->K; ++k) {
            const double a = (double)arow[k];
            const double abs_a = fabs(a);
            const float *brow = job->B + k * job->ldb;
            for (int64_t j = 0; j < job->N; ++j) {
                const double b = (double)brow[j];
                c[j] += a * b;
                d[j] += abs_a * fabs(b);
            }
        }
    }
    return NULL;
}

static int clamp_threads(int nthreads, int64_t work) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > work) nthreads = (int)(work > 0 ? work : 1);
    return nthreads;
}

/*
 * Rows of C selected by rows[0..nrows): C and Den are nrows x N (packed).
 * Returns 0 on success, -1 on bad arguments, -2 if a thread cannot start.
 */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     const int64_t *rows, int64_t nrows,
                     double *C, double *Den, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || nrows < 0) return -1;
    if (lda < K || ldb < N) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;

    nthreads = clamp_threads(nthreads, nrows);
    pthread_t tid[256];
    rows_job jobs[256];
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        rows_job *job = &jobs[t];
        job->N = N; job->K = K; job->lda = lda; job->ldb = ldb;
        job->A = A; job->B = B; job->rows = rows;
        job->r_begin = nrows * t / nthreads;
        job->r_end = nrows * (t + 1) / nthreads;
        job->C = C; job->Den = Den;
        if (t == nthreads - 1) break; /* the caller's thread takes the last share */
        if (pthread_create(&tid[t], NULL, rows_worker, job) != 0) { rc = -2; break; }
        ++started;
    }
    if (rc == 0) rows_worker(&jobs[nthreads - 1]);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    return rc;
}

typedef struct {
    int64_t K, lda, ncols;
    const float *A;
    const double *bcols; /* ncols x K: column cols[c] of B, widened */
    int64_t i_begin, i_end;
    double *C, *Den; /* M x ncols, packed */
} cols_job;

static void *cols_worker(void *p) {
    cols_job *job = (cols_job *)p;
    for (int64_t i = job->i_begin; i < job->i_end; ++i) {
        const float *arow = job->A + i * job->lda;
        for (int64_t c = 0; c < job->ncols; ++c) {
            const double *bcol = job->bcols + c * job->K;
            double s = 0.0, d = 0.0;
            for (int64_t k = 0; k < job->K; ++k) {
                const double a = (double)arow[k];
                s += a * bcol[k];
                d += fabs(a) * fabs(bcol[k]);
            }
            job->C[i * job->ncols + c] = s;
            job->Den[i * job->ncols + c] = d;
        }
    }
    return NULL;
}

/*
 * Columns of C selected by cols[0..ncols): C and Den are M x ncols (packed).
 * Same arithmetic as oracle_gemm_rows; the selected columns of B are first
 * copied into contiguous vectors (a change of memory order only).
 */
int oracle_gemm_cols(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     const int64_t *cols, int64_t ncols,
                     double *C, double *Den, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || ncols < 0) return -1;
    if (lda < K || ldb < N) return -1;
    for (int64_t c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return -1;
    if (ncols == 0 || M == 0) return 0;

    double *bcols = (double *)malloc((size_t)(ncols * (K > 0 ? K : 1)) * sizeof(double));
    if (!bcols) return -2;
    for (int64_t c = 0; c < ncols; ++c)
        for (int64_t k = 0; k < K; ++k)
            bcols[c * K + k] = (double)B[k * ldb + cols[c]];

    nthreads = clamp_threads(nthreads, M);
    pthread_t tid[256];
    cols_job jobs[256];
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        cols_job *job = &jobs[t];
        job->K = K; job->lda = lda; job->ncols = ncols;
        job->A = A; job->bcols = bcols;
        job->i_begin = M * t / nthreads;
        job->i_end = M * (t + 1) / nthreads;
        job->C = C; job->Den = Den;
        if (t == nthreads - 1) break;
        if (pthread_create(&tid[t], NULL, cols_worker, job) != 0) { rc = -2; break; }
        ++started;
    }
    if (rc == 0) cols_worker(&jobs[nthreads - 1]);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    free(bcols);
    return rc;
}
