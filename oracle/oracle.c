/*
 * Oracle for dense GEMM: a plain, slow, obviously correct CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark use it.  It shares no code, header
 * or constant with the GPU library.
 *
 * What it computes ("Learning to develop for GPUs through the GEMM operation",
 * section "Matrix product"): for A of size M x K and B of size K x N the
 * product C is M x N, and each C element is the sum over k of the products of
 * the matching row of A and column of B:
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *
 * The page writes it as three nested loops over a column-major layout.  Here
 * the same definition is written for row-major storage with leading
 * dimensions (element strides between consecutive rows), as the library's
 * interface uses, and with C overwritten rather than accumulated into:
 *
 *     C_ref[i*ldc + j] = sum_k (double)A[i*lda + k] * (double)B[k*ldb + j]
 *     S    [i*lds + j] = sum_k |A[i*lda + k]| * |B[k*ldb + j]|
 *
 * Both sums run in ascending k, in double precision.  The loop order is
 * i-k-j so that the inner j loop walks rows of B and C contiguously; each
 * element's sum still sees its terms in ascending k, so the order is the same
 * as the i-j-k triple loop.  S is the scale used by the tolerance test
 * |C - C_ref| <= tol * S.
 *
 * Exactness: a product of two fp32 (24-bit significand) or two bf16 (8-bit)
 * values is exact in fp64 (53-bit significand).  The only rounding is the fp64
 * accumulation, bounded by (K-1) * 2^-53 * S.
 *
 * bf16 inputs arrive as raw 16-bit patterns; a bf16 value is the upper half of
 * an IEEE binary32, so it is decoded exactly by placing the 16 bits in the high
 * half of a 32-bit word.
 *
 * Rows are split across POSIX threads; each thread owns whole rows of C and S,
 * so the threading does not change any sum.
 *
 * Status codes: 0 on success, -1 on an invalid argument (negative size, a
 * leading dimension smaller than its row, a null pointer with a non-empty
 * operand), -2 if a thread could not be started.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { IN_F32 = 0, IN_BF16 = 1 };

/* Decode one operand element to double, exactly. */
static double load_elem(const void *base, int kind, int64_t idx)
{
    if (kind == IN_F32)
        return (double)((const float *)base)[idx];
    uint32_t w = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

typedef struct {
    int64_t M, N, K;
    const void *A; int64_t lda;
    const void *B; int64_t ldb;
    double *C; int64_t ldc;
    double *S; int64_t lds;
    int kind;
    int64_t row_begin, row_end;
    double *bscratch; /* N doubles: one decoded row of B */
} rows_job;

/* C_ref and S for rows [row_begin, row_end): i-k-j order, ascending k. */
static void gemm_rows(const rows_job *jb)
{
    const int64_t N = jb->N, K = jb->K;
    for (int64_t i = jb->row_begin; i < jb->row_end; ++i) {
        double *c = jb->C + i * jb->ldc;
        double *s = jb->S ? jb->S + i * jb->lds : NULL;
        for (int64_t j = 0; j < N; ++j) {
            c[j] = 0.0;
            if (s) s[j] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_elem(jb->A, jb->kind, i * jb->lda + k);
            const double abs_a = fabs(a);
            double *b = jb->bscratch;
            for (int64_t j = 0; j < N; ++j)
                b[j] = load_elem(jb->B, jb->kind, k * jb->ldb + j);
            for (int64_t j = 0; j < N; ++j)
                c[j] += a * b[j];
            if (s)
                for (int64_t j = 0; j < N; ++j)
                    s[j] += abs_a * fabs(b[j]);
        }
    }
}

static void *gemm_rows_thread(void *arg)
{
    gemm_rows((const rows_job *)arg);
    return NULL;
}

static int check_args(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                      const void *B, int64_t ldb, const double *C, int64_t ldc,
                      const double *S, int64_t lds)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (lda < (K > 0 ? K : 1) || ldb < (N > 0 ? N : 1) || ldc < (N > 0 ? N : 1))
        return -1;
    if (S && lds < (N > 0 ? N : 1)) return -1;
    if (M > 0 && N > 0 && !C) return -1;
    if (M > 0 && K > 0 && !A) return -1;
    if (K > 0 && N > 0 && !B) return -1;
    return 0;
}

static int oracle_gemm(int kind, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, const void *B, int64_t ldb,
                       double *C, int64_t ldc, double *S, int64_t lds, int nthreads)
{
    int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc, S, lds);
    if (rc) return rc;
    if (M == 0 || N == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = (int)M;

    rows_job *jobs = calloc((size_t)nthreads, sizeof *jobs);
    pthread_t *tids = calloc((size_t)nthreads, sizeof *tids);
    double *scratch = malloc((size_t)nthreads * (size_t)N * sizeof(double));
    if (!jobs || !tids || !scratch) {
        free(jobs); free(tids); free(scratch);
        return -2;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        rows_job *jb = &jobs[t];
        jb->M = M; jb->N = N; jb->K = K;
        jb->A = A; jb->lda = lda; jb->B = B; jb->ldb = ldb;
        jb->C = C; jb->ldc = ldc; jb->S = S; jb->lds = lds;
        jb->kind = kind;
        jb->row_begin = M * t / nthreads;
        jb->row_end = M * (t + 1) / nthreads;
        jb->bscratch = scratch + (size_t)t * (size_t)N;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, gemm_rows_thread, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    gemm_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    /* If a thread failed to start, its rows were not computed: rc says so. */
    free(jobs); free(tids); free(scratch);
    return rc;
}

int oracle_gemm_f32(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *C, int64_t ldc, double *S, int64_t lds, int nthreads)
{
    return oracle_gemm(IN_F32, M, N, K, A, lda, B, ldb, C, ldc, S, lds, nthreads);
}

int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                     double *C, int64_t ldc, double *S, int64_t lds, int nthreads)
{
    return oracle_gemm(IN_BF16, M, N, K, A, lda, B, ldb, C, ldc, S, lds, nthreads);
}

/*
 * Selected entries only: for each t, the single element (I[t], J[t]) of C_ref
 * and of S, as the dot product of row I[t] of A with column J[t] of B in
 * ascending k.  Used to check full-size results on a sample of positions.
 */
static int oracle_entries(int kind, int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda, const void *B, int64_t ldb,
                          int64_t count, const int64_t *I, const int64_t *J,
                          double *C, double *S)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (lda < (K > 0 ? K : 1) || ldb < (N > 0 ? N : 1)) return -1;
    if (count > 0 && (!I || !J || !C)) return -1;
    if (K > 0 && count > 0 && (!A || !B)) return -1;
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = I[t], j = J[t];
        if (i < 0 || i >= M || j < 0 || j >= N) return -1;
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_elem(A, kind, i * lda + k);
            const double b = load_elem(B, kind, k * ldb + j);
            c += a * b;
            s += fabs(a) * fabs(b);
        }
        C[t] = c;
        if (S) S[t] = s;
    }
    return 0;
}

int oracle_entries_f32(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda, const float *B, int64_t ldb,
                       int64_t count, const int64_t *I, const int64_t *J,
                       double *C, double *S)
{
    return oracle_entries(IN_F32, M, N, K, A, lda, B, ldb, count, I, J, C, S);
}

int oracle_entries_bf16(int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                        int64_t count, const int64_t *I, const int64_t *J,
                        double *C, double *S)
{
    return oracle_entries(IN_BF16, M, N, K, A, lda, B, ldb, count, I, J, C, S);
}
