/*
 * gemm_oracle.c -- the CPU oracle for row-major GEMM.  TEST INFRASTRUCTURE ONLY:
 * it exists to check the HIP library and is called from the tests, the smoke
 * check and the benchmark's CPU-baseline leg, never from the product path.
 *
 * What it computes (MindNotes 'GEMM' page, section "core problem and
 * arithmetic characteristics": C = alpha*op(A)op(B) + beta*C with op(A) of
 * size MxK, op(B) of size KxN, C of size MxN, where C[i][j] is the dot product
 * of row i of op(A) with column j of op(B); op is the identity or the
 * transpose, chosen per operand):
 *
 *     ref[i][j]   = alpha * sum_{k=0}^{K-1} a(i,k)*b(k,j)  + beta * C[i][j]
 *     bound[i][j] = |alpha| * sum_k |a(i,k)|*|b(k,j)|     + |beta| * |C[i][j]|
 *
 * with a(i,k) = op(A)[i][k] and b(k,j) = op(B)[k][j].
 *
 * in IEEE double precision.  The loop is the plain triple loop of the ssxxe.cn
 * V100 SGEMM article, section 1.2 (its CPU reference), with the accumulator
 * widened from float to double: for each output row i, k runs in ascending
 * order and each product A[i][k]*B[k][j] is added to a double accumulator for
 * column j (the i-k-j order adds exactly the same terms in exactly the same
 * order per element as i-j-k; it only walks B by rows).  Every input value is a
 * float (the fp16 path hands over its binary16 values widened exactly), so each
 * product of two of them is exact in double; only the additions round.
 *
 * Storage (MindNotes 'GEMM' page, section "Leading Dimension (lda, ldb, ldc)"):
 * every matrix is row-major with its own leading dimension.  a(i,k) is
 * A[i*lda + k], or A[k*lda + i] when A is stored transposed (K x M); b(k,j) is
 * B[k*ldb + j], or B[j*ldb + k] when B is stored transposed (N x K); (i,j) of C
 * is C[i*ldc + j].  The ld-width pad at the end of each row is never read.
 *
 * Where the pages say nothing the BLAS reference semantics are taken: C is not
 * read when beta == 0 (so a C full of NaN cannot leak in), A and B are not read
 * when alpha == 0, and K == 0 leaves ref = beta*C.
 *
 * Rows may be computed for a chosen subset (``rows``), and the rows are shared
 * out over POSIX threads; neither changes any element's summation order.
 *
 * Build: gcc -O3 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread
 * (no contraction of a*b+c into an FMA, no reassociation).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdlib.h>

typedef struct {
    int transA, transB;
    int M, N, K;
    double alpha, beta;
    const float *A, *B, *C;
    long long lda, ldb, ldc;
    const int *rows;   /* NULL: rows 0..nrows-1 */
    int nrows;
    double *ref, *bound; /* nrows x N, row r holds output row rows[r] */
    int next;          /* next row index to take (guarded by lock) */
    pthread_mutex_t lock;
} oracle_job;

static void oracle_one_row(const oracle_job *jb, int r, double *acc, double *acc_abs)
{
    const int i = jb->rows ? jb->rows[r] : r;
    const int N = jb->N;
    for (int j = 0; j < N; ++j) {
        acc[j] = 0.0;
        acc_abs[j] = 0.0;
    }
    if (jb->alpha != 0.0) {
        for (int k = 0; k < jb->K; ++k) {
            const double a = jb->transA ? (double)jb->A[(size_t)k * (size_t)jb->lda + (size_t)i]
                                        : (double)jb->A[(size_t)i * (size_t)jb->lda + (size_t)k];
            const double a_abs = fabs(a);
            for (int j = 0; j < N; ++j) {
                const double b = jb->transB ? (double)jb->B[(size_t)j * (size_t)jb->ldb + (size_t)k]
                                            : (double)jb->B[(size_t)k * (size_t)jb->ldb + (size_t)j];
                acc[j] += a * b;
                acc_abs[j] += a_abs * fabs(b);
            }
        }
    }
    double *ref = jb->ref + (size_t)r * (size_t)N;
    double *bound = jb->bound + (size_t)r * (size_t)N;
    const float *crow = jb->C ? jb->C + (size_t)i * (size_t)jb->ldc : NULL;
    for (int j = 0; j < N; ++j) {
        double ab = jb->alpha != 0.0 ? jb->alpha * acc[j] : 0.0;
        double ab_bound = jb->alpha != 0.0 ? fabs(jb->alpha) * acc_abs[j] : 0.0;
        if (jb->beta != 0.0) {
            const double c = (double)crow[j];
            ref[j] = ab + jb->beta * c;
            bound[j] = ab_bound + fabs(jb->beta) * fabs(c);
        } else {
            ref[j] = ab;
            bound[j] = ab_bound;
        }
    }
}

static void *oracle_worker(void *arg)
{
    oracle_job *jb = (oracle_job *)arg;
    double *acc = (double *)malloc(sizeof(double) * (size_t)(jb->N > 0 ? jb->N : 1) * 2);
    if (!acc) return (void *)1;
    double *acc_abs = acc + (jb->N > 0 ? jb->N : 1);
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        int r = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (r >= jb->nrows) break;
        oracle_one_row(jb, r, acc, acc_abs);
    }
    free(acc);
    return NULL;
}

/*
 * oracle_gemm: ref and bound for the rows listed in ``rows`` (or all M rows
 * when rows == NULL, in which case nrows must equal M).  transA / transB
 * (0 or 1) say whether A / B are stored transposed.  ``C`` may be NULL when
 * beta == 0.  Returns 0 on success, -1 on bad arguments, -2 on allocation or
 * thread failure.
 */
int oracle_gemm(int transA, int transB, int M, int N, int K, double alpha,
                const float *A, long long lda, const float *B, long long ldb,
                double beta, const float *C, long long ldc,
                const int *rows, int nrows, double *ref, double *bound, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0) return -1;
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return -1;
    if (!rows && nrows != M) return -1;
    const int a_cols = transA ? M : K, b_cols = transB ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1)) return -1;
    if (beta != 0.0 && !C && nrows > 0 && N > 0) return -1;
    if (rows)
        for (int r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;

    oracle_job jb;
    jb.transA = transA; jb.transB = transB;
    jb.M = M; jb.N = N; jb.K = K;
    jb.alpha = alpha; jb.beta = beta;
    jb.A = A; jb.B = B; jb.C = C;
    jb.lda = lda; jb.ldb = ldb; jb.ldc = ldc;
    jb.rows = rows; jb.nrows = nrows;
    jb.ref = ref; jb.bound = bound;
    jb.next = 0;
    pthread_mutex_init(&jb.lock, NULL);

    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows;
    int rc = 0;
    if (nthreads == 1) {
        if (oracle_worker(&jb) != NULL) rc = -2;
    } else {
        pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
        if (!tid) {
            pthread_mutex_destroy(&jb.lock);
            return -2;
        }
        int started = 0;
        for (; started < nthreads; ++started)
            if (pthread_create(&tid[started], NULL, oracle_worker, &jb) != 0) break;
        if (started == 0) rc = -2;
        for (int t = 0; t < started; ++t) {
            void *ret = NULL;
            pthread_join(tid[t], &ret);
            if (ret != NULL) rc = -2;
        }
        free(tid);
    }
    pthread_mutex_destroy(&jb.lock);
    return rc;
}
