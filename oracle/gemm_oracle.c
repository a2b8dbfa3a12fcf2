/*
 * CPU oracle for the single-precision dense matrix product C = A.B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the HIP
 * library and is built by gcc, not hipcc.
 *
 * What it computes (the plain definition, written out):
 *   C[i][j] = sum_{k=0}^{K-1} A[i][k] * B(k, j)          for 0 <= i < M, 0 <= j < N
 *   S[i][j] = sum_{k=0}^{K-1} |A[i][k] * B(k, j)|        (error scale for the tolerance)
 * with
 *   A[i][k]  = A[i*lda + k]   if layout_a == 0 (A row-major)
 *            = A[k*lda + i]   if layout_a == 1 (A column-major: column k contiguous)
 *   B(k, j)  = B[k*ldb + j]   if layout_b == 0 (B row-major)
 *            = B[j*ldb + k]   if layout_b == 1 (B column-major: column j contiguous)
 * The column-major A index is the pages' column-major convention applied to
 * the first operand (the reading of the linear-layer layouts: transposed A).
 *
 * Sources (pages: "GEMM 性能优化", "GPU 算子优化中的数据复用",
 * "PMPP Chapter 06: Performance considerations"):
 *  - C = A x B and its 2*M*N*K flop count (one multiply plus one add per
 *    (i,j,k)): "GEMM 性能优化", section 指标与目标; "GPU 算子优化中的数据复用",
 *    section 2 (什么是数据复用).
 *  - the sum runs along K, so splitting K into pieces and adding the partial
 *    sums gives the same product: "GEMM 性能优化", 台阶 1 (Shared Memory Tiling).
 *  - index conventions (A and C row-major, B row-major M[k*Width+col] or
 *    column-major M[col*Width+k]) and out-of-range terms contributing nothing:
 *    "PMPP Chapter 06", section 1 (Memory coalescing) and its corner-turning
 *    example.
 *
 * Arithmetic: every product of two float32 values is exact in double (24+24
 * significant bits <= 53), and each element is summed sequentially in k order
 * 0..K-1 in double.  No blocking, no reordering of any element's sum, no fused
 * multiply-add (built with -ffp-contract=off).  The row-major-B routine walks
 * k in the outer loop and j in the inner loop; that only interleaves work on
 * *different* elements, each element still sees the terms k = 0, 1, ..., K-1
 * in that order, so the result is bit-identical to the i-j-k triple loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1

static int oracle_args_ok(int64_t m, int64_t n, int64_t k, int layout_a, int layout_b,
                          int64_t lda, int64_t ldb)
{
    if (m < 0 || n < 0 || k < 0) return 0;
    if (layout_a != 0 && layout_a != 1) return 0;
    if (layout_b != 0 && layout_b != 1) return 0;
    if (layout_a == 0 && lda < k) return 0;
    if (layout_a == 1 && lda < m) return 0;
    if (layout_b == 0 && ldb < n) return 0;
    if (layout_b == 1 && ldb < k) return 0;
    return 1;
}

/* A[i][kk] for either layout of A. */
static double a_at(const float *A, int64_t lda, int layout_a, int64_t i, int64_t kk)
{
    return layout_a == 0 ? (double)A[i * lda + kk] : (double)A[kk * lda + i];
}

/* Full product.  C and S are M x N double arrays with row stride ldr. */
int oracle_gemm_f64_ex(int64_t m, int64_t n, int64_t k, int layout_a, int layout_b,
                       const float *A, int64_t lda,
                       const float *B, int64_t ldb,
                       double *C, double *S, int64_t ldr)
{
    if (!oracle_args_ok(m, n, k, layout_a, layout_b, lda, ldb) || ldr < n) return ORACLE_BAD_ARGS;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        double *c = C + i * ldr;
        double *s = S + i * ldr;
        if (layout_b == 0) {
            for (int64_t j = 0; j < n; ++j) { c[j] = 0.0; s[j] = 0.0; }
            for (int64_t kk = 0; kk < k; ++kk) {
                const double a = a_at(A, lda, layout_a, i, kk);
                const float *b_row = B + kk * ldb;          /* B(kk, j) = B[kk*ldb + j] */
                for (int64_t j = 0; j < n; ++j) {
                    const double p = a * (double)b_row[j];
                    c[j] += p;
                    s[j] += fabs(p);
                }
            }
        } else {
            for (int64_t j = 0; j < n; ++j) {
                const float *b_col = B + j * ldb;           /* B(kk, j) = B[j*ldb + kk] */
                double acc = 0.0, acc_abs = 0.0;
                for (int64_t kk = 0; kk < k; ++kk) {
                    const double p = a_at(A, lda, layout_a, i, kk) * (double)b_col[kk];
                    acc += p;
                    acc_abs += fabs(p);
                }
                c[j] = acc;
                s[j] = acc_abs;
            }
        }
    }
    return ORACLE_OK;
}

/* Row-major A. */
int oracle_gemm_f64(int64_t m, int64_t n, int64_t k, int layout_b,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    double *C, double *S, int64_t ldr)
{
    return oracle_gemm_f64_ex(m, n, k, 0, layout_b, A, lda, B, ldb, C, S, ldr);
}

/* The same sum for a list of individual elements (rows[t], cols[t]); used where
 * a full product would take too long on the host. */
int oracle_gemm_f64_sampled_ex(int64_t m, int64_t n, int64_t k, int layout_a, int layout_b,
                               const float *A, int64_t lda,
                               const float *B, int64_t ldb,
                               int64_t count, const int64_t *rows, const int64_t *cols,
                               double *c_out, double *s_out)
{
    if (!oracle_args_ok(m, n, k, layout_a, layout_b, lda, ldb) || count < 0) return ORACLE_BAD_ARGS;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= n) return ORACLE_BAD_ARGS;

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            const double b = layout_b == 0 ? (double)B[kk * ldb + j] : (double)B[j * ldb + kk];
            const double p = a_at(A, lda, layout_a, i, kk) * b;
            acc += p;
            acc_abs += fabs(p);
        }
        c_out[t] = acc;
        s_out[t] = acc_abs;
    }
    return ORACLE_OK;
}

/* Row-major A. */
int oracle_gemm_f64_sampled(int64_t m, int64_t n, int64_t k, int layout_b,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            int64_t count, const int64_t *rows, const int64_t *cols,
                            double *c_out, double *s_out)
{
    return oracle_gemm_f64_sampled_ex(m, n, k, 0, layout_b, A, lda, B, ldb, count, rows, cols, c_out, s_out);
}

/* Number of OpenMP threads a parallel region here uses (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the OpenMP thread count of later calls (the benchmark times the small
 * case single-threaded as well); returns the previous count. */
int oracle_set_num_threads(int threads)
{
#ifdef _OPENMP
    int before = omp_get_max_threads();
    if (threads > 0) omp_set_num_threads(threads);
    return before;
#else
    (void)threads;
    return 1;
#endif
}
