/*
 * Dense FP32 GEMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU product path never calls it, and it shares
 * no code, header or constant with the GPU path.
 *
 * What it computes (the "golden reference" of the UIUC ECE408 Lecture 12 final
 * project page, project_template.cu section 3): for every output element
 *
 *     C(i,j) = (float) S(i,j),   S(i,j) = sum over k = 0, 1, ..., K-1 of
 *                                         (double)A(i,k) * (double)B(k,j)
 *
 * with S starting at +0.0, accumulated in IEEE binary64 with k ascending, and
 * the final conversion to binary32 rounding to nearest even.  The page writes
 * the loop for packed row-major operands; here A(i,k) = A[i*lda + k],
 * B(k,j) = B[k*ldb + j] and C(i,j) = C[i*ldc + j] (the usual row-major
 * leading-dimension convention; with lda = K, ldb = ldc = N it is the page's
 * loop exactly).
 *
 * Build: plain C with the host compiler, -O2 -ffp-contract=off, OpenMP over
 * output rows.  A row is computed by one thread and no element's summation
 * order depends on the thread count, so results are identical for any
 * OMP_NUM_THREADS.
 */
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/*
 * Full product.  Loop order i -> k -> j with one binary64 accumulator per
 * output column of row i: every accumulator S(i,j) still receives its terms
 * in k-ascending order, exactly as the i -> j -> k loop on the page does, while
 * B is read along its rows.  Returns 0, or -1 if scratch memory is missing.
 */
int oracle_gemm_f32(int M, int N, int K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    float *C, int64_t ldc)
{
    int failed = 0;
    if (M <= 0 || N <= 0)
        return 0;
#pragma omp parallel reduction(| : failed)
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (acc == NULL) {
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int i = 0; i < M; ++i) {
                for (int j = 0; j < N; ++j)
                    acc[j] = 0.0;
                for (int k = 0; k < K; ++k) {
                    const double a = (double)A[(int64_t)i * lda + k];
                    const float *brow = B + (int64_t)k * ldb;
                    for (int j = 0; j < N; ++j)
                        acc[j] += a * (double)brow[j];
                }
                for (int j = 0; j < N; ++j)
                    C[(int64_t)i * ldc + j] = (float)acc[j];
            }
            free(acc);
        }
    }
    return failed ? -1 : 0;
}

/*
 * Selected elements only: out[t] = C(rows[t], cols[t]) by the same definition,
 * one k-ascending binary64 dot product per requested element.  Used where the
 * full product is too large to compute on the host.
 */
void oracle_gemm_f32_at(int K,
                        const float *A, int64_t lda,
                        const float *B, int64_t ldb,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t];
        const int64_t j = cols[t];
        double s = 0.0;
        for (int k = 0; k < K; ++k)
            s += (double)A[i * lda + k] * (double)B[(int64_t)k * ldb + j];
        out[t] = (float)s;
    }
}

/* Threads an OpenMP parallel region of this library will use. */
int oracle_threads(void)
{
    return omp_get_max_threads();
}

/* Sets that thread count (n >= 1); rows are still split the same way, so
 * the results do not change. */
void oracle_set_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}
