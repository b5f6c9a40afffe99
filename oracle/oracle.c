/*
 * CPU oracle for the int8 x int8 -> int32 matrix product.  TEST
 * INFRASTRUCTURE ONLY: nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the bench use it.  It shares no code, header or table with the GPU path.
 *
 * What it computes (the plain definition, no tiling, blocking or fusion):
 *
 *     C[i][j] = wrap32( sum_{k<K} A[i][k] * B[k][j] ),   0 <= i < M, 0 <= j < N
 *
 * with A and B read as signed int8, the sum taken exactly in int64 and wrap32
 * the two's-complement reduction mod 2^32.  This is the product C = A x B that
 * the TPU notes feed through the 256x256 INT8 multiply-accumulate array
 * ("Motivation for and Evaluation of the First Tensor Processing Unit" notes,
 * sections "TPU介绍" and "TPU使用的技术"), written as the naive triple loop
 * whose traffic the CUDA tutorial analyses ("CUDA编程实践", section 3,
 * 矩阵乘, the naive-matmul paragraph).
 *
 * Storage:
 *   A row-major:        A(i,k) = A[i*lda + k]
 *   B row-major:        B(k,j) = B[k*ldb + j]        (b_col_major == 0)
 *   B column-major:     B(k,j) = B[j*ldb + k]        (b_col_major != 0)
 *   C row-major:        C(i,j) = C[i*ldc + j]; entries j >= N of a row untouched
 *
 * The loop order per layout only keeps the innermost loop unit-stride; integer
 * sums are exact, so it does not change any value.  Rows of C are spread over
 * OpenMP threads.  The return value counts elements whose exact sum fell
 * outside the int32 range (they are still written, wrapped).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int32_t wrap32(int64_t s) { return (int32_t)(uint32_t)(uint64_t)s; }

static int out_of_int32(int64_t s) { return s < INT32_MIN || s > INT32_MAX; }

int64_t oracle_gemm_s8s8s32(int64_t M, int64_t N, int64_t K,
                            const int8_t *A, int64_t lda,
                            const int8_t *B, int64_t ldb, int b_col_major,
                            int32_t *C, int64_t ldc)
{
    int64_t overflow = 0;
    if (M <= 0 || N <= 0) return 0;
    if (b_col_major) {
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
        for (int64_t i = 0; i < M; ++i) {
            const int8_t *a = A + i * lda;
            for (int64_t j = 0; j < N; ++j) {
                const int8_t *b = B + j * ldb;
                int64_t s = 0;
                for (int64_t k = 0; k < K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
                overflow += out_of_int32(s);
                C[i * ldc + j] = wrap32(s);
            }
        }
    } else {
#pragma omp parallel reduction(+ : overflow)
        {
            int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; ++i) {
                memset(acc, 0, sizeof(int64_t) * (size_t)N);
                const int8_t *a = A + i * lda;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t aik = a[k];
                    const int8_t *b = B + k * ldb;
                    for (int64_t j = 0; j < N; ++j) acc[j] += aik * (int64_t)b[j];
                }
                for (int64_t j = 0; j < N; ++j) {
                    overflow += out_of_int32(acc[j]);
                    C[i * ldc + j] = wrap32(acc[j]);
                }
            }
            free(acc);
        }
    }
    return overflow;
}

/* One element of C, by the same definition, for sampled checks at sizes where
 * the full product is too slow on the host. */
int32_t oracle_gemm_element(int64_t i, int64_t j, int64_t K,
                            const int8_t *A, int64_t lda,
                            const int8_t *B, int64_t ldb, int b_col_major)
{
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t b = b_col_major ? B[j * ldb + k] : B[k * ldb + j];
        s += (int64_t)A[i * lda + k] * b;
    }
    return wrap32(s);
}

/* Many sampled elements: out[t] = C[rows[t]][cols[t]]. */
void oracle_gemm_elements(int64_t count, const int64_t *rows, const int64_t *cols, int64_t K,
                          const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                          int b_col_major, int32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t)
        out[t] = oracle_gemm_element(rows[t], cols[t], K, A, lda, B, ldb, b_col_major);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count for the following calls (timing on one core or on all). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
