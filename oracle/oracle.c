/*
 * CPU oracle for row-major FP32 matrix multiplication. TEST INFRASTRUCTURE
 * ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg load
 * it; the product library never does, and the two share no code.
 *
 * What it computes (the LeetGPU problem statement in "LeetGPU |
 * 02_Matrix_Multiplication", sections "Problem Description" and CUDA
 * "Approach"; the same definition in section 1 of the study notes "CUDA 学习笔记
 * Matrix Multiplication：LeetGPU FP32 矩阵乘法"):
 *
 *     C[m,k] = sum over n = 0 .. N-1 of A[m,n] * B[n,k]
 *
 * with A (M x N), B (N x K) and C (M x K) all row-major, so that A[m,n] sits at
 * A[m*N + n], B[n,k] at B[n*K + k] and C[m,k] at C[m*K + k].
 *
 * The method reaches exactly this value up to rounding order, so the oracle is
 * the definition written out, in double precision, as the tutorial "分块计算与矩阵乘法"
 * (section 3, its CPU reference) does: every FP32 x FP32 product is exact in
 * double (24 + 24 significant bits <= 53), so the only error is in the N - 1
 * double additions. Alongside each sum it keeps
 *
 *     S[m,k] = sum over n of |A[m,n]| * |B[n,k]|
 *
 * which scales the acceptance tolerance |C_gpu - C| <= 1e-5 * S + 1e-6.
 *
 * The full product walks m, then n, then k: for one row m it adds the term
 * A[m,n] * B[n,k] into every accumulator k before moving to n + 1. That is a
 * loop interchange of the definition; each element still sums its terms in the
 * order n = 0, 1, ..., N - 1. Rows are independent, so OpenMP splits them over
 * threads without changing any element's arithmetic.
 *
 * Pins: the worked examples of the pages, exact rational brute force, numpy's
 * float64 product, and algebraic identities (tests/test_oracle.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Full product. C and S are M*K doubles each (S may be NULL). threads <= 0
 * means the OpenMP default. */
void oracle_gemm(const float *A, const float *B, int64_t M, int64_t N,
                 int64_t K, double *C, double *S, int threads)
{
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(threads)
#endif
    for (int64_t m = 0; m < M; ++m) {
        double *c = C + m * K;
        double *s = S ? S + m * K : NULL;
        for (int64_t k = 0; k < K; ++k) {
            c[k] = 0.0;
            if (s)
                s[k] = 0.0;
        }
        for (int64_t n = 0; n < N; ++n) {
            const double a = (double)A[m * N + n];
            const float *b = B + n * K;
            for (int64_t k = 0; k < K; ++k)
                c[k] += a * (double)b[k];
            if (s) {
                const double abs_a = fabs(a);
                for (int64_t k = 0; k < K; ++k)
                    s[k] += abs_a * fabs((double)b[k]);
            }
        }
    }
}

/* Selected elements only: for i < count, element (rows[i], cols[i]) of the
 * product, its sum taken over n = 0 .. N-1 in order. C and S hold count
 * doubles each (S may be NULL). Returns the number of out-of-range
 * coordinates found (those elements are left untouched). */
int64_t oracle_gemm_at(const float *A, const float *B, int64_t M, int64_t N,
                       int64_t K, const int64_t *rows, const int64_t *cols,
                       int64_t count, double *C, double *S)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = rows[i], k = cols[i];
        if (m < 0 || m >= M || k < 0 || k >= K) {
            ++bad;
            continue;
        }
        double c = 0.0, s = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a = (double)A[m * N + n];
            const double b = (double)B[n * K + k];
            c += a * b;
            s += fabs(a) * fabs(b);
        }
        C[i] = c;
        if (S)
            S[i] = s;
    }
    return bad;
}

/* Threads the full product would use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
