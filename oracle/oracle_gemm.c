/*
 * CPU oracle for the bf16 GEMM  C[M,N] = A[M,K] * B[K,N]  (fp32 accumulate,
 * bf16 result on the device; fp64 accumulate and one final rounding here).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no header, helper or
 * constant with the HIP library.
 *
 * What it follows.  The problem every page turns on is a tiled matmul whose
 * consumer accumulates in fp32 and whose epilogue converts the fp32 results
 * to bf16 ("Allow separate sub-DAG for load and compute warp groups with
 * warp-specialized circular buffering", section "Pseudo-code": the compute
 * warp group's epilogue converts fp32 results to bf16).  The pipelining,
 * circular buffering and scheduling on the pages ("Use mbarrier for WAR for
 * circular buffering", both code listings; the same issue's "Scheduling
 * Proposal") change *when* the operands arrive, never *what* is summed, so the
 * oracle is the plain definition of the product:
 *
 *   C[i][j] = round_bf16( sum_{k=0}^{K-1} A[i][k] * B[k][j] )
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes of the repository):
 *   - final rounding is IEEE round-to-nearest, ties to even, applied once,
 *     directly from the fp64 sum (never through fp32, which would round twice);
 *   - the sum is taken in increasing k, starting from +0.0;
 *   - a bf16 value is the upper half of an IEEE binary32 word, so decoding is
 *     exact: (bits << 16) reinterpreted as binary32, then widened to fp64;
 *   - every product of two bf16 values is exact in fp64 (8-bit x 8-bit
 *     significands), so fused or unfused multiply-add give the same sum;
 *   - NaN inputs give the canonical quiet NaN 0x7FC0; results whose magnitude
 *     rounds above the largest finite bf16 become +-Inf.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bits -> fp64, exact. */
static double decode_bf16(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* fp64 -> bf16 bits, round to nearest, ties to even, in one step.
 *
 * bf16 keeps 8 significant bits (1 implicit + 7 stored) and the binary32
 * exponent range: normals cover [2^-126, 2^128) with quantum 2^(E-7) in the
 * binade [2^E, 2^(E+1)); subnormals have the fixed quantum 2^-133.  The value
 * is scaled by its quantum (an exact power-of-two scaling), rounded to an
 * integer with ties to even, and scaled back.  The rounded value is exactly
 * representable in bf16 and hence in binary32, so encoding it by way of a
 * binary32 store is exact. */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    if (isinf(ax))
        return (uint16_t)(sign | 0x7F80);

    int e2;
    frexp(ax, &e2);           /* ax = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;           /* ax in [2^E, 2^(E+1)) */
    int qexp = (E < -126) ? -133 : (E - 7);
    double n = ldexp(ax, -qexp);          /* exact */
    double fl = floor(n);
    double frac = n - fl;                 /* exact */
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double v = ldexp(r, qexp);            /* exact */

    /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    if (v > ldexp(255.0, 120))
        return (uint16_t)(sign | 0x7F80);

    float f = (float)v;                   /* exact: v has <= 8 significant bits */
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(sign | ((w >> 16) & 0x7FFF));
}

/* Elementwise exact decoding of n bf16 bit patterns to fp64 (the decoder the
 * sums use, exported so that it can be checked on every bit pattern). */
void oracle_decode_array(int64_t n, const uint16_t *bits, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode_bf16(bits[i]);
}

/* Elementwise rounding of n fp64 values to bf16 bits. */
void oracle_round_array(int64_t n, const double *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(x[i]);
}

/* Element (k, j) of the right operand.  b_nk == 0: B is K x N row-major with
 * leading dimension ldb (B[k*ldb + j]).  b_nk != 0: B is stored transposed,
 * N x K row-major (Bt[j*ldb + k]). */
static double b_at(const uint16_t *B, int64_t ldb, int b_nk, int64_t k, int64_t j)
{
    return b_nk ? decode_bf16(B[j * ldb + k]) : decode_bf16(B[k * ldb + j]);
}

/* Sum for one row i of C, kept in fp64: acc[j] = sum_k a(i,k) b(k,j), summed
 * in increasing k from +0.0.  For B stored N x K the natural order is j then
 * k; for B stored K x N it is k then j with a row of accumulators, so that B
 * is walked along its rows.  Each acc[j] sees the same terms in the same
 * order either way, so the two loop orders give bit-identical sums. */
static void row_f64(int64_t i, int64_t N, int64_t K,
                    const uint16_t *A, int64_t lda,
                    const uint16_t *B, int64_t ldb, int b_nk, double *acc)
{
    for (int64_t j = 0; j < N; ++j)
        acc[j] = 0.0;
    if (b_nk) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += decode_bf16(A[i * lda + k]) * b_at(B, ldb, 1, k, j);
            acc[j] = s;
        }
    } else {
        for (int64_t k = 0; k < K; ++k) {
            double a = decode_bf16(A[i * lda + k]);
            for (int64_t j = 0; j < N; ++j)
                acc[j] += a * b_at(B, ldb, 0, k, j);
        }
    }
}

/* fp64 product without the final rounding: Cf[i*ldc + j] = sum_k a(i,k) b(k,j).
 * Rows of C are independent, so they are shared among threads.  Returns 0, or
 * -1 if the row buffer could not be allocated. */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const uint16_t *A, int64_t lda,
                    const uint16_t *B, int64_t ldb, int b_nk,
                    double *Cf, int64_t ldc)
{
    int64_t i;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        double *acc = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        row_f64(i, N, K, A, lda, B, ldb, b_nk, acc);
        for (int64_t j = 0; j < N; ++j)
            Cf[i * ldc + j] = acc[j];
        free(acc);
    }
    return fail ? -1 : 0;
}

/* The oracle proper: the fp64 sum of each element, rounded once to bf16.
 * Returns 0, or -1 if a row buffer could not be allocated. */
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda,
                     const uint16_t *B, int64_t ldb, int b_nk,
                     uint16_t *C, int64_t ldc)
{
    int64_t i;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        double *acc = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        row_f64(i, N, K, A, lda, B, ldb, b_nk, acc);
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = oracle_f64_to_bf16(acc[j]);
        free(acc);
    }
    return fail ? -1 : 0;
}

/* Number of threads an OpenMP parallel region here would use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
