/*
 * gemv_oracle.c - plain CPU reference for the decode GEMV  y[m][n] = sum_k W[n][k] * X[m][k].
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the bench's
 * CPU-baseline leg load this library. The product path never calls it, links it or shares
 * any source, header or helper with it.
 *
 * What it computes (the definition, written out):
 *   - The operation is the batch-1 (or skinny-batch) GEMV of the decode-GEMV page
 *     ("Decode GEMV at half of HBM bandwidth", inferenceinterviews.com): a row-major
 *     [N, K] bf16 weight times a bf16 vector, one output per row, the reduction running
 *     along each contiguous row ("A strong answer", the split-K kernel and the note after
 *     it; the GPU performance chains page, "A coalesced warp load").
 *   - Inputs are widened before the multiply, as the tiled-GEMM page prescribes for bf16
 *     inputs ("What interviewers probe next", the bf16-with-fp32-accumulation question).
 *     Here the widening goes to fp64 instead of fp32, so that the reference carries no
 *     fp32 summation error of its own.
 *   - A bf16 value is the upper half of a binary32: its 16 bits shifted left by 16 and
 *     reinterpreted. That conversion is exact, and so is the widening to fp64.
 *   - The product of two bf16 values has at most 16 significant bits and an exponent in
 *     [-266, 255], so every product is exact in fp64. The only rounding is the fp64
 *     summation, done in plain k-ascending order.
 *   - Next to each output it returns s_abs = sum_k |W[n][k] * X[m][k]|, the magnitude the
 *     parity tolerance is scaled by.
 *
 * Rows may be processed by several OpenMP threads; each output's sum is still one thread's
 * k-ascending loop, so the result does not depend on the thread count.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: the summation order must stay as
 * written).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* The number of threads a call with `nthreads` uses (1 when built without OpenMP). */
int oracle_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Decode `count` bf16 bit patterns to their exact fp64 values. */
void oracle_bf16_to_f64(const uint16_t *bits, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = bf16_value(bits[i]);
}

/*
 * W:  bf16 bits, row n at W + n*ldw, elements k = 0..K-1 (ldw >= K).
 * X:  bf16 bits, vector m at X + m*ldx (ldx >= K).
 * Y:  fp64 [M][N] dense, Y[m*N + n] = sum_k W[n][k] * X[m][k].
 * S:  fp64 [M][N] dense, S[m*N + n] = sum_k |W[n][k] * X[m][k]|.
 * nthreads <= 0 lets the OpenMP runtime choose.
 * Returns 0, or -1 for a bad argument (nothing written).
 */
int oracle_gemv_f64(const uint16_t *W, int64_t N, int64_t K, int64_t ldw,
                    const uint16_t *X, int64_t M, int64_t ldx,
                    double *Y, double *S, int nthreads)
{
    if (!W || !X || !Y || !S || N < 0 || K < 0 || M < 0 || ldw < K || ldx < K)
        return -1;
    int64_t total = M * N;
    int threads = oracle_threads(nthreads);
    (void)threads;
#pragma omp parallel for schedule(static) num_threads(threads)
    for (int64_t t = 0; t < total; ++t) {
        int64_t m = t / N;
        int64_t n = t % N;
        const uint16_t *w = W + n * ldw;
        const uint16_t *x = X + m * ldx;
        double sum = 0.0;
        double mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = bf16_value(w[k]) * bf16_value(x[k]);
            sum += p;
            mag += fabs(p);
        }
        Y[m * N + n] = sum;
        S[m * N + n] = mag;
    }
    return 0;
}
