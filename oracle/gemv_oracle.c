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

/*
 * INT4 weights. The decode-GEMV page's follow-up turns the weights into INT4: a quarter of
 * the bytes, unpacked in registers while the next loads are in flight. It fixes no storage
 * format; the one this oracle defines (and the GPU path reads):
 *   - a weight is a signed 4-bit integer v in [-8, 7], stored as a two's-complement nibble;
 *   - row n of the packed matrix starts at Wq + n*ldq (bytes); element k is the low nibble
 *     of byte k/2 when k is even and the high nibble when k is odd (so the 32-bit word
 *     holding elements 8j..8j+7 has element 8j+i in bits 4i..4i+3);
 *   - each run of 128 consecutive elements of a row (group k/128) shares one bf16 scale,
 *     scale[n][g] at Sc + n*lds + g;
 *   - the weight's value is v * scale.
 * v has 4 significant bits and the scale 8, so the weight and its product with a bf16 x
 * are exact in fp64; the only rounding is again the k-ascending fp64 summation.
 */
#define ORACLE_Q4_GROUP 128

static double q4_weight(const uint8_t *row, const uint16_t *scales, int64_t j)
{
    int nibble = (j & 1) ? (row[j >> 1] >> 4) : (row[j >> 1] & 0x0F);
    int v = nibble >= 8 ? nibble - 16 : nibble;
    return (double)v * bf16_value(scales[j / ORACLE_Q4_GROUP]);
}

/* Dequantize an [N][K] INT4 matrix into fp64 out[n*K + j]. Returns 0, or -1. */
int oracle_q4_dequant_f64(const uint8_t *Wq, int64_t N, int64_t K, int64_t ldq,
                          const uint16_t *Sc, int64_t lds, double *out)
{
    if (!Wq || !Sc || !out || N < 0 || K < 0 || ldq < (K + 1) / 2 ||
        lds < (K + ORACLE_Q4_GROUP - 1) / ORACLE_Q4_GROUP)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K; ++j)
            out[n * K + j] = q4_weight(Wq + n * ldq, Sc + n * lds, j);
    return 0;
}

/*
 * Y[m*N + n] = sum_j w_nj * X[m][j] with w from the INT4 format above, and
 * Sabs[m*N + n] = sum_j |w_nj * X[m][j]|. X as for oracle_gemv_f64. Returns 0, or -1.
 */
int oracle_gemv_q4_f64(const uint8_t *Wq, int64_t N, int64_t K, int64_t ldq,
                       const uint16_t *Sc, int64_t lds, const uint16_t *X, int64_t M,
                       int64_t ldx, double *Y, double *Sabs, int nthreads)
{
    if (!Wq || !Sc || !X || !Y || !Sabs || N < 0 || K < 0 || M < 0 || ldq < (K + 1) / 2 ||
        lds < (K + ORACLE_Q4_GROUP - 1) / ORACLE_Q4_GROUP || ldx < K)
        return -1;
    int threads = oracle_threads(nthreads);
    (void)threads;
#pragma omp parallel for schedule(static) num_threads(threads)
    for (int64_t t = 0; t < M * N; ++t) {
        const int64_t vec = t / N, row = t % N;
        const uint8_t *packed = Wq + row * ldq;
        const uint16_t *scales = Sc + row * lds;
        const uint16_t *xv = X + vec * ldx;
        double total = 0.0, magnitude = 0.0;
        for (int64_t j = 0; j < K; j++) {
            const double term = q4_weight(packed, scales, j) * bf16_value(xv[j]);
            total += term;
            magnitude += fabs(term);
        }
        Y[vec * N + row] = total;
        Sabs[vec * N + row] = magnitude;
    }
    return 0;
}

/*
 * RMSNorm prologue. The GPU performance chains page ("Fused RMSNorm traffic") notes that at
 * decode batch 1 a normalisation moves trivial bytes and costs its launches; fused into the
 * projection that consumes it (QKV, gate_up), those launches disappear. The pages do not
 * write the normalisation out; this is the usual RMSNorm (mean of squares plus eps, inverse
 * square root, per-element gain gamma) followed by the GEMV, with no rounding in between:
 *   rms_inv = 1 / sqrt( (1/K) * sum_k h_k^2 + eps )
 *   y[n]    = rms_inv * sum_k W[n][k] * (gamma_k * h_k)
 * with h (the residual-stream vector), gamma and W in bf16 and eps >= 0. The products
 * h_k^2 and W*gamma*h are exact in fp64 (at most 24 significant bits); the sums run in
 * k-ascending order; the square root and the divisions are IEEE fp64. Sabs holds
 * rms_inv * sum_k |W[n][k] * gamma_k * h_k|, the magnitude the tolerance scales with.
 * Returns 0, or -1 for a bad argument.
 */
int oracle_gemv_rmsnorm_f64(const uint16_t *W, int64_t N, int64_t K, int64_t ldw,
                            const uint16_t *H, const uint16_t *G, double eps,
                            double *Y, double *Sabs, int nthreads)
{
    if (!W || !H || !G || !Y || !Sabs || N < 0 || K < 1 || ldw < K || !(eps >= 0.0))
        return -1;
    double squares = 0.0;
    for (int64_t i = 0; i < K; i++) {
        const double hv = bf16_value(H[i]);
        squares += hv * hv;
    }
    const double rms_inv = 1.0 / sqrt(squares / (double)K + eps);
    int threads = oracle_threads(nthreads);
    (void)threads;
#pragma omp parallel for schedule(static) num_threads(threads)
    for (int64_t row = 0; row < N; ++row) {
        const uint16_t *wrow = W + row * ldw;
        double dot = 0.0, size = 0.0;
        for (int64_t i = 0; i < K; i++) {
            const double part = bf16_value(wrow[i]) * (bf16_value(G[i]) * bf16_value(H[i]));
            dot += part;
            size += fabs(part);
        }
        Y[row] = rms_inv * dot;
        Sabs[row] = rms_inv * size;
    }
    return 0;
}
