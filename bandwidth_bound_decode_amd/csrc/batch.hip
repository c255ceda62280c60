// batch.hip - skinny-batch GEMV (2 <= M <= 16) with X staged in LDS.
//
// At M > 1 every weight vector a lane loads is multiplied by M input vectors. Loading those
// from L2 per wave, as the general kernel does, moves M / R bytes of X per byte of W through
// the vector-memory path; on MI355X that made the time grow by ~2.3 us per extra vector.
// Here a workgroup stages X once per chunk of U wave steps into LDS and its waves read it
// from there:
//   - WAVES compute waves stream W, R rows each, in bursts of U wave steps, and issue the
//     next burst's loads before they use the current one (the next burst is in flight
//     across the per-chunk barrier);
//   - one more wave keeps X staged B - 1 chunks ahead in a ring of B LDS buffers, with
//     direct global-to-LDS loads. Compute waves issue no such loads, so their LDS reads wait
//     on nothing but LDS;
//   - one workgroup barrier per chunk: chunk c is staged, and every compute wave is done
//     with chunk c - 1, whose buffer the staging wave then refills.
// Each (row, m) output is summed in the same per-lane order as the batch-1 kernels (vectors
// in K order, then the same DPP tree), so batch row m is bitwise equal to a batch-1 call on
// X[m]. Measured cost that remains: the dot products themselves, ~0.75 us per extra vector
// at 4096 x 14336 (VALU-bound beyond M ~ 8).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt operand for vmcnt(v), 0 <= v <= 63, with export and LDS/scalar counts at their
// maxima.
constexpr int vmcnt_only(int v) { return 0xF70 | (v & 0xF) | ((v >> 4) << 14); }

template <int M, int R, int U, int WAVES, int B>
__global__ void __launch_bounds__(64 * (WAVES + 1))
    gemv_batch(const uint16_t *w, const uint16_t *x, float *y, int n, int k, int ldw, int ldx,
               int ldy)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    constexpr int kItems = M * U;                    // 1 KiB wave steps of X per chunk
    constexpr int kChunk = kItems * 1024;
    static_assert((B - 2) * kItems <= 63, "staging lead exceeds the vmcnt range");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int chunks = k / (kWaveStep * U);

    if (wave == WAVES) {                             // the staging wave
        // Chunk c into buffer c % B; past the last chunk it stages the last one again, into
        // a buffer nobody reads any more, so every round issues the same number of loads.
        auto stage = [&](int c) {
            const int cc = min(c, chunks - 1);
            unsigned char *dst = lds + (c % B) * kChunk;
#pragma unroll
            for (int i = 0; i < kItems; ++i) {
                const int m = i / U, u = i - (i / U) * U;
                __builtin_amdgcn_global_load_lds(
                    (global_void *)(x + (int64_t)m * ldx + kWaveStep * (cc * U + u) + kVecElems * lane),
                    (lds_void *)(dst + i * 1024), 16, 0, 0);
            }
        };
#pragma unroll
        for (int c = 0; c < B - 1; ++c)
            stage(c);
        for (int c = 0; c < chunks; ++c) {
            __builtin_amdgcn_s_waitcnt(vmcnt_only((B - 2) * kItems));   // chunk c has landed
            __builtin_amdgcn_s_barrier();            // ...and everyone is done with chunk c-1
            stage(c + B - 1);                        // into chunk c-1's buffer
        }
        return;
    }

    const int row0 = (blockIdx.x * WAVES + wave) * R;
    const uint16_t *wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)   // rows past N re-read row N-1; their sums are discarded
        wr[r] = w + (int64_t)min(row0 + r, n - 1) * ldw + kVecElems * lane;
    u32x4 wb[2][U][R];
    // Past the last chunk the loads read X (cached), keeping the number of loads per round
    // static so that the compiler's wait counts stay those of a full pipeline.
    auto issue = [&](int buf, int c) {
        const bool real = c < chunks;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                wb[buf][u][r] = load_stream(real ? wr[r] + kWaveStep * (c * U + u)
                                                 : x + kVecElems * lane);
    };
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[r][m] = 0.f;
    issue(0, 0);
    for (int c0 = 0;; c0 += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = c0 + h;
            if (c < chunks) {
                __builtin_amdgcn_s_barrier();        // chunk c staged
                issue(h ^ 1, c + 1);
                __builtin_amdgcn_sched_barrier(0);   // the next burst goes out before any wait
                const u32x4 *xs = reinterpret_cast<const u32x4 *>(lds + (c % B) * kChunk) + lane;
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const u32x4 xv = xs[kWaveLanes * (m * U + u)];
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r][m] = dot8(wb[h][u][r], xv, acc[r][m]);
                    }
            }
        }
        if (c0 + 2 >= chunks)
            break;
    }
    float out = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float s = lane63(wave_sum(acc[r][m]));
            if (lane == r * M + m)
                out = s;
        }
    if (lane < R * M) {
        const int r = lane / M, m = lane - (lane / M) * M;
        if (row0 + r < n)
            y[(int64_t)m * ldy + row0 + r] = out;
    }
}

// Ring depth per (M, U): as deep as the vmcnt range and ~96 KiB of LDS allow.
constexpr int ring_for(int m, int u) { return (2 * m * u <= 63 && 4 * m * u <= 64) ? 4 : 3; }

template <int M, int R, int U, int WAVES>
constexpr const void *kernel_of()
{
    return reinterpret_cast<const void *>(&gemv_batch<M, R, U, WAVES, ring_for(M, U)>);
}

struct BatchKernel {
    int r, u, waves;
    const void *fn;
    int ring;
};

// The compiled tiles, one per M; the plan picks the same (R, U, waves) (plan.cpp).
const BatchKernel *batch_kernel(int m)
{
#define BBD_BATCH(M, R, U, W) {R, U, W, kernel_of<M, R, U, W>(), ring_for(M, U)}
    static const BatchKernel table[] = {
        BBD_BATCH(2, 1, 4, 8),  BBD_BATCH(3, 2, 2, 4),  BBD_BATCH(4, 2, 2, 4),
        BBD_BATCH(5, 2, 2, 4),  BBD_BATCH(6, 2, 2, 4),  BBD_BATCH(7, 2, 2, 4),
        BBD_BATCH(8, 2, 2, 4),  BBD_BATCH(9, 2, 1, 8),  BBD_BATCH(10, 2, 1, 8),
        BBD_BATCH(11, 2, 1, 8), BBD_BATCH(12, 2, 1, 8), BBD_BATCH(13, 2, 1, 8),
        BBD_BATCH(14, 2, 1, 8), BBD_BATCH(15, 2, 1, 8), BBD_BATCH(16, 2, 1, 8),
    };
#undef BBD_BATCH
    return m >= 2 && m <= 16 ? &table[m - 2] : nullptr;
}

}  // namespace

namespace bbd {

// Launch a validated call on the LDS-staged batch kernel if it qualifies: 2 <= M <= 16, no
// split, one weight matrix, the plan's tile being the compiled one for this M, K a whole
// number of chunks, W and X 16-byte aligned with ldw and ldx multiples of 8. *done is false
// (and nothing is launched) otherwise.
gemv_status launch_batch(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                         int64_t ldx, void *stream, bool *done)
{
    *done = false;
    const BatchKernel *bk = batch_kernel(p->m);
    if (!bk || nseg != 1 || p->splits != 1 || p->rows_per_wave != bk->r ||
        p->unroll != bk->u || p->waves_per_block != bk->waves ||
        p->k % ((int64_t)kWaveStep * bk->u) != 0 || ((uintptr_t)X & 15u) || ldx % 8 != 0 ||
        ((uintptr_t)segs[0].W & 15u) || segs[0].ldw % 8 != 0)
        return GEMV_OK;
    const size_t lds = (size_t)bk->ring * p->m * bk->u * 1024;
    // Allow the kernel more than the default dynamic LDS, once per kernel.
    static std::atomic<bool> allowed[GEMV_MAX_M + 1];
    hipError_t e = hipSuccess;
    if (!allowed[p->m].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(bk->fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return record_hip_error((int)e, GEMV_ERR_DEVICE);
        allowed[p->m].store(true, std::memory_order_release);
    }
    *done = true;
    const uint16_t *w = static_cast<const uint16_t *>(segs[0].W);
    const uint16_t *x = static_cast<const uint16_t *>(X);
    float *y = segs[0].Y;
    int n = (int)p->n, k = (int)p->k, ldw = (int)segs[0].ldw, ldxi = (int)ldx,
        ldy = (int)segs[0].ldy;
    void *args[] = {&w, &x, &y, &n, &k, &ldw, &ldxi, &ldy};
    e = hipLaunchKernel(bk->fn, dim3((unsigned)p->grid_x), dim3(kWaveLanes * (bk->waves + 1)),
                        args, lds, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
