// whole.hip - the lean batch-1 kernels for rows that are a whole number of bursts.
//
// They live in a translation unit of their own, so they are a small code object of their
// own rather than a few kernels among the ~260 of the general path.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

// Waves per SIMD the occupancy hint allows: as many as the registers one burst of U
// single-row loads needs (the general kernel's formula at M = 1, R = 1).
template <int U>
constexpr int whole_waves_per_simd()
{
    return 512 / (4 * U * 2 + 1 + 24) >= 8 ? 8 : 512 / (4 * U * 2 + 1 + 24);
}

// The batch-1 decode shapes (K a multiple of 512 U, one row per wave, no split, one weight
// matrix, 16-byte aligned) run a kernel with nothing else in it: a 32-byte argument block,
// no slice arithmetic, no remainder paths, no output-routing branches. Measured on MI355X it
// is 0.2-0.4 us per launch faster than the general kernel on the same tile (down_proj
// 4096 x 14336: 18.3-18.4 us against 18.8 us). It sums every row in the same order as
// gemv_fast, so the two give bitwise the same result.
template <int U>
__global__ void __launch_bounds__(512)
    __attribute__((amdgpu_waves_per_eu(1, whole_waves_per_simd<U>())))
        gemv_whole(const uint16_t *w, const uint16_t *x, float *y, int n, int k, int ldw)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x;                       // one single-wave workgroup per row
    const int steps = k / kWaveStep;
    const uint16_t *wr = w + (int64_t)min(row, n - 1) * ldw;
    float acc = 0.f;
    for (int s = 0; s < steps; s += U) {
        u32x4 wv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            wv[u] = load_stream(wr + kVecElems * (lane + kWaveLanes * (s + u)));
#pragma unroll
        for (int u = 0; u < U; ++u)
            xv[u] = load_cached(x + kVecElems * (lane + kWaveLanes * (s + u)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc = dot8(wv[u], xv[u], acc);
    }
    const float sum = lane63(wave_sum(acc));
    if (lane == 0 && row < n)
        y[row] = sum;
}

// The fused form (QKV, gate_up): up to four weight matrices with one leading dimension,
// each row's segment picked per wave from values held in scalar registers.
// Field order matters: the scalars come first, next to the segment tables, so that every
// argument arrives in the first batch of scalar loads instead of after the segment selects.
struct WholeMultiArgs {
    const uint16_t *x;
    int32_t ldw;
    int32_t bursts;
    int32_t row0[GEMV_MAX_SEGMENTS];        // first row of each segment; INT32_MAX unused
    const uint16_t *w[GEMV_MAX_SEGMENTS];   // row 0 of each segment (segment 0 repeated)
    float *y[GEMV_MAX_SEGMENTS];
};

template <int U>
__global__ void __launch_bounds__(512)
    __attribute__((amdgpu_waves_per_eu(1, whole_waves_per_simd<U>())))
        gemv_whole_multi(WholeMultiArgs a)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x;
    // Segments are in row order, so segment j = d1 + d2 + d3 with d_i = (row >= row0[i])
    // monotone in i, and each pointer is segment 0's plus the sum of d_i times the step
    // from segment i-1 to segment i. Arithmetic rather than a select chain: no branches,
    // so every argument load stays in the first batch, and no address select (which
    // would move the arguments to scratch). Pointers stay offsets from segment 0's, so
    // they keep the global address space.
    const int64_t d1 = row >= a.row0[1], d2 = row >= a.row0[2], d3 = row >= a.row0[3];
    const int64_t w0 = (int64_t)a.w[0], y0 = (int64_t)a.y[0];
    const int64_t dw = d1 * ((int64_t)a.w[1] - w0) + d2 * ((int64_t)a.w[2] - (int64_t)a.w[1]) +
                       d3 * ((int64_t)a.w[3] - (int64_t)a.w[2]);
    const int64_t dy = d1 * ((int64_t)a.y[1] - y0) + d2 * ((int64_t)a.y[2] - (int64_t)a.y[1]) +
                       d3 * ((int64_t)a.y[3] - (int64_t)a.y[2]);
    const int local = row - (int)(d1 * (a.row0[1] - a.row0[0]) + d2 * (a.row0[2] - a.row0[1]) +
                                  d3 * (a.row0[3] - a.row0[2]));
    const uint16_t *wp = a.w[0] + dw / (int64_t)sizeof(uint16_t) + (int64_t)local * a.ldw +
                         kVecElems * lane;
    float *yp = a.y[0] + dy / (int64_t)sizeof(float) + local;
    const uint16_t *xp = a.x + kVecElems * lane;
    float acc = 0.f;
    // bursts >= 1 (the host guarantees it): a do-while lets every argument load go out in
    // the first batch, instead of a second round trip after a zero-trip test.
    int b = 0;
    do {
        u32x4 wv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            wv[u] = load_stream(wp + kWaveStep * u);
#pragma unroll
        for (int u = 0; u < U; ++u)
            xv[u] = load_cached(xp + kWaveStep * u);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc = dot8(wv[u], xv[u], acc);
        wp += kWaveStep * U;
        xp += kWaveStep * U;
    } while (++b < a.bursts);
    const float sum = lane63(wave_sum(acc));
    if (lane == 0)
        *yp = sum;
}


const void *find_whole(int u, bool multi)
{
    switch (u) {
    case 2: return multi ? reinterpret_cast<const void *>(&gemv_whole_multi<2>)
                         : reinterpret_cast<const void *>(&gemv_whole<2>);
    case 4: return multi ? reinterpret_cast<const void *>(&gemv_whole_multi<4>)
                         : reinterpret_cast<const void *>(&gemv_whole<4>);
    case 8: return multi ? reinterpret_cast<const void *>(&gemv_whole_multi<8>)
                         : reinterpret_cast<const void *>(&gemv_whole<8>);
    default: return nullptr;
    }
}

}  // namespace

namespace bbd {

// Launch a validated call on the whole-row kernels if it qualifies: batch 1, one row per
// single-wave workgroup, no split, K a whole number of bursts, 16-byte aligned W and X
// with ldw a multiple of 8, and one leading dimension for every segment. *done is false
// (and nothing is launched) otherwise.
gemv_status launch_whole(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                         void *stream, bool *done)
{
    *done = false;
    if (p->m != 1 || p->rows_per_wave != 1 || p->waves_per_block != 1 || p->splits != 1 ||
        p->k % ((int64_t)kWaveStep * p->unroll) != 0 || ((uintptr_t)X & 15u))
        return GEMV_OK;
    for (int i = 0; i < nseg; ++i)
        if (((uintptr_t)segs[i].W & 15u) || segs[i].ldw % 8 != 0 || segs[i].ldw != segs[0].ldw)
            return GEMV_OK;
    const void *kernel = find_whole(p->unroll, nseg > 1);
    if (!kernel)
        return GEMV_OK;
    *done = true;
    WholeMultiArgs wm;
    const uint16_t *w1 = static_cast<const uint16_t *>(segs[0].W);
    const uint16_t *x1 = static_cast<const uint16_t *>(X);
    float *y1 = segs[0].Y;
    int n1 = (int)p->n, k1 = (int)p->k, ldw1 = (int)segs[0].ldw;
    void *single_args[] = {&w1, &x1, &y1, &n1, &k1, &ldw1};
    void *multi_args[] = {&wm};
    void **args = single_args;
    const int32_t bursts = (int32_t)(p->k / ((int64_t)kWaveStep * p->unroll));
    if (nseg > 1) {
        args = multi_args;
        int64_t row0 = 0;
        for (int i = 0; i < GEMV_MAX_SEGMENTS; ++i) {
            const int src = i < nseg ? i : 0;
            wm.w[i] = static_cast<const uint16_t *>(segs[src].W);
            wm.y[i] = segs[src].Y;
            wm.row0[i] = i < nseg ? (int32_t)row0 : INT32_MAX;
            if (i < nseg)
                row0 += segs[i].n;
        }
        wm.x = static_cast<const uint16_t *>(X);
        wm.ldw = (int32_t)segs[0].ldw;
        wm.bursts = bursts;
    }
    hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)p->grid_x), dim3(kWaveLanes), args,
                                   (size_t)p->lds_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
