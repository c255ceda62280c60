// norm.hip - batch-1 GEMV with the RMSNorm of its input fused in front.
//
// At decode batch 1 a normalisation moves trivial bytes and costs its launch (GPU performance
// chains page, "Fused RMSNorm traffic"); the projections that consume the normalised vector
// (QKV, gate_up) can compute it themselves. Operation: y = rms_inv * W . (gamma * h) with
// rms_inv = 1 / sqrt(mean(h^2) + eps) and no rounding between the norm and the GEMV.
//
// A workgroup of WAVES waves takes blocks of WAVES consecutive rows (one per wave) and first
// builds the normalised input's numerator u = gamma * h in LDS. u is exact in fp32 (two 8-bit
// significands) but not a bf16 value, so it is stored as the exact sum of two bf16 values,
// u = hi + lo (hi the bf16 rounding of u, lo = u - hi, which fits in 8 significant bits);
// the main loop then multiplies each 16-byte weight vector by both halves with
// v_dot2c_f32_bf16 into two accumulator chains (all products exact), added once per lane
// at the end. The workgroup also sums h^2 (dot2 of h with itself in per-thread chains, the
// DPP tree per wave, the waves in order) and takes
// rms_inv = 1 / sqrt(sum / K + eps) with IEEE fp32 operations; every workgroup does the
// same arithmetic on the same data, so every row sees the same rms_inv. The row's dot
// product is then scaled by it once.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

struct NormArgs {
    const uint16_t *h;
    const uint16_t *gamma;
    int k;                      // a multiple of 8
    int ldw;                    // shared by every segment
    float eps;
    int rows;                   // total rows over the segments
    int row0[GEMV_MAX_SEGMENTS];   // first global row of each segment (INT32_MAX when unused)
    const uint16_t *w[GEMV_MAX_SEGMENTS];
    float *y[GEMV_MAX_SEGMENTS];
};

// bf16 bits of the round-to-nearest-even of a finite float.
__device__ __forceinline__ unsigned bf16_rne(float f)
{
    const unsigned b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Elements 2i, 2i+1 of a packed bf16 vector as floats.
__device__ __forceinline__ float lo_half(unsigned d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float hi_half(unsigned d) { return __uint_as_float(d & 0xFFFF0000u); }

struct NormRow {
    const uint16_t *w;
    float *y;
};

// The weight row of global row `row` (clamped onto the last row) and its output slot.
// Segments are in row order, so segment j = d1 + d2 + d3 with d_i = (row >= row0[i]); the
// pointers are segment 0's plus the sum of d_i times the step to segment i (arithmetic, not
// a select chain, which would move the arguments to scratch).
__device__ __forceinline__ NormRow norm_row(const NormArgs &a, int row)
{
    const int rr = min(row, a.rows - 1);
    const int64_t d1 = rr >= a.row0[1], d2 = rr >= a.row0[2], d3 = rr >= a.row0[3];
    const int64_t w0 = (int64_t)a.w[0], y0 = (int64_t)a.y[0];
    const int64_t dw = d1 * ((int64_t)a.w[1] - w0) + d2 * ((int64_t)a.w[2] - (int64_t)a.w[1]) +
                       d3 * ((int64_t)a.w[3] - (int64_t)a.w[2]);
    const int64_t dy = d1 * ((int64_t)a.y[1] - y0) + d2 * ((int64_t)a.y[2] - (int64_t)a.y[1]) +
                       d3 * ((int64_t)a.y[3] - (int64_t)a.y[2]);
    const int local = rr - (int)(d1 * (a.row0[1] - a.row0[0]) + d2 * (a.row0[2] - a.row0[1]) +
                                 d3 * (a.row0[3] - a.row0[2]));
    return {a.w[0] + dw / (int64_t)sizeof(uint16_t) + (int64_t)local * a.ldw,
            a.y[0] + dy / (int64_t)sizeof(float) + local};
}

template <int U>
__device__ __forceinline__ void norm_burst(const uint16_t *wr, int s0, int vecs, int lane,
                                           u32x4 (&wv)[U])
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        wv[u] = load_stream(wr + kVecElems * min(s0 + lane + kWaveLanes * u, vecs - 1));
}

// Workgroups take row blocks (one row per wave) blockIdx.x, blockIdx.x + gridDim.x, ...,
// so the staging is paid once per workgroup; the first burst of the first row is issued
// before the staging, so its latency and the staging's overlap.
template <int U>
__global__ void __launch_bounds__(512) gemv_rmsnorm(NormArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int vecs = a.k / kVecElems;
    u32x4 *uhi = reinterpret_cast<u32x4 *>(lds);
    u32x4 *ulo = uhi + vecs;
    float *partials = reinterpret_cast<float *>(ulo + vecs);   // one per wave
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int waves = (int)(blockDim.x >> 6);
    const int blocks = (a.rows + waves - 1) / waves;

    int blk = blockIdx.x;
    NormRow nr = norm_row(a, blk * waves + wave);
    u32x4 wv[U];
    // Vector loads retire in order. When every thread stages exactly one vector (the decode
    // shapes), its h and gamma loads go out before the first weight burst, so the staging
    // waits for them only; otherwise the burst goes first.
    const bool one = vecs == (int)blockDim.x;
    u32x4 h0 = {0, 0, 0, 0}, g0 = {0, 0, 0, 0};
    if (one) {
        h0 = load_cached(a.h + kVecElems * (int)threadIdx.x);
        g0 = load_cached(a.gamma + kVecElems * (int)threadIdx.x);
    }
    norm_burst<U>(nr.w, 0, vecs, lane, wv);

    // u = gamma * h as hi + lo in LDS, and this thread's share of sum h^2.
    float sq = 0.f;
    auto stage = [&](int v, u32x4 hv, u32x4 gv) {
        const unsigned hd[4] = {hv.x, hv.y, hv.z, hv.w};
        const unsigned gd[4] = {gv.x, gv.y, gv.z, gv.w};
        unsigned hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float u0 = lo_half(hd[i]) * lo_half(gd[i]);   // exact
            const float u1 = hi_half(hd[i]) * hi_half(gd[i]);
            sq = dot2(hd[i], hd[i], sq);
            const unsigned b0 = bf16_rne(u0), b1 = bf16_rne(u1);
            const unsigned r0 = bf16_rne(u0 - __uint_as_float(b0 << 16));   // exact
            const unsigned r1 = bf16_rne(u1 - __uint_as_float(b1 << 16));
            hi[i] = b0 | (b1 << 16);
            lo[i] = r0 | (r1 << 16);
        }
        uhi[v] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        ulo[v] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    };
    // The one-vector case in a block of its own: inside the general loop the compiler waits
    // for every outstanding load (the weight burst too) before the first vector.
    if (one) {
        stage((int)threadIdx.x, h0, g0);
    } else {
        for (int v = (int)threadIdx.x; v < vecs; v += (int)blockDim.x)
            stage(v, load_cached(a.h + kVecElems * v), load_cached(a.gamma + kVecElems * v));
    }
    const float wsq = lane63(wave_sum(sq));
    if (lane == 0)
        partials[wave] = wsq;
    __syncthreads();
    float total = partials[0];
    for (int i = 1; i < waves; ++i)
        total += partials[i];
    const float rms_inv = 1.0f / sqrtf(total / (float)a.k + a.eps);

    for (;;) {
        // The products with hi and with lo go to separate chains, added once per lane.
        float acc_hi = 0.f, acc_lo = 0.f;
        for (int s0 = 0; s0 < vecs; s0 += kWaveLanes * U) {
            if (s0 > 0)
                norm_burst<U>(nr.w, s0, vecs, lane, wv);
            __builtin_amdgcn_sched_barrier(0);   // the burst's loads before the first use
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = s0 + lane + kWaveLanes * u;
                const int vc = min(v, vecs - 1);
                const float nh = dot8(wv[u], uhi[vc], acc_hi);
                const float nl = dot8(wv[u], ulo[vc], acc_lo);
                acc_hi = v < vecs ? nh : acc_hi;
                acc_lo = v < vecs ? nl : acc_lo;
            }
        }
        const float sum = lane63(wave_sum(acc_hi + acc_lo));
        if (lane == 0 && blk * waves + wave < a.rows)
            *nr.y = rms_inv * sum;
        blk += gridDim.x;
        if (blk >= blocks)
            break;
        nr = norm_row(a, blk * waves + wave);
        norm_burst<U>(nr.w, 0, vecs, lane, wv);
    }
}

const void *find_rmsnorm(int u)
{
    switch (u) {
    case 1: return reinterpret_cast<const void *>(&gemv_rmsnorm<1>);
    case 2: return reinterpret_cast<const void *>(&gemv_rmsnorm<2>);
    case 4: return reinterpret_cast<const void *>(&gemv_rmsnorm<4>);
    case 8: return reinterpret_cast<const void *>(&gemv_rmsnorm<8>);
    default: return nullptr;
    }
}

}  // namespace

namespace bbd {

gemv_status launch_rmsnorm(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *H,
                           const void *gamma, float eps, void *stream)
{
    const void *fn = find_rmsnorm(p->unroll);
    if (!fn)
        return GEMV_ERR_INVALID_ARG;
    NormArgs a;
    a.h = static_cast<const uint16_t *>(H);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.k = (int)p->k;
    a.ldw = (int)segs[0].ldw;
    a.eps = eps;
    a.rows = (int)p->n;
    int64_t row0 = 0;
    for (int i = 0; i < GEMV_MAX_SEGMENTS; ++i) {
        if (i < nseg) {
            a.row0[i] = (int)row0;
            a.w[i] = static_cast<const uint16_t *>(segs[i].W);
            a.y[i] = segs[i].Y;
            row0 += segs[i].n;
        } else {
            a.row0[i] = INT32_MAX;   // never selected
            a.w[i] = a.w[0];
            a.y[i] = a.y[0];
        }
    }
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p->grid_x), dim3((unsigned)p->block_threads),
                                   args, (size_t)p->lds_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
