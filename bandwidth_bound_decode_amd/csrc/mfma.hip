// mfma.hip - skinny-batch GEMV on the matrix cores (by default for 8 <= M <= 16).
//
// The VALU kernels multiply every weight vector a lane loads by M input vectors with
// v_dot2 instructions; past M ~ 8 that arithmetic, not HBM, sets the time (about 0.75 us
// per extra vector at 4096 x 14336). Here one v_mfma_f32_16x16x32_bf16 takes 16 weight rows
// (A operand) and 16 input vectors (B operand) over 32 K elements, so the arithmetic per
// weight byte no longer grows with M. Batches below 16 repeat the last vector in the unused
// B columns, whose outputs are never stored.
//
// Operand layout of the 16x16x32 bf16 MFMA on gfx950 (checked on the device against an
// exact integer product): lane l holds A[l % 16][8 (l / 16) .. +8) and B[8 (l / 16) .. +8)
// [l % 16] as 8 packed bf16, and D[4 (l / 16) + e][l % 16] in accumulator register e. Only
// the pairing of A and B elements matters to the sum, so K element 32 u + 8 g + e of a chunk
// goes to lane group g of MFMA u: each 16-byte load then covers 64 contiguous bytes of 16
// rows (of W) or of 16 vectors (of X).
//
// Work split (measured on MI355X at 4096 x 14336, M = 8..16; probe sweep of tiles per wave,
// MFMAs per burst, waves per workgroup and split counts):
//   - a workgroup owns 32 rows (two 16-row tiles, which share every X fragment, halving X
//     traffic against one tile) and one K slice; its 8 waves take the slice's 64-element
//     chunks in turn, starting at a per-workgroup rotation so that workgroups running side
//     by side read different column ranges of their rows;
//   - per chunk a wave loads both tiles' W and the chunk's X (six 16-byte loads per lane)
//     before its four MFMAs; W goes through the cache like X (for this access pattern the
//     streaming hint measured slower);
//   - the 8 waves' partial tiles are summed in LDS in wave order, then stored; a plan that
//     splits K (too few 32-row blocks for the CUs) stores device-coherent partials and the
//     last workgroup of a row block to arrive adds them in slice order, as the VALU
//     kernels' split combine does.
// The order of every sum is fixed, so results are reproducible bit for bit; they differ in
// rounding from the VALU kernels' (a different summation order).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTiles = kMfmaRowsPerBlock / 16;   // 16-row tiles per workgroup
constexpr int kU = kMfmaChunk / 32;              // MFMAs per chunk and tile
constexpr int kThreads = kWaveLanes * kMfmaWaves;

__device__ __forceinline__ floatx4 mfma(u32x4 a, u32x4 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// y[m][row] = sum_k w[row][k] x[m][k] for the 32-row block blockIdx.x and the K slice
// blockIdx.y (of gridDim.y). With one slice the result goes to y; with several, to
// partial[slice][m][row] and then, by the last arrival, to y.
__global__ void __launch_bounds__(kThreads)
    gemv_mfma(const uint16_t *w, const uint16_t *x, float *y, float *partial,
              unsigned *tickets, int n, int k, int ldw, int ldx, int ldy, int m, int slice)
{
    __shared__ floatx4 red[kMfmaWaves - 1][kTiles][kWaveLanes];
    __shared__ unsigned s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int i16 = lane & 15, g = lane >> 4;
    const int splits = gridDim.y, s = blockIdx.y;
    const int row0 = blockIdx.x * kMfmaRowsPerBlock;
    const int k0 = s * slice;
    const int chunks = min(slice, k - k0) / kMfmaChunk;

    const uint16_t *wr[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
        wr[t] = w + (int64_t)min(row0 + 16 * t + i16, n - 1) * ldw + k0 + 8 * g;
    const uint16_t *xr = x + (int64_t)min(i16, m - 1) * ldx + k0 + 8 * g;

    const int turns = (chunks - wave + kMfmaWaves - 1) / kMfmaWaves;
    const int rot = (int)((blockIdx.x * 37u + (unsigned)s * 11u) % (unsigned)chunks);
    floatx4 acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
        acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < turns; ++i) {
        int c = wave + i * kMfmaWaves + rot;
        c = c >= chunks ? c - chunks : c;
        u32x4 a[kTiles][kU], b[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int t = 0; t < kTiles; ++t)
                a[t][u] = load_cached(wr[t] + c * kMfmaChunk + 32 * u);
#pragma unroll
        for (int u = 0; u < kU; ++u)
            b[u] = load_cached(xr + c * kMfmaChunk + 32 * u);
        __builtin_amdgcn_sched_barrier(0);   // every load of the chunk before the first MFMA
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int t = 0; t < kTiles; ++t)
                acc[t] = mfma(a[t][u], b[u], acc[t]);
    }

    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
            red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
#pragma unroll
            for (int v = 0; v < kMfmaWaves - 1; ++v)
                acc[t] += red[v][t][lane];
            const int row = row0 + 16 * t + 4 * g;
            if (i16 < m) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (row + e >= n)
                        continue;
                    if (splits == 1)
                        y[(int64_t)i16 * ldy + row + e] = acc[t][e];
                    else   // device-coherent, for the workgroup that adds the slices up
                        __hip_atomic_store(partial + ((int64_t)s * m + i16) * n + row + e,
                                           acc[t][e], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
    if (splits == 1)
        return;

    // Split combine: every store above has completed before the barrier, and only then
    // is the ticket taken, so the last arrival finds all slices' partials.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned ticket = __hip_atomic_fetch_add(tickets + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        s_last = ticket == (unsigned)splits - 1;
    }
    __syncthreads();
    if (!s_last)
        return;
    const int rows = min(kMfmaRowsPerBlock, n - row0);
    const int64_t plane = (int64_t)m * n;
    for (int t = threadIdx.x; t < rows * m; t += kThreads) {
        const int mi = t / rows;
        const int row = row0 + (t - mi * rows);
        const float *src = partial + (int64_t)mi * n + row;
        float v = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int sl = 1; sl < splits; ++sl)
            v += __hip_atomic_load(src + sl * plane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        y[(int64_t)mi * ldy + row] = v;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(tickets + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

namespace bbd {

gemv_status launch_mfma(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                        int64_t ldx, unsigned *ws_tickets, float *ws_partial, void *stream,
                        bool *done)
{
    *done = false;
    if (!p->mfma || nseg != 1 || ((uintptr_t)X & 15u) || ldx % 8 != 0 ||
        ((uintptr_t)segs[0].W & 15u) || segs[0].ldw % 8 != 0)
        return GEMV_OK;
    *done = true;
    const uint16_t *w = static_cast<const uint16_t *>(segs[0].W);
    const uint16_t *x = static_cast<const uint16_t *>(X);
    float *y = segs[0].Y;
    float *partial = nullptr;
    unsigned *tickets = nullptr;
    if (p->mfma_splits > 1) {
        tickets = ws_tickets;
        partial = ws_partial;
    }
    int n = (int)p->n, k = (int)p->k, ldw = (int)segs[0].ldw, ldxi = (int)ldx,
        ldy = (int)segs[0].ldy, m = p->m, slice = (int)p->mfma_slice;
    void *args[] = {&w, &x, &y, &partial, &tickets, &n, &k, &ldw, &ldxi, &ldy, &m, &slice};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(gemv_mfma),
                                   dim3((unsigned)p->mfma_grid_x, (unsigned)p->mfma_splits),
                                   dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
