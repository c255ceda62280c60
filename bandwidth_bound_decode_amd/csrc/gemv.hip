// gemv.hip - gfx950 (CDNA4) kernels for the decode GEMV and the launching half of the C ABI.
//
// Y[m][n] = sum_k W[n][k] * X[m][k], W row-major bf16, X bf16, fp32 accumulation.
//
// Kernel design (decode-GEMV page, "Decode GEMV at half of HBM bandwidth", "A strong
// answer"; GPU performance chains page, "A coalesced warp load"):
//   - One 64-lane wave owns R output rows over one K slice. Lane l reads the 16-byte
//     vectors l, l+64, l+128, ... of each row, so one wave-wide load instruction covers
//     1 KiB of contiguous row bytes - the wave64 form of "lanes walk along K".
//   - Each lane issues U x R independent 16-byte W loads (nontemporal: W is read once)
//     before it consumes any, which is what keeps enough bytes in flight per CU for
//     Little's law on HBM3E (cause 2 of the section above).
//   - The multiply-add is v_dot2c_f32_bf16: two bf16 products summed into an fp32
//     accumulator per instruction, with no widening step. One accumulator chain per
//     (row, batch) per lane, in vector order, so the summation order depends only on the
//     K slice - not on R, U or M.
//   - A fixed DPP tree reduces the 64 lane partials (quad_perm, row_half_mirror,
//     row_mirror, row_bcast:15, row_bcast:31), then lane 63 holds the row sum.
//   - Split-K (cause 1): blockIdx.y selects the K slice. With more than one slice each
//     wave writes its partial sums to the workspace (pass 1); the workgroup that arrives
//     last for a row block - found with one ticket counter per row block - then adds the S
//     partials of each of its outputs in slice order 0, 1, ..., S-1 (pass 2) and resets
//     the counter. The order is fixed, so the result is bitwise reproducible; no atomic
//     ever touches a sum (the page's follow-up on a result that differs in the last bit
//     between runs). Doing pass 2 inside the same launch saves a kernel launch per GEMV,
//     which on this GPU costs about as much as streaming 30 MB.
// There is no LDS staging of W: a GEMV has no reuse of W (the page's common mistakes).
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <array>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

struct Seg {
    const uint16_t *w;  // row 0 of the segment's weight
    int64_t ldw;
    float *y;           // row 0 of the segment's output
    int64_t ldy;
    int32_t row0;       // first global row of the segment (INT32_MAX when unused)
    int32_t pad;
};

// Kernel arguments of a single-segment launch (every gemv_run). They are kept small - the
// fields an unsplit launch reads fit in one 64-byte line, and no kernel reads the implicit
// dispatch arguments - because on MI355X a launch's start-up grows with the argument bytes
// its waves fetch before the first weight load (measured: ~0.1-0.25 us per launch for a
// 240-byte argument block).
struct Args {
    const uint16_t *w0;     // segment 0 (the only one)
    float *y0;
    const uint16_t *x;
    int32_t ldw0;
    int32_t ldy0;
    int32_t ldx;
    int32_t n;
    int32_t k;
    int32_t slice;
    int32_t waves;          // waves per workgroup
    int32_t rows;           // rows per wave (unaligned kernel)
    float *partial;         // [S][M][N] when the plan splits K, else null
    unsigned *tickets;      // [grid_x] arrival counters, zero between calls (split plans only)
};

// Fused launches (nseg > 1) add every segment, in row order, segment 0 repeated.
struct ArgsMulti : Args {
    Seg seg[GEMV_MAX_SEGMENTS];
};

template <bool MULTI>
using ArgsT = typename std::conditional<MULTI, ArgsMulti, Args>::type;

// Segment holding global row `row`. The single-segment instances (MULTI = false, every
// gemv_run) read only the argument header, so their prologue is one batch of scalar loads
// before the first weight load. Otherwise segments are in row order, unused slots start at
// INT32_MAX, and every field is picked with selects. Works for uniform and per-lane rows.
struct RowRef {
    const uint16_t *w;
    float *y;
    int64_t ldy;
};

// A kernel-argument value known to be the same in every lane, pinned to scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ RowRef locate_multi(const ArgsMulti &p, int row)
{
    // Every field is first read as a uniform value; selecting between struct members
    // directly is folded into an address select, which spills the by-value arguments to
    // scratch and turns every load into a flat load.
    uint64_t w[GEMV_MAX_SEGMENTS], y[GEMV_MAX_SEGMENTS];
    int64_t ldw[GEMV_MAX_SEGMENTS], ldy[GEMV_MAX_SEGMENTS];
    int row0[GEMV_MAX_SEGMENTS];
#pragma unroll
    for (int i = 0; i < GEMV_MAX_SEGMENTS; ++i) {
        w[i] = uniform64((uint64_t)p.seg[i].w);
        y[i] = uniform64((uint64_t)p.seg[i].y);
        ldw[i] = (int64_t)uniform64((uint64_t)p.seg[i].ldw);
        ldy[i] = (int64_t)uniform64((uint64_t)p.seg[i].ldy);
        row0[i] = __builtin_amdgcn_readfirstlane(p.seg[i].row0);
    }
    const int j = (row >= row0[1]) + (row >= row0[2]) + (row >= row0[3]);
    const uint64_t wj = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : w[3];
    const uint64_t yj = j == 0 ? y[0] : j == 1 ? y[1] : j == 2 ? y[2] : y[3];
    const int64_t ldwj = j == 0 ? ldw[0] : j == 1 ? ldw[1] : j == 2 ? ldw[2] : ldw[3];
    const int64_t ldyj = j == 0 ? ldy[0] : j == 1 ? ldy[1] : j == 2 ? ldy[2] : ldy[3];
    const int local = row - (j == 0 ? row0[0] : j == 1 ? row0[1] : j == 2 ? row0[2] : row0[3]);
    // Pointers are rebuilt as offsets from segment 0's pointers so that they keep the
    // global address space (a pointer made from an integer becomes a flat pointer).
    const int64_t dw = (int64_t)(wj - w[0]) / (int64_t)sizeof(uint16_t);
    const int64_t dy = (int64_t)(yj - y[0]) / (int64_t)sizeof(float);
    return {p.seg[0].w + dw + (int64_t)local * ldwj, p.seg[0].y + dy + local, ldyj};
}

template <bool MULTI>
__device__ __forceinline__ RowRef locate(const ArgsT<MULTI> &p, int row)
{
    if constexpr (!MULTI)
        return {p.w0 + (int64_t)row * p.ldw0, p.y0 + row, p.ldy0};
    else
        return locate_multi(p, row);
}

// Reduce R x M lane partials, then lane (r * M + m) stores output (row_first + r, m).
template <int M, int R, bool MULTI>
__device__ __forceinline__ void finish(const ArgsT<MULTI> &p, float (&acc)[R][M], int row_first,
                                       int split, int lane)
{
    float out = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float s = lane63(wave_sum(acc[r][m]));
            if (lane == r * M + m)
                out = s;
        }
    }
    if (lane < R * M) {
        int r = lane / M;
        int m = lane - r * M;
        int row = row_first + r;
        if (row < p.n) {
            if (p.partial) {
                // Agent-scope store: coherent across the XCDs' separate L2 caches, so the
                // workgroup that adds the partials up can read it from any XCD.
                __hip_atomic_store(p.partial + ((int64_t)split * M + m) * p.n + row, out,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                RowRef ref = locate<MULTI>(p, row);
                ref.y[(int64_t)m * ref.ldy] = out;
            }
        }
    }
}

// Pass 2 of split-K, run by the whole workgroup after its waves stored their partials.
// The last of the S workgroups of row block blockIdx.x to arrive sums the partials of the
// block's rows in slice order and leaves the ticket at zero for the next call.
//
// Ordering without cache maintenance: partials are written and read with agent-scope
// (device-coherent) stores and loads, every wave waits until its stores have completed
// before the workgroup barrier, and only then does one lane take the ticket. A workgroup
// that draws the last ticket therefore finds every other slice's partials in coherent
// memory. L2 write-back / invalidate fences are avoided on purpose: issued per workgroup
// they cost more than the whole GEMV.
template <bool MULTI>
__device__ __forceinline__ void combine_if_last(const ArgsT<MULTI> &p, int m_count,
                                                int rows_per_block)
{
    __shared__ unsigned s_last;
    __builtin_amdgcn_s_waitcnt(0);      // this wave's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned ticket = __hip_atomic_fetch_add(p.tickets + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        s_last = ticket == gridDim.y - 1;
    }
    __syncthreads();
    if (!s_last)
        return;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows = min(rows_per_block, p.n - row0);
    const int64_t plane = (int64_t)m_count * p.n;   // one slice's partials
    for (int t = threadIdx.x; t < rows * m_count; t += p.waves * kWaveLanes) {
        const int m = t / rows;
        const int row = row0 + (t - m * rows);
        const float *src = p.partial + (int64_t)m * p.n + row;
        float v = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (unsigned sl = 1; sl < gridDim.y; ++sl)
            v += __hip_atomic_load(src + sl * plane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        RowRef ref = locate<MULTI>(p, row);
        ref.y[(int64_t)m * ref.ldy] = v;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(p.tickets + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------- fast path
// VGPRs a fast-path wave needs to hold every load of one unrolled step at once, plus
// accumulators and addressing; the occupancy hint below lets the compiler use that many
// instead of interleaving waits into the load burst to stay at 8 waves per SIMD.
template <int M, int R, int U>
constexpr int fast_vgprs()
{
    return 4 * U * (R + M) + R * M + 24;
}

template <int M, int R, int U>
constexpr int fast_waves_per_simd()
{
    return 512 / fast_vgprs<M, R, U>() >= 8 ? 8 : 512 / fast_vgprs<M, R, U>();
}

// One wave's R rows over its K slice (split = blockIdx.y).
template <int M, int R, int U, bool MULTI>
__device__ __forceinline__ void fast_rows(const ArgsT<MULTI> &p, int row_first, int lane)
{
    const int split = blockIdx.y;
    const int k0 = split * p.slice;
    const int len = min(p.k - k0, p.slice);
    const int nvec = len >> 3;
    const int rem = len & 7;
    const int full = nvec >> 6;   // steps in which every lane has a vector

    const uint16_t *wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        // Rows past N (last wave of the grid) re-read row N-1; their sums are discarded.
        int row = min(row_first + r, p.n - 1);
        wrow[r] = locate<MULTI>(p, row).w + k0;
    }
    const uint16_t *xk = p.x + k0;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[r][m] = 0.f;

    int step = 0;
    for (; step + U <= full; step += U) {
        u32x4 wv[U][R];
        u32x4 xv[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[u][r] = load_stream(wrow[r] + 8 * (lane + 64 * (step + u)));
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < M; ++m)
                xv[u][m] = load_cached(xk + (int64_t)m * p.ldx + 8 * (lane + 64 * (step + u)));
        // Keep the whole burst of loads ahead of the first use: without this the
        // scheduler interleaves waits into it to save registers, cutting loads in flight.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[r][m] = dot8(wv[u][r], xv[u][m], acc[r][m]);
    }
    if (__builtin_expect(step < full, 0)) {
        // Fewer than U full steps left: issue them as one burst too (wave-uniform
        // predicates), so the remainder costs one memory latency, not one per step.
        const int rest = full - step;
        u32x4 wv[U][R];
        u32x4 xv[U][M];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < rest)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    wv[u][r] = load_stream(wrow[r] + 8 * (lane + 64 * (step + u)));
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < rest)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    xv[u][m] = load_cached(xk + (int64_t)m * p.ldx + 8 * (lane + 64 * (step + u)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < rest)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc[r][m] = dot8(wv[u][r], xv[u][m], acc[r][m]);
    }
    // Last, partial wave step: only lanes whose vector lies inside the slice.
    const int v_last = lane + 64 * full;
    if (__builtin_expect(v_last < nvec, 0)) {
        u32x4 wv[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            wv[r] = load_stream(wrow[r] + 8 * v_last);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            u32x4 xv = load_cached(xk + (int64_t)m * p.ldx + 8 * v_last);
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r][m] = dot8(wv[r], xv, acc[r][m]);
        }
    }
    // Ragged tail of fewer than 8 elements (only the final slice can have one).
    if (__builtin_expect(lane < rem, 0)) {
        const int kk = 8 * nvec + lane;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float w = bf16_to_f32(wrow[r][kk]);
#pragma unroll
            for (int m = 0; m < M; ++m)
                acc[r][m] = fmaf(w, bf16_to_f32(xk[(int64_t)m * p.ldx + kk]), acc[r][m]);
        }
    }
    finish<M, R, MULTI>(p, acc, row_first, split, lane);
}

// W and X 16-byte aligned with leading dimensions that are multiples of 8. Only the SPLIT
// instances contain the combine (and its LDS flag and barriers); every wave, including one
// past N in the last workgroup, reaches it.
template <int M, int R, int U, bool SPLIT, bool MULTI>
__global__ void __launch_bounds__(512)
    __attribute__((amdgpu_waves_per_eu(1, fast_waves_per_simd<M, R, U>()))) gemv_fast(ArgsT<MULTI> p)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = p.waves;
    const int row_first = (blockIdx.x * waves + wave) * R;
    // No early exit for waves past N (only in the last workgroup): their rows are clamped to
    // N-1 and their stores skipped, which keeps the prologue free of argument-dependent
    // branches.
    fast_rows<M, R, U, MULTI>(p, row_first, lane);
    if constexpr (SPLIT)
        combine_if_last<MULTI>(p, M, waves * R);
}

// ---------------------------------------------------------------------------- unaligned
// Any 2-byte-aligned layout. Per row, the 16-byte vectors are placed where the row's W
// address is 16-byte aligned (starting at element h, 0 <= h < 8); the up to 7 elements
// before the first vector and after the last one are scalar. The matching x window sits
// at a shift q (per row and batch) from X's own 16-byte grid; it is read as five dwords
// from the 4-byte boundary at or just below it and shifted into place, or element by
// element near the ends of a row of X.

typedef unsigned int u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// x[k .. k+7] for k >= 1 and k + 10 <= K, q as below: the window starts at an element
// offset of q & 1 from a 4-byte boundary, so four dwords from there and one more hold it,
// and a byte shift of 0 or 2 per dword extracts it (no data-dependent select).
__device__ __forceinline__ u32x4 x_window_interior(const uint16_t *xr, int k, int q)
{
    const unsigned *d = reinterpret_cast<const unsigned *>(xr + k - (q & 1));
    const u32x4 a = *reinterpret_cast<const u32x4_a4 *>(d);
    const unsigned e = d[4];
    const unsigned sh = (unsigned)(q & 1) * 2u;   // bytes
    const unsigned a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w;
    u32x4 r;
    r.x = __builtin_amdgcn_alignbyte(a1, a0, sh);
    r.y = __builtin_amdgcn_alignbyte(a2, a1, sh);
    r.z = __builtin_amdgcn_alignbyte(a3, a2, sh);
    r.w = __builtin_amdgcn_alignbyte(e, a3, sh);
    return r;
}

// x[k .. k+7] of one row of X with k + 8 <= K; q = element offset of x + k from the
// 16-byte grid.
__device__ __forceinline__ u32x4 x_window(const uint16_t *xr, int k, int K, int q)
{
    if (k >= 1 && k + 10 <= K)
        return x_window_interior(xr, k, q);
    u32x4 r;
    r.x = (unsigned)xr[k + 0] | ((unsigned)xr[k + 1] << 16);
    r.y = (unsigned)xr[k + 2] | ((unsigned)xr[k + 3] << 16);
    r.z = (unsigned)xr[k + 4] | ((unsigned)xr[k + 5] << 16);
    r.w = (unsigned)xr[k + 6] | ((unsigned)xr[k + 7] << 16);
    return r;
}

// Vectors each lane loads before using any, per batch size: the x windows take two loads
// per vector and batch row, so the burst shrinks as M grows (registers).
template <int M>
constexpr int unaligned_unroll()
{
    return M <= 3 ? 4 : M <= 6 ? 2 : 1;
}

template <int M, bool SPLIT, bool MULTI>
__global__ void __launch_bounds__(512) gemv_unaligned(ArgsT<MULTI> p)
{
    constexpr int U = unaligned_unroll<M>();
    const int rows_per_wave = p.rows;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = p.waves;
    const int row_first = (blockIdx.x * waves + wave) * rows_per_wave;
    const int split = blockIdx.y;
    const int k0 = split * p.slice;
    const int kend = min(p.k, k0 + p.slice);

    for (int r = 0; r < rows_per_wave; ++r) {
        const int row = row_first + r;
        if (row >= p.n)
            break;
        const uint16_t *wr = locate<MULTI>(p, row).w;
        const int h = (int)((8u - (unsigned)(((uintptr_t)wr >> 1) & 7u)) & 7u);
        const int ka = k0 + h;                        // first vector start (k0 % 8 == 0)
        const int nvec = ka + 8 <= kend ? (kend - ka) >> 3 : 0;
        const int head_end = min(ka, kend);
        const int tail_begin = max(head_end, ka + 8 * nvec);

        int q[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            q[m] = (int)((((uintptr_t)(p.x + (int64_t)m * p.ldx) >> 1) + (unsigned)h) & 7u);

        float acc[1][M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[0][m] = 0.f;

        // Lane l takes vectors l, l + 64, ... in increasing order, in bursts of U per lane
        // with every load of a burst issued before the first use. Vectors [vlo, vend) have
        // their x windows inside every row of X with room for the five-dword read; a burst
        // made only of those takes the short path, the others (the first when vector 0 sits
        // at the very start of X, and the last, partial one) clamp their loads and window
        // reads into range and drop the out-of-range vectors from the sums.
        const int vlo = ka >= 1 ? 0 : 1;
        const int vhi = p.k - 10 - ka >= 0 ? ((p.k - 10 - ka) >> 3) + 1 : 0;
        const int vend = max(vlo, min(nvec, vhi));
        for (int v0 = 0; v0 < nvec; v0 += 64 * U) {
            u32x4 wv[U], xv[U][M];
            if (v0 >= vlo && v0 + 64 * U <= vend) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    wv[u] = load_stream(wr + ka + 8 * (v0 + lane + 64 * u));
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        xv[u][m] = x_window_interior(p.x + (int64_t)m * p.ldx,
                                                     ka + 8 * (v0 + lane + 64 * u), q[m]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc[0][m] = dot8(wv[u], xv[u][m], acc[0][m]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    wv[u] = load_stream(wr + ka + 8 * min(v0 + lane + 64 * u, nvec - 1));
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        xv[u][m] = x_window(p.x + (int64_t)m * p.ldx,
                                            ka + 8 * min(v0 + lane + 64 * u, nvec - 1), p.k, q[m]);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool in = v0 + lane + 64 * u < nvec;
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc[0][m] = in ? dot8(wv[u], xv[u][m], acc[0][m]) : acc[0][m];
                }
            }
        }
        // Lanes 0..7 take the head elements, lanes 8..15 the tail elements.
        const int kk = lane < 8 ? k0 + lane : tail_begin + (lane - 8);
        const bool take = lane < 8 ? kk < head_end : (lane < 16 && kk < kend);
        if (take) {
            float w = bf16_to_f32(wr[kk]);
#pragma unroll
            for (int m = 0; m < M; ++m)
                acc[0][m] = fmaf(w, bf16_to_f32(p.x[(int64_t)m * p.ldx + kk]), acc[0][m]);
        }
        finish<M, 1, MULTI>(p, acc, row, split, lane);
    }
    if constexpr (SPLIT)
        combine_if_last<MULTI>(p, M, waves * rows_per_wave);
}

// Unsplit single-matrix calls take this form of the unaligned path. Rows whose W addresses
// have the same offset from the 16-byte grid - row r and r + T, where T = 8 / gcd(ldw, 8) -
// start their vectors at the same element h and so meet the same x windows; a workgroup owns
// rows of one such class (blockIdx.y), copies the M shifted x rows into LDS, and its waves
// then stream W with aligned loads and read the windows from LDS, exactly as the aligned
// kernels read x. When the M rows do not fit, they are staged `chunk` vectors at a time,
// with a barrier between chunks. Each lane takes vectors l, l + 64, ... in increasing order
// and then the head and tail elements, as gemv_unaligned does, so both give bitwise the
// same result on those rows.
// The rows of a class past its last whole group of 8 (at most 7, the tail rows) are summed
// differently: all 8 waves of one workgroup share each such row, wave w taking the w-th
// eighth of its vectors and reading x from global memory, and the 8 wave sums are added in
// wave order. A lone leftover row (4097 rows in 8 classes leave one) then costs an eighth
// of a pass instead of a whole extra pass for one workgroup (measured at 4097 x 14337:
// 26.3 us against 22.8 us at 4096 rows). Which rows are tail rows depends only on N and the
// classes, and their order on nothing but K, so every M sums each row the same way.
// Two shapes of wave: R rows per wave, U vectors per lane and row per burst (the same bytes
// in flight). One row per wave spreads the rows over more waves; two rows per wave halve
// the LDS reads of x, which at larger M bound the kernel.
struct ShiftShape {
    int r, u;
};
constexpr ShiftShape kShiftShapes[2] = {{1, 4}, {2, 2}};
// One row per wave up to M = 4, two above (measured at 4097 x 14337, M = 1..16).
constexpr int shift_shape_of(int m) { return m <= 4 ? 0 : 1; }
constexpr int kTailGroup = 8;   // tail rows: those past the last whole group of this many
constexpr int kShiftWaves = 8;  // waves per workgroup of the class-staged kernel

template <int M, int R, int U>
__global__ void __launch_bounds__(512) gemv_unaligned_lds(Args p, int classes, int chunk)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    u32x4 *xs = reinterpret_cast<u32x4 *>(lds);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int waves = (int)(blockDim.x >> 6);
    const int cls = blockIdx.y;
    const int class_rows = (p.n - cls + classes - 1) / classes;
    const int tail0 = class_rows & ~(kTailGroup - 1);   // rows [tail0, class_rows): tail rows
    const int ntail = class_rows - tail0;
    const int blocks = (tail0 + waves * R - 1) / (waves * R);   // row blocks of the rest
    const bool has_main = (int)blockIdx.x < blocks;   // uniform per workgroup
    if (!has_main && (int)blockIdx.x >= ntail)
        return;
    const uint16_t *w_cls = p.w0 + (int64_t)cls * p.ldw0;
    const int h = (int)((8u - (unsigned)(((uintptr_t)w_cls >> 1) & 7u)) & 7u);
    const int ka = min(h, p.k);
    const int nvec = ka + 8 <= p.k ? (p.k - ka) >> 3 : 0;
    const int tail_begin = ka + 8 * nvec;
    int q[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        q[m] = (int)((((uintptr_t)(p.x + (int64_t)m * p.ldx) >> 1) + (unsigned)h) & 7u);

    // Windows inside every row of X (vectors [vlo, vend)) are read without branches, SV per
    // thread and row of X in flight before any is written; the at most two others element
    // by element. Vectors [c0, c1) of every row of X go to xs[m * chunk + v - c0].
    constexpr int SV = M <= 4 ? 4 : M <= 8 ? 2 : 1;
    const int threads = (int)blockDim.x;
    const int tid = (int)threadIdx.x;
    const int vlo = ka >= 1 ? 0 : 1;
    const int vhi = p.k - 10 - ka >= 0 ? ((p.k - 10 - ka) >> 3) + 1 : 0;
    const int vend = min(nvec, vhi);
    // after_first() (the chunk's first weight burst) is issued right after the first batch
    // of x loads: vector loads retire in order, so the x writes then wait for x only. The
    // first pass runs on every lane (its loads are clamped), so the burst is wave-uniform.
    auto stage = [&](int c0, int c1, auto &&after_first) {
        bool first = true;
        if (vend > vlo) {
            const int i0 = max(c0, vlo), i1 = min(c1, vend);
            if (i1 > i0) {
                int v0 = i0 + tid;
                do {
                    u32x4 t[SV][M];
#pragma unroll
                    for (int i = 0; i < SV; ++i) {
                        const int vc = min(v0 + i * threads, i1 - 1);
#pragma unroll
                        for (int m = 0; m < M; ++m)
                            t[i][m] = x_window_interior(p.x + (int64_t)m * p.ldx, ka + 8 * vc,
                                                        q[m]);
                    }
                    if (first) {
                        after_first();
                        first = false;
                    }
#pragma unroll
                    for (int i = 0; i < SV; ++i) {
                        const int v = v0 + i * threads;
                        if (v < i1) {
#pragma unroll
                            for (int m = 0; m < M; ++m)
                                xs[m * chunk + v - c0] = t[i][m];
                        }
                    }
                    v0 += SV * threads;
                } while (v0 < i1);
            }
            if (first) {
                after_first();
                first = false;
            }
            // the edge vectors of the chunk: [c0, min(c1, vlo)) and [max(c0, vend), c1)
            const int e1 = max(0, min(c1, vlo) - c0);
            const int e2 = max(0, c1 - max(c0, vend));
            for (int e = tid; e < e1 + e2; e += threads) {
                const int v = e < e1 ? c0 + e : max(c0, vend) + (e - e1);
#pragma unroll
                for (int m = 0; m < M; ++m)
                    xs[m * chunk + v - c0] = x_window(p.x + (int64_t)m * p.ldx, ka + 8 * v, p.k, q[m]);
            }
        } else {
            after_first();
            for (int v = c0 + tid; v < c1; v += threads) {
#pragma unroll
                for (int m = 0; m < M; ++m)
                    xs[m * chunk + v - c0] = x_window(p.x + (int64_t)m * p.ldx, ka + 8 * v, p.k, q[m]);
            }
        }
    };

    const uint16_t *wr[R];
    u32x4 wv[U][R];
    auto burst = [&](int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[u][r] = load_stream(wr[r] + 8 * min(s0 + lane + 64 * u, nvec - 1));
    };
    auto rows_of = [&](int blk) {   // rows past tail0 re-read row tail0 - 1, unstored
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = min((blk * waves + wave) * R + r, tail0 - 1);
            wr[r] = p.w0 + (int64_t)(cls + classes * j) * p.ldw0 + ka;
        }
    };

    // Tail rows first: workgroup b takes tail rows b, b + gridDim.x, ... of its class. They
    // read x from global memory, so their latency overlaps the other workgroups' streams
    // and this workgroup's own x staging instead of trailing its last row block.
    constexpr int kTailU = M <= 4 ? 4 : 2;   // vectors per lane in flight on a tail row
    const int per = (nvec + waves - 1) / waves;
    const int vb = wave * per, ve = min(nvec, vb + per);   // this wave's vectors of the row
    __shared__ float sums[kShiftWaves * M];                // [wave][m]
    for (int t = blockIdx.x; t < ntail; t += gridDim.x) {
        const int j = tail0 + t;
        const uint16_t *wrow = p.w0 + (int64_t)(cls + classes * j) * p.ldw0 + ka;
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[m] = 0.f;
        for (int v0 = vb; v0 < ve; v0 += 64 * kTailU) {
            u32x4 tw[kTailU];
#pragma unroll
            for (int u = 0; u < kTailU; ++u)
                tw[u] = load_stream(wrow + 8 * min(v0 + lane + 64 * u, ve - 1));
#pragma unroll
            for (int u = 0; u < kTailU; ++u) {
                const int v = v0 + lane + 64 * u;
                const int vc = min(v, ve - 1);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const u32x4 xv = x_window(p.x + (int64_t)m * p.ldx, ka + 8 * vc, p.k, q[m]);
                    const float next = dot8(tw[u], xv, acc[m]);
                    acc[m] = v < ve ? next : acc[m];
                }
            }
        }
        if (wave == 0) {   // lanes 0..7 the head elements, lanes 8..15 the tail elements
            const int kk = lane < 8 ? lane : tail_begin + (lane - 8);
            const bool take = lane < 8 ? kk < ka : (lane < 16 && kk < p.k);
            if (take) {
                const float w = bf16_to_f32(wrow[kk - ka]);
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[m] = fmaf(w, bf16_to_f32(p.x[(int64_t)m * p.ldx + kk]), acc[m]);
            }
        }
        float ws[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            ws[m] = lane63(wave_sum(acc[m]));
        __syncthreads();   // the previous tail row's sums have been read
        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                sums[wave * M + m] = ws[m];
        }
        __syncthreads();
        if (wave == 0 && lane < M) {
            float v = sums[lane];
            for (int w = 1; w < waves; ++w)
                v += sums[w * M + lane];
            p.y0[(int64_t)lane * p.ldy0 + cls + classes * j] = v;
        }
    }

    // When the M rows of x fit (chunk >= nvec) they are staged once and serve every row
    // block this workgroup takes; otherwise each row block stages them chunk by chunk.
    const bool once = chunk >= nvec;
    if (has_main) {
        rows_of(blockIdx.x);
        if (once) {
            stage(0, nvec, [&] {
                if (nvec > 0)
                    burst(0);   // the first weights are in flight while x is staged
            });
            __syncthreads();
        } else if (nvec > 0) {
            burst(0);
        }
        for (int blk = blockIdx.x;;) {
            float acc[R][M];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[r][m] = 0.f;
            // chunk is a multiple of 64 * U (or covers the row), so every lane still meets its
            // vectors l, l + 64, ... in increasing order, whatever the chunking.
            for (int c0 = 0; c0 < nvec; c0 += chunk) {
                const int c1 = min(nvec, c0 + chunk);
                if (!once) {
                    // Chunks: the burst goes out before the barrier, while other waves finish
                    // the previous chunk (measured faster here than after the first x loads).
                    if (c0 > 0)
                        burst(c0);
                    __syncthreads();   // every wave is done with the previous contents
                    stage(c0, c1, [] {});
                    __syncthreads();
                }
                for (int s0 = c0; s0 < c1; s0 += 64 * U) {
                    if (s0 > c0)
                        burst(s0);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int v = s0 + lane + 64 * u;
                        const int vc = min(v, c1 - 1);
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            const u32x4 xv = xs[m * chunk + vc - c0];
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                const float next = dot8(wv[u][r], xv, acc[r][m]);
                                acc[r][m] = v < c1 ? next : acc[r][m];
                            }
                        }
                    }
                }
            }
            // Lanes 0..7 take the head elements, lanes 8..15 the tail elements.
            const int kk = lane < 8 ? lane : tail_begin + (lane - 8);
            const bool take = lane < 8 ? kk < ka : (lane < 16 && kk < p.k);
            if (take) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float w = bf16_to_f32(wr[r][kk - ka]);
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        acc[r][m] = fmaf(w, bf16_to_f32(p.x[(int64_t)m * p.ldx + kk]), acc[r][m]);
                }
            }
            float out = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float sum = lane63(wave_sum(acc[r][m]));
                    if (lane == r * M + m)
                        out = sum;
                }
            const int j0 = (blk * waves + wave) * R;
            if (lane < R * M) {
                const int r = lane / M, m = lane - (lane / M) * M;
                if (j0 + r < tail0)
                    p.y0[(int64_t)m * p.ldy0 + cls + classes * (j0 + r)] = out;
            }
            blk += gridDim.x;
            if (blk >= blocks)
                break;
            rows_of(blk);
            if (nvec > 0)
                burst(0);
        }
    }
}

template <size_t... I>
std::array<const void *, GEMV_MAX_M> unaligned_lds_table(std::index_sequence<I...>)
{
    return {reinterpret_cast<const void *>(
        &gemv_unaligned_lds<(int)I + 1, kShiftShapes[shift_shape_of((int)I + 1)].r,
                            kShiftShapes[shift_shape_of((int)I + 1)].u>)...};
}

// [M - 1], each M on its wave shape
const std::array<const void *, GEMV_MAX_M> kUnalignedLds =
    unaligned_lds_table(std::make_index_sequence<GEMV_MAX_M>{});

// ---------------------------------------------------------------------------- dispatch
// Kernel handles for hipLaunchKernel; fused instances take ArgsMulti, the others Args.
template <size_t I, bool SPLIT, bool MULTI>
const void *fast_at()
{
    constexpr bbd::Variant v = bbd::kVariants[I];
    return reinterpret_cast<const void *>(&gemv_fast<v.m, v.r, v.u, SPLIT, MULTI>);
}

constexpr size_t kNumVariants = sizeof(bbd::kVariants) / sizeof(bbd::kVariants[0]);
using KernelTable = std::array<const void *, kNumVariants>;

template <bool SPLIT, bool MULTI, size_t... I>
KernelTable fast_table(std::index_sequence<I...>)
{
    return {fast_at<I, SPLIT, MULTI>()...};
}

// [split][multi]
const KernelTable kFast[2][2] = {
    {fast_table<false, false>(std::make_index_sequence<kNumVariants>{}),
     fast_table<false, true>(std::make_index_sequence<kNumVariants>{})},
    {fast_table<true, false>(std::make_index_sequence<kNumVariants>{}),
     fast_table<true, true>(std::make_index_sequence<kNumVariants>{})}};

using UnalignedTable = std::array<const void *, GEMV_MAX_M>;

template <bool SPLIT, bool MULTI, size_t... I>
UnalignedTable unaligned_table(std::index_sequence<I...>)
{
    return {reinterpret_cast<const void *>(&gemv_unaligned<(int)I + 1, SPLIT, MULTI>)...};
}

const UnalignedTable kUnaligned[2][2] = {
    {unaligned_table<false, false>(std::make_index_sequence<GEMV_MAX_M>{}),
     unaligned_table<false, true>(std::make_index_sequence<GEMV_MAX_M>{})},
    {unaligned_table<true, false>(std::make_index_sequence<GEMV_MAX_M>{}),
     unaligned_table<true, true>(std::make_index_sequence<GEMV_MAX_M>{})}};

const void *find_fast(int m, int r, int u, bool split, bool multi)
{
    for (size_t i = 0; i < kNumVariants; ++i)
        if (bbd::kVariants[i].m == m && bbd::kVariants[i].r == r && bbd::kVariants[i].u == u)
            return kFast[split][multi][i];
    return nullptr;
}

gemv_status device_error(hipError_t e) { return record_hip_error((int)e, GEMV_ERR_DEVICE); }


// Launch an unsplit single-matrix unaligned call on gemv_unaligned_lds; *done tells whether
// it did. The staged chunk of x is the whole row when the M rows fit in kShiftMaxLds, else
// the largest multiple of a burst (64 lanes x U vectors) that fits.
gemv_status launch_unaligned_lds(gemv_plan_t p, const gemv_segment &seg, const void *X,
                                 int64_t ldx, void *stream, bool *done)
{
    *done = false;
    const int64_t vecs = p->k / 8;   // vectors per row of the class with the most
    if (p->splits != 1 || vecs == 0)
        return GEMV_OK;
    const int64_t per_vec = (int64_t)p->m * (int64_t)sizeof(u32x4);
    const int shape = shift_shape_of(p->m);
    const ShiftShape sh = kShiftShapes[shape];
    const int64_t burst = (int64_t)kWaveLanes * sh.u;
    int64_t chunk_vecs = vecs;
    if (vecs * per_vec > (int64_t)kShiftMaxLds)
        chunk_vecs = (int64_t)kShiftMaxLds / per_vec / burst * burst;
    if (chunk_vecs < 1)
        return GEMV_OK;
    int chunk = (int)chunk_vecs;
    const size_t bytes = (size_t)(chunk_vecs * per_vec);
    const void *fn = kUnalignedLds[p->m - 1];
    static std::atomic<bool> allowed[2][GEMV_MAX_M + 1];
    if (bytes > 64 * 1024 && !allowed[shape][p->m].load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kShiftMaxLds);
        if (e != hipSuccess)
            return device_error(e);
        allowed[shape][p->m].store(true, std::memory_order_release);
    }
    *done = true;
    // Rows r and r + classes start at the same offset from the 16-byte grid.
    int g = (int)(seg.ldw % 8);
    int classes = 8;
    if (g == 0)
        classes = 1;
    else if (g % 4 == 0)
        classes = 2;
    else if (g % 2 == 0)
        classes = 4;
    const int waves = kShiftWaves;
    // Row blocks of whole groups of kTailGroup rows in the largest class, and the most tail
    // rows any class has (each needs a workgroup of its class).
    const int64_t class_rows = (p->n + classes - 1) / classes;
    const int64_t main_rows = class_rows / kTailGroup * kTailGroup;
    int64_t blocks = (main_rows + (int64_t)sh.r * waves - 1) / ((int64_t)sh.r * waves);
    int64_t tails = 0;
    for (int c = 0; c < classes; ++c)
        tails = std::max<int64_t>(tails, ((p->n - c + classes - 1) / classes) % kTailGroup);
    // When x fits, workgroups take row blocks blockIdx.x, + gridDim.x, ...: no more of them
    // per class than the classes' share of what the device holds at once, so none waits for
    // a slot and x is staged once per workgroup. Chunked x is staged per row block anyway,
    // and there one row block per workgroup measured faster.
    if (chunk_vecs >= vecs) {
        // The occupancy query, cached per kernel for the last LDS size asked about (one
        // 64-bit word: bytes in the high half, workgroups per CU in the low half).
        static std::atomic<uint64_t> occ[2][GEMV_MAX_M + 1];
        const uint64_t seen = occ[shape][p->m].load(std::memory_order_relaxed);
        int per_cu = 0;
        if (seen >> 32 == (uint64_t)bytes) {
            per_cu = (int)(seen & 0xFFFFFFFFu);
        } else {
            hipError_t oe = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, fn, kWaveLanes * waves, bytes);
            if (oe != hipSuccess)
                return device_error(oe);
            occ[shape][p->m].store(((uint64_t)bytes << 32) | (uint32_t)per_cu,
                                   std::memory_order_relaxed);
        }
        const int64_t resident = (int64_t)std::max(per_cu, 1) * p->dev.compute_units;
        blocks = std::min(blocks, std::max<int64_t>(1, (resident + classes - 1) / classes));
    }
    blocks = std::max(blocks, tails);
    if (blocks < 1)
        blocks = 1;
    Args a;
    memset(&a, 0, sizeof a);
    a.w0 = static_cast<const uint16_t *>(seg.W);
    a.y0 = seg.Y;
    a.x = static_cast<const uint16_t *>(X);
    a.ldw0 = (int32_t)seg.ldw;
    a.ldy0 = (int32_t)seg.ldy;
    a.ldx = p->m > 1 ? (int32_t)ldx : 0;
    a.n = (int32_t)p->n;
    a.k = (int32_t)p->k;
    a.slice = (int32_t)p->k;
    a.waves = waves;
    a.rows = sh.r;
    void *args[] = {&a, &classes, &chunk};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks, (unsigned)classes),
                                   dim3(kWaveLanes * waves), args, bytes,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : device_error(e);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned2(const void *p) { return ((uintptr_t)p & 1u) == 0; }

// Validation of everything but the workspace, shared by gemv_run, gemv_fused_run and
// gemv_run_static; makes no HIP call.
gemv_status validate_call(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                          int64_t ldx)
{
    if (!p || !segs || nseg < 1 || nseg > GEMV_MAX_SEGMENTS || !X ||
        p->weights != GEMV_WEIGHTS_BF16 || p->prologue != 0)
        return GEMV_ERR_INVALID_ARG;
    if (p->m > 1 && ldx < p->k)
        return GEMV_ERR_INVALID_ARG;
    if (p->m > 1 && ldx > INT32_MAX)
        return GEMV_ERR_INVALID_ARG;
    int64_t rows = 0;
    for (int i = 0; i < nseg; ++i) {
        const gemv_segment &s = segs[i];
        if (!s.W || !s.Y || s.n < 1 || s.ldw < p->k || s.ldy < s.n || s.ldw > INT32_MAX ||
            s.ldy > INT32_MAX)
            return GEMV_ERR_INVALID_ARG;
        rows += s.n;
    }
    if (rows != p->n)
        return GEMV_ERR_INVALID_ARG;
    if (!aligned2(X))
        return GEMV_ERR_MISALIGNED;
    for (int i = 0; i < nseg; ++i)
        if (!aligned2(segs[i].W) || !aligned4(segs[i].Y))
            return GEMV_ERR_MISALIGNED;
    return GEMV_OK;
}

// Validation shared by gemv_run and gemv_fused_run (caller's workspace); no HIP call.
gemv_status validate(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                     int64_t ldx, void *ws, size_t ws_bytes)
{
    gemv_status st = validate_call(p, segs, nseg, X, ldx);
    if (st != GEMV_OK)
        return st;
    if (p->workspace) {
        if (!ws || ws_bytes < p->workspace)
            return GEMV_ERR_WORKSPACE;
        if (!aligned4(ws))
            return GEMV_ERR_MISALIGNED;
    }
    return GEMV_OK;
}

// Launch a validated call. A split launch (VALU or matrix-core) takes its arrival tickets
// and partial sums from `tickets` and `partials`; an unsplit one touches neither.
gemv_status launch_on(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                      int64_t ldx, unsigned *tickets, float *partials, void *stream)
{
    gemv_status st;
    bool fast = aligned16(X) && (p->m == 1 || ldx % 8 == 0);
    for (int i = 0; i < nseg; ++i)
        fast = fast && aligned16(segs[i].W) && segs[i].ldw % 8 == 0;

    bool done = false;
    st = bbd::launch_whole(p, segs, nseg, X, stream, &done);
    if (done || st != GEMV_OK)
        return st;
    st = bbd::launch_mfma(p, segs, nseg, X, ldx, tickets, partials, stream, &done);
    if (done || st != GEMV_OK)
        return st;
    st = bbd::launch_batch(p, segs, nseg, X, ldx, stream, &done);
    if (done || st != GEMV_OK)
        return st;
    if (!fast && nseg == 1) {
        st = bbd::launch_mfma_unaligned(p, segs[0], X, ldx, stream, &done);
        if (done || st != GEMV_OK)
            return st;
        st = launch_unaligned_lds(p, segs[0], X, ldx, stream, &done);
        if (done || st != GEMV_OK)
            return st;
    }

    ArgsMulti a;
    memset(&a, 0, sizeof a);
    a.w0 = static_cast<const uint16_t *>(segs[0].W);
    a.y0 = segs[0].Y;
    a.x = static_cast<const uint16_t *>(X);
    a.ldw0 = (int32_t)segs[0].ldw;
    a.ldy0 = (int32_t)segs[0].ldy;
    a.ldx = p->m > 1 ? (int32_t)ldx : 0;
    a.n = (int32_t)p->n;
    a.k = (int32_t)p->k;
    a.slice = (int32_t)p->slice;
    a.waves = p->waves_per_block;
    a.rows = p->rows_per_wave;
    a.tickets = p->splits > 1 ? tickets : nullptr;
    a.partial = p->splits > 1 ? partials : nullptr;
    const bool multi = nseg > 1;
    if (multi) {
        int64_t row0 = 0;
        for (int i = 0; i < GEMV_MAX_SEGMENTS; ++i) {
            Seg &sg = a.seg[i];
            if (i < nseg) {
                sg.w = static_cast<const uint16_t *>(segs[i].W);
                sg.ldw = segs[i].ldw;
                sg.y = segs[i].Y;
                sg.ldy = segs[i].ldy;
                sg.row0 = (int32_t)row0;
                row0 += segs[i].n;
            } else {
                sg.row0 = INT32_MAX;            // never selected by locate()
            }
        }
    }
    // A single-segment kernel takes the Args prefix of the same object.
    Args single = a;

    const void *kernel = fast ? find_fast(p->m, p->rows_per_wave, p->unroll, p->splits > 1, multi)
                              : kUnaligned[p->splits > 1][multi][p->m - 1];
    if (!kernel)
        return GEMV_ERR_INVALID_ARG;
    void *args[] = {multi ? static_cast<void *>(&a) : static_cast<void *>(&single)};
    hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)p->grid_x, (unsigned)p->grid_y),
                                   dim3((unsigned)p->block_threads), args,
                                   (size_t)p->lds_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return device_error(e);
    return GEMV_OK;
}

// gemv_run / gemv_fused_run: the caller's workspace holds the tickets, then the partials.
gemv_status launch(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                   int64_t ldx, void *ws, size_t ws_bytes, void *stream)
{
    gemv_status st = validate(p, segs, nseg, X, ldx, ws, ws_bytes);
    if (st != GEMV_OK)
        return st;
    unsigned *tickets = nullptr;
    float *partials = nullptr;
    if (p->workspace) {
        tickets = static_cast<unsigned *>(ws);
        partials = reinterpret_cast<float *>(static_cast<char *>(ws) + p->partial_offset);
    }
    return launch_on(p, segs, nseg, X, ldx, tickets, partials, stream);
}

// The plan's LDS reservation assumes an allocation unit; confirm with the runtime's
// occupancy calculator that it admits exactly the intended workgroups per CU, and search
// the sizes that could (from kLdsPerCU / blocks down) if it does not. A cap the kernel's
// registers already enforce, or one no size achieves, is dropped.
gemv_status fit_cap(gemv_plan_t p, int device)
{
    const void *kernel = find_fast(p->m, p->rows_per_wave, p->unroll, p->splits > 1, false);
    if (!kernel)
        return GEMV_OK;
    int prev = 0;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess)
        e = hipSetDevice(device);
    if (e != hipSuccess)
        return device_error(e);
    const int blocks = p->waves_per_cu / p->waves_per_block;
    int unlimited = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&unlimited, kernel, p->block_threads, 0);
    int chosen = 0;
    if (e == hipSuccess && unlimited > blocks) {
        for (int bytes = bbd::kLdsPerCU / blocks / 256 * 256;
             e == hipSuccess && bytes * (blocks + 1) > bbd::kLdsPerCU; bytes -= 256) {
            int got = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&got, kernel, p->block_threads,
                                                             (size_t)bytes);
            if (e == hipSuccess && got == blocks) {
                chosen = bytes;
                break;
            }
        }
    }
    (void)hipSetDevice(prev);
    if (e != hipSuccess)
        return device_error(e);
    p->lds_bytes = chosen;
    if (!chosen)
        p->waves_per_cu = 0;
    return GEMV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Scratch for gemv_run_static: the split launches' arrival tickets (the first
// GEMV_STATIC_TICKET_SLOTS words) and partial sums (the rest), one copy per GPU, held until
// the process ends. Host code never uses this name as an address (on the host it is only a
// stand-in for the device symbol): the per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[GEMV_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kStaticMaxDevices = 64;
constexpr size_t kStaticTicketBytes = (size_t)GEMV_STATIC_TICKET_SLOTS * sizeof(unsigned);
static_assert(kStaticTicketBytes % 256 == 0, "partial sums start 256-byte aligned");
static_assert(GEMV_STATIC_SCRATCH_BYTES > kStaticTicketBytes, "room for partial sums");

std::mutex g_scratch_mutex;                                   // serialises the set-up
std::atomic<char *> g_scratch_ptr[kStaticMaxDevices];         // device address, per device

__global__ void __launch_bounds__(256) clear_words(unsigned *p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// The device address of `scratch` on `device`, looked up once per device with that device
// current. The first look-up also enqueues, on `stream`, a kernel that zeroes the ticket
// region (a fill kernel rather than a memset, so a capture that records it holds no memset
// node); every completed split call leaves its tickets at zero again.
gemv_status static_scratch(int device, void *stream, char **out)
{
    *out = nullptr;
    if (device < 0 || device >= kStaticMaxDevices)
        return record_hip_error(0, GEMV_ERR_DEVICE);
    char *ptr = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (ptr) {
        *out = ptr;
        return GEMV_OK;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (ptr) {
        *out = ptr;
        return GEMV_OK;
    }
    int prev = 0;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != device)
        e = hipSetDevice(device);
    void *addr = nullptr;
    if (e == hipSuccess)
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e == hipSuccess) {
        unsigned *tickets = static_cast<unsigned *>(addr);
        int words = GEMV_STATIC_TICKET_SLOTS;
        void *args[] = {&tickets, &words};
        e = hipLaunchKernel(reinterpret_cast<const void *>(clear_words),
                            dim3((unsigned)(GEMV_STATIC_TICKET_SLOTS / 256)), dim3(256), args, 0,
                            static_cast<hipStream_t>(stream));
    }
    if (prev != device)
        (void)hipSetDevice(prev);
    if (e != hipSuccess)
        return device_error(e);
    ptr = static_cast<char *>(addr);
    g_scratch_ptr[device].store(ptr, std::memory_order_release);
    *out = ptr;
    return GEMV_OK;
}

}  // namespace

extern "C" gemv_status gemv_run_static(gemv_plan_t p, const void *W, int64_t ldw, const void *X,
                                       int64_t ldx, float *Y, int64_t ldy, void *stream)
{
    if (!p)
        return GEMV_ERR_INVALID_ARG;
    gemv_segment seg = {W, p->n, ldw, Y, ldy};
    gemv_status st = validate_call(p, &seg, 1, X, ldx);
    if (st != GEMV_OK)
        return st;
    if (!p->workspace)                      // unsplit: no scratch at all
        return launch_on(p, &seg, 1, X, ldx, nullptr, nullptr, stream);
    // The launch that splits (VALU, matrix-core or both) must fit the static layout.
    int64_t blocks = 0;
    if (p->splits > 1)
        blocks = p->grid_x;
    if (p->mfma && p->mfma_splits > 1 && p->mfma_grid_x > blocks)
        blocks = p->mfma_grid_x;
    const size_t partial_bytes = p->workspace - p->partial_offset;
    if (blocks > GEMV_STATIC_TICKET_SLOTS ||
        partial_bytes > (size_t)GEMV_STATIC_SCRATCH_BYTES - kStaticTicketBytes)
        return GEMV_ERR_WORKSPACE;
    int device = p->device;
    if (device < 0) {
        hipError_t e = hipGetDevice(&device);
        if (e != hipSuccess)
            return device_error(e);
    }
    char *base = nullptr;
    st = static_scratch(device, stream, &base);
    if (st != GEMV_OK)
        return st;
    return launch_on(p, &seg, 1, X, ldx, reinterpret_cast<unsigned *>(base),
                     reinterpret_cast<float *>(base + kStaticTicketBytes), stream);
}

struct gemv_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

extern "C" gemv_status gemv_plan(gemv_plan_t *out, int64_t n, int64_t k, int m, int device,
                                 const gemv_plan_opts *opts)
{
    if (!out)
        return GEMV_ERR_INVALID_ARG;
    *out = nullptr;
    if (n < 1 || k < 1 || m < 1 || m > GEMV_MAX_M || device < 0)
        return GEMV_ERR_INVALID_ARG;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return device_error(e);
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return record_hip_error(0, GEMV_ERR_DEVICE);
    // MI355X: 8.0 TB/s HBM3E (published peak); the plan uses it only to report Little's law.
    gemv_device_desc dev = {prop.multiProcessorCount, 8.0e12, bbd::kDefaultLatency};
    gemv_status st = gemv_plan_for(out, n, k, m, &dev, opts);
    if (st != GEMV_OK)
        return st;
    (*out)->device = device;
    // The LDS reservation that enforces a resident-wave cap is for the bf16 kernels; INT4
    // and RMSNorm plans size their LDS for what they stage, and a cap there only limits
    // their grid.
    if ((*out)->waves_per_cu > 0 && (*out)->weights == GEMV_WEIGHTS_BF16 &&
        (*out)->prologue == 0) {
        st = fit_cap(*out, device);
        if (st != GEMV_OK) {
            gemv_plan_destroy(*out);
            *out = nullptr;
        }
    }
    return st;
}

extern "C" gemv_status gemv_run(gemv_plan_t p, const void *W, int64_t ldw, const void *X,
                                int64_t ldx, float *Y, int64_t ldy, void *workspace,
                                size_t ws_bytes, void *stream)
{
    if (!p)
        return GEMV_ERR_INVALID_ARG;
    gemv_segment seg = {W, p->n, ldw, Y, ldy};
    return launch(p, &seg, 1, X, ldx, workspace, ws_bytes, stream);
}

extern "C" gemv_status gemv_int4_run(gemv_plan_t p, const void *Wq, int64_t ldq, const void *S,
                                     int64_t lds, const void *X, float *Y, void *stream)
{
    if (!p || !Wq || !S || !X || !Y || p->weights != GEMV_WEIGHTS_INT4)
        return GEMV_ERR_INVALID_ARG;
    const int64_t groups = (p->k + kInt4Group - 1) / kInt4Group;
    if (ldq < p->k / 2 || ldq % 16 != 0 || ldq > INT32_MAX || lds < groups || lds > INT32_MAX)
        return GEMV_ERR_INVALID_ARG;
    if (!aligned16(Wq) || !aligned16(X) || !aligned2(S) || !aligned4(Y))
        return GEMV_ERR_MISALIGNED;
    return bbd::launch_int4(p, Wq, ldq, S, lds, X, Y, stream);
}

extern "C" gemv_status gemv_rmsnorm_run(gemv_plan_t p, const gemv_segment *segs, int nseg,
                                        const void *H, const void *gamma, float eps,
                                        void *stream)
{
    if (!p || !segs || nseg < 1 || nseg > GEMV_MAX_SEGMENTS || !H || !gamma ||
        p->prologue != GEMV_PROLOGUE_RMSNORM || !(eps >= 0.f) || !(eps <= 3.4e38f))
        return GEMV_ERR_INVALID_ARG;
    int64_t rows = 0;
    for (int i = 0; i < nseg; ++i) {
        const gemv_segment &s = segs[i];
        if (!s.W || !s.Y || s.n < 1 || s.ldw < p->k || s.ldw > INT32_MAX || s.ldw % 8 != 0 ||
            s.ldw != segs[0].ldw)
            return GEMV_ERR_INVALID_ARG;
        rows += s.n;
    }
    if (rows != p->n)
        return GEMV_ERR_INVALID_ARG;
    if (!aligned16(H) || !aligned16(gamma))
        return GEMV_ERR_MISALIGNED;
    for (int i = 0; i < nseg; ++i)
        if (!aligned16(segs[i].W) || !aligned4(segs[i].Y))
            return GEMV_ERR_MISALIGNED;
    return bbd::launch_rmsnorm(p, segs, nseg, H, gamma, eps, stream);
}

extern "C" gemv_status gemv_fused_run(gemv_plan_t p, const gemv_segment *segs, int nseg,
                                      const void *X, int64_t ldx, void *workspace,
                                      size_t ws_bytes, void *stream)
{
    return launch(p, segs, nseg, X, ldx, workspace, ws_bytes, stream);
}

extern "C" gemv_status gemv_graph_begin(void *stream)
{
    if (!stream)
        return GEMV_ERR_CAPTURE;
    hipError_t e = hipStreamBeginCapture(static_cast<hipStream_t>(stream),
                                         hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_CAPTURE);
    return GEMV_OK;
}

extern "C" gemv_status gemv_graph_end(void *stream, gemv_graph_t *out)
{
    if (!out)
        return GEMV_ERR_INVALID_ARG;
    *out = nullptr;
    if (!stream)
        return GEMV_ERR_CAPTURE;
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &graph);
    if (e != hipSuccess || !graph)
        return record_hip_error((int)e, GEMV_ERR_CAPTURE);
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return device_error(e);
    }
    gemv_graph_s *g = new (std::nothrow) gemv_graph_s{graph, exec};
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return GEMV_ERR_INVALID_ARG;
    }
    *out = g;
    return GEMV_OK;
}

extern "C" gemv_status gemv_graph_launch(gemv_graph_t g, void *stream)
{
    if (!g)
        return GEMV_ERR_INVALID_ARG;
    hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return device_error(e);
    return GEMV_OK;
}

extern "C" void gemv_graph_destroy(gemv_graph_t g)
{
    if (!g)
        return;
    (void)hipGraphExecDestroy(g->exec);
    (void)hipGraphDestroy(g->graph);
    delete g;
}

namespace bbd {

namespace {
thread_local int g_last_hip_error = 0;
}

gemv_status record_hip_error(int hip_error, gemv_status status)
{
    g_last_hip_error = hip_error;
    return status;
}

}  // namespace bbd

extern "C" int gemv_last_hip_error(void) { return bbd::g_last_hip_error; }
