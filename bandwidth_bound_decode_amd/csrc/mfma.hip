// mfma.hip - skinny-batch GEMV on the matrix cores (by default for 2 <= M <= 16).
//
// The VALU kernels multiply every weight vector a lane loads by M input vectors with
// v_dot2 instructions, so their time grows with M (about 0.6 us per extra vector at
// 4096 x 14336: 19.9 us at M = 2, 24.4 at 8, 28.3 at 16). Here one v_mfma_f32_16x16x32_bf16
// takes 16 weight rows (A operand) and 16 input vectors (B operand) over 32 K elements, so
// the arithmetic per weight byte does not grow with M (19.4 us at M = 2, 19.8 at 8). Batches
// below 16 repeat vectors in the unused B columns, whose outputs are never stored.
//
// Two kernels: gemv_mfma for aligned single-matrix calls (below), and gemv_mfma_unaligned
// (at the end) for calls whose W or x rows are off the 16-byte grid, from M = 10.
//
// Operand layout of the 16x16x32 bf16 MFMA on gfx950 (checked on the device against an
// exact integer product): lane l holds A[l % 16][8 (l / 16) .. +8) and B[8 (l / 16) .. +8)
// [l % 16] as 8 packed bf16, and D[4 (l / 16) + e][l % 16] in accumulator register e. Only
// the pairing of A and B elements matters to the sum, so K element 32 u + 8 g + e of a chunk
// goes to lane group g of MFMA u: every 16-byte operand is 8 contiguous K elements of one
// row (of W) or one vector (of X).
//
// Work split (measured on MI355X at 4096 x 14336, M = 2..16; probe sweeps of tiles per
// workgroup, chunk sizes, MFMAs per burst, waves per workgroup and split counts):
//   - a workgroup owns T 16-row tiles and one K slice; its 8 waves take the slice's chunks
//     in turn, starting at a per-workgroup rotation so that workgroups running side by
//     side read different column ranges of their rows. Two forms: T = 2 with 64-element
//     chunks (the two tiles share every X fragment, halving X traffic against one tile),
//     and T = 1 with 128-element chunks: twice the row blocks, so 4096 rows fill 256 CUs
//     with no split and no combine (19.8 us against 21.1 us at M = 8). T = 1 stages 8 X
//     vectors for M <= 8 and 16 above; with 16 it reads as many X bytes as W bytes at
//     M = 16, which the split it avoids is worth up to M = 14 at K = 14336 and at every M
//     at K = 4096 (e.g. 4096 x 4096, M = 9..16: 7.3-7.8 against 9.2 us split);
//   - a chunk row is one or two 128-byte lines. Loaded straight in the operand layout,
//     every load instruction touches 16 rows x 64 bytes (half of 16 cache lines); a
//     read-only probe of that pattern streamed W at 4.3-5.7 TB/s against 6.4 TB/s for
//     whole lines. So the wave moves the chunk into a private LDS buffer with direct
//     global-to-LDS loads that each cover one line of 8 rows (W with the streaming hint),
//     then reads the operands from LDS. Load lane l takes row l / 8 of its 8 and the
//     16-byte piece (l % 8) ^ (l / 8) of that row's line, and writes LDS slot l; the XOR
//     puts the 8 rows an operand read gathers in 8 different bank groups. MFMA u of a
//     chunk takes K elements 32 u + 8 g .. + 8 in lane group g, i.e. piece 4 (u % 2) + g of
//     line u / 2, on both the A and the B side;
//   - per chunk: the direct loads, the wait for them, the LDS operand reads, the next
//     chunk's loads (once the reads are in registers), then the MFMAs;
//   - the 8 waves' partial tiles are summed in LDS in wave order, then stored; a plan that
//     splits K (too few row blocks for the CUs) stores device-coherent partials and the
//     last workgroup of a row block to arrive adds them in slice order, as the VALU
//     kernels' split combine does.
// The order of every sum is fixed, so results are reproducible bit for bit; they differ in
// rounding from the VALU kernels' (a different summation order).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = kWaveLanes * kMfmaWaves;
constexpr int kLineRows = 8;                     // rows (or X vectors) per direct load
constexpr int kLineElems = 64;                   // bf16 elements in a 128-byte line
constexpr int kCachePolicyNT = 2;                // the streaming hint on a direct load
constexpr int kWaitVmOnly = 0x0F70;              // s_waitcnt vmcnt(0)
constexpr int kWaitLgkmOnly = 0xC07F;            // s_waitcnt lgkmcnt(0)

__device__ __forceinline__ floatx4 mfma(u32x4 a, u32x4 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// y[m][row] = sum_k w[row][k] x[m][k] for the row block blockIdx.x (T 16-row tiles) and
// the K slice blockIdx.y (of gridDim.y), in chunks of CH elements. XV: X vectors staged
// per chunk (16, or 8 when M <= 8: B lanes 8..15 then repeat vectors 0..7, and their
// output columns are never stored; vectors past M repeat vector M - 1, whose lines the
// memory system then fetches once). With one slice the result goes to y; with several,
// to partial[slice][m][row] and then, by the last arrival, to y.
template <int T, int XV, int CH>
__global__ void __launch_bounds__(kThreads)
    gemv_mfma(const uint16_t *w, const uint16_t *x, float *y, float *partial,
              unsigned *tickets, int n, int k, int ldw, int ldx, int ldy, int m, int slice)
{
    constexpr int kRows = 16 * T;                    // rows per workgroup
    constexpr int kLines = CH / kLineElems;          // 128-byte lines per row per chunk
    constexpr int kU = CH / 32;                      // MFMAs per tile per chunk
    constexpr int kWGroups = kRows / kLineRows;      // 8-row groups of W
    constexpr int kXGroups = XV / kLineRows;         // 8-vector groups of X
    constexpr int kWLoads = kWGroups * kLines;
    constexpr int kXLoads = kXGroups * kLines;
    static_assert(CH % kLineElems == 0 && (XV == 8 || XV == 16), "unsupported form");
    __shared__ floatx4 red[kMfmaWaves - 1][T][kWaveLanes];
    // Each wave's chunk: load j = group * kLines + line (1 KiB each), W groups first.
    __shared__ u32x4 stage[kMfmaWaves][kWLoads + kXLoads][kWaveLanes];
    __shared__ unsigned s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int i16 = lane & 15, g = lane >> 4;
    const int splits = gridDim.y, s = blockIdx.y;
    const int row0 = blockIdx.x * kRows;
    const int k0 = s * slice;
    const int chunks = min(slice, k - k0) / CH;

    // Load side: row (or vector) lr of each group, piece lq of each of its lines.
    const int lr = lane >> 3, lq = (lane & 7) ^ lr;
    const uint16_t *gw[kWGroups];
#pragma unroll
    for (int j = 0; j < kWGroups; ++j)   // rows past N re-read row N-1; never stored
        gw[j] = w + (int64_t)min(row0 + kLineRows * j + lr, n - 1) * ldw + k0 + 8 * lq;
    const uint16_t *gx[kXGroups];
#pragma unroll
    for (int j = 0; j < kXGroups; ++j)   // vectors past M repeat the last one
        gx[j] = x + (int64_t)min(kLineRows * j + lr, m - 1) * ldx + k0 + 8 * lq;
    // Read side: operand lane (i16, g) of MFMA u takes piece 4 (u % 2) + g of line u / 2 of
    // row i16, which group i16 / 8 (of its tile, or of X) left in slot
    // 8 (i16 % 8) + ((4 (u % 2) + g) ^ (i16 % 8)).
    const int ri = i16 & 7, hj = i16 >> 3;
    const int xg = kXGroups == 2 ? hj : 0;
    int slot[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        slot[h] = kLineRows * ri + ((4 * h + g) ^ ri);
    u32x4 (&buf)[kWLoads + kXLoads][kWaveLanes] = stage[wave];

    const int turns = (chunks - wave + kMfmaWaves - 1) / kMfmaWaves;
    const int rot = (int)((blockIdx.x * 37u + (unsigned)s * 11u) % (unsigned)chunks);
    auto issue = [&](int i) {
        int c = wave + i * kMfmaWaves + rot;
        c = c >= chunks ? c - chunks : c;
#pragma unroll
        for (int j = 0; j < kWGroups; ++j)
#pragma unroll
            for (int l = 0; l < kLines; ++l)
                __builtin_amdgcn_global_load_lds(
                    (global_void *)(gw[j] + c * CH + kLineElems * l),
                    (lds_void *)&buf[j * kLines + l][0], 16, 0, kCachePolicyNT);
#pragma unroll
        for (int j = 0; j < kXGroups; ++j)
#pragma unroll
            for (int l = 0; l < kLines; ++l)
                __builtin_amdgcn_global_load_lds(
                    (global_void *)(gx[j] + c * CH + kLineElems * l),
                    (lds_void *)&buf[kWLoads + j * kLines + l][0], 16, 0, 0);
    };
    floatx4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (turns > 0)
        issue(0);
    for (int i = 0; i < turns; ++i) {
        __builtin_amdgcn_s_waitcnt(kWaitVmOnly);   // this chunk's lines have landed
        u32x4 a[T][kU], b[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                a[t][u] = buf[(2 * t + hj) * kLines + u / 2][slot[u & 1]];
            b[u] = buf[kWLoads + xg * kLines + u / 2][slot[u & 1]];
        }
        // The buffer is free once the reads are in registers; then the next chunk goes out.
        __builtin_amdgcn_s_waitcnt(kWaitLgkmOnly);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < turns)
            issue(i + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[t] = mfma(a[t][u], b[u], acc[t]);
    }

    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
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
    const int rows = min(kRows, n - row0);
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

// Unaligned rows (W rows or x rows not on the 16-byte grid) on the matrix cores, for larger
// batches, where the VALU kernels' work per weight grows with M. Rows c, c + C, c + 2C, ...
// (C = 8 / gcd(ldw, 8) classes) start at the same offset h from the 16-byte grid, so each
// class is an aligned matrix: base w + c ldw + h, row stride C ldw (a multiple of 8
// elements). A workgroup owns one 16-row tile of one class; the 1-D grid lists the tiles
// every class has first (class fastest), then each class's remaining tiles. Within a tile:
//   - the 8 waves take the class rows' whole 128-element chunks in turn from a
//     per-workgroup rotation and stream them through a private LDS buffer as the aligned
//     kernel does (direct loads of 8 rows x 128 bytes, XOR-swizzled slots; rows past the
//     class end are not loaded and never stored). A row's chunks start 16- but not 128-byte
//     aligned, so neighbouring chunks share a cache line; without the streaming hint the
//     second reader finds it in L2 (measured at 4097 x 14337, M = 16: 52.4 against 55.6 us,
//     HBM reads 1.12 against 1.24 times the algorithmic bytes);
//   - B comes from x in registers: for x row i16 at K element e, one 4-byte-aligned 16-byte
//     load and one dword give 9 dwords, and v_alignbyte by the row's 2-byte phase picks the
//     8 elements starting at e. These loads go out with the chunk's W lines;
//   - chunks whose x window would leave the row (the first when h = 0: the window starts
//     one element early; the last one or two) and the ragged end take one wave each, with
//     W loaded in the operand layout and x element by element, before the stream;
//   - the h head elements and the < 8 tail elements past the last whole vector are summed
//     per (x row, tile row) pair in fp32 by one thread each and added after the waves' sums.
// The order of every sum is fixed: bitwise reproducible, within the VALU kernels' tolerance
// (another summation order).
constexpr int kUnalChunk = 128;

__global__ void __launch_bounds__(kThreads)
    gemv_mfma_unaligned(const uint16_t *w, const uint16_t *x, float *y, int n, int k, int ldw,
                        int ldx, int ldy, int m, int classes)
{
    constexpr int CH = kUnalChunk;
    constexpr int kLines = CH / kLineElems, kU = CH / 32, kWLoads = 2 * kLines;
    __shared__ floatx4 red[kMfmaWaves - 1][kWaveLanes];
    __shared__ u32x4 stage[kMfmaWaves][kWLoads][kWaveLanes];
    __shared__ float edge_sums[16 * 16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int i16 = lane & 15, g = lane >> 4;

    // This workgroup's class and first class row.
    int cls = -1, j0 = 0;
    {
        const int id = blockIdx.x;
        const int common = n / classes / 16;   // whole tiles every class has
        if (id < common * classes) {
            cls = id % classes;
            j0 = id / classes * 16;
        } else {
            int r = id - common * classes;
            for (int c = 0; c < classes; ++c) {
                const int extra = ((n - c + classes - 1) / classes + 15) / 16 - common;
                if (r < extra) {
                    cls = c;
                    j0 = (common + r) * 16;
                    break;
                }
                r -= extra;
            }
        }
    }
    if (cls < 0)
        return;   // not reached with the launch's grid (the tile count)
    const int crows = (n - cls + classes - 1) / classes;
    const uint16_t *wc = w + (int64_t)cls * ldw;
    const int64_t cs = (int64_t)classes * ldw;
    const int h = (int)((8u - (unsigned)(((uintptr_t)wc >> 1) & 7u)) & 7u);
    const int ka = min(h, k);                                   // head elements
    const int nvec = ka + 8 <= k ? (k - ka) >> 3 : 0;           // aligned 8-element vectors
    const uint16_t *wb = wc + ka;
    const int full = nvec * 8 / CH;                             // whole chunks
    const int total = (nvec * 8 + CH - 1) / CH;                 // with the ragged one
    const int c_lo = ka == 0 && full > 0 ? 1 : 0;
    int c_hi = full;
    while (c_hi > c_lo && ka + c_hi * CH + 2 > k)
        --c_hi;
    const int dma = c_hi - c_lo;                                // streamed chunks

    // Load side of the stream: row lr of each 8-row group, piece lq of each line.
    const int lr = lane >> 3, lq = (lane & 7) ^ lr;
    const uint16_t *gw[2];
    bool gv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        gv[j] = j0 + 8 * j + lr < crows;
        gw[j] = wb + (int64_t)min(j0 + 8 * j + lr, crows - 1) * cs + 8 * lq;
    }
    const int ri = i16 & 7, hj = i16 >> 3;
    int slot[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
        slot[q] = kLineRows * ri + ((4 * q + g) ^ ri);
    u32x4 (&buf)[kWLoads][kWaveLanes] = stage[wave];

    // B side: x row i16 (past M the last row; those columns are never stored).
    const uint16_t *xb = x + (int64_t)min(i16, m - 1) * ldx;
    const unsigned phase = (unsigned)((((uintptr_t)xb >> 1) + (unsigned)ka) & 1u);
    const unsigned sh = phase * 2u;
    const uint16_t *xw = xb + ka - (int)phase;   // 4-byte aligned

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const int turns = dma > wave ? (dma - wave + kMfmaWaves - 1) / kMfmaWaves : 0;
    const int rot = dma > 0 ? (int)((blockIdx.x * 37u + (unsigned)cls * 11u) % (unsigned)dma) : 0;
    u32x4 xa[2][kU];
    unsigned xe[2][kU];
    auto issue = [&](int i, int sb) {
        int c = wave + i * kMfmaWaves + rot;
        c = (c >= dma ? c - dma : c) + c_lo;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (gv[j]) {
#pragma unroll
                for (int l = 0; l < kLines; ++l)
                    __builtin_amdgcn_global_load_lds(
                        (global_void *)(gw[j] + c * CH + kLineElems * l),
                        (lds_void *)&buf[j * kLines + l][0], 16, 0, 0);
            }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const unsigned *d = reinterpret_cast<const unsigned *>(xw + c * CH + 32 * u + 8 * g);
            xa[sb][u] = *reinterpret_cast<const u32x4_a4 *>(d);
            xe[sb][u] = d[4];
        }
    };

    // Head and tail elements of pair p = (x row p / 16, tile row p % 16); indices clamped,
    // products past the ends dropped.
    const int tail_begin = ka + 8 * nvec;
    const int pidx = wave * kWaveLanes + lane;
    const int pr = pidx & 15, pm = min(pidx >> 4, m - 1);
    const uint16_t *hw = wc + (int64_t)min(j0 + pr, crows - 1) * cs;
    const uint16_t *hx = x + (int64_t)pm * ldx;
    unsigned short hwv[16], hxv[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int kh = min(e, k - 1), kt = min(tail_begin + e, k - 1);
        hwv[e] = hw[kh];
        hxv[e] = hx[kh];
        hwv[8 + e] = hw[kt];
        hxv[8 + e] = hx[kt];
    }
    // The edge and ragged chunks ([0, c_lo) and [c_hi, total), at most 3), one per wave.
    const int nrest = c_lo + (total - c_hi);
    const bool rest = wave < nrest;
    const int rc = wave < c_lo ? wave : c_hi + (wave - c_lo);
    u32x4 ra[kU], rb[kU];
    if (rest) {
        const uint16_t *wa = wb + (int64_t)min(j0 + i16, crows - 1) * cs;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int vc = min(rc * (CH / 8) + 4 * u + g, nvec - 1);
            ra[u] = load_stream(wa + 8 * vc);
            const uint16_t *xv = xb + ka + 8 * vc;
            rb[u].x = (unsigned)xv[0] | ((unsigned)xv[1] << 16);
            rb[u].y = (unsigned)xv[2] | ((unsigned)xv[3] << 16);
            rb[u].z = (unsigned)xv[4] | ((unsigned)xv[5] << 16);
            rb[u].w = (unsigned)xv[6] | ((unsigned)xv[7] << 16);
        }
    }
    if (turns > 0)
        issue(0, 0);
    if (rest) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int v = rc * (CH / 8) + 4 * u + g;
            const u32x4 z = {0, 0, 0, 0};
            acc = mfma(v < nvec ? ra[u] : z, rb[u], acc);
        }
    }
    {
        float es = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < ka)
                es = fmaf(__uint_as_float((unsigned)hwv[e] << 16),
                          __uint_as_float((unsigned)hxv[e] << 16), es);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (tail_begin + e < k)
                es = fmaf(__uint_as_float((unsigned)hwv[8 + e] << 16),
                          __uint_as_float((unsigned)hxv[8 + e] << 16), es);
        if (pidx < 16 * 16)
            edge_sums[pidx] = es;
    }
    // The stream: per chunk the wait for its W lines and x windows, the LDS operand reads,
    // the next chunk's loads (into the other x registers), then the MFMAs.
    auto step = [&](int i, auto sbc) {
        constexpr int sb = decltype(sbc)::value;
        __builtin_amdgcn_s_waitcnt(kWaitVmOnly);
        u32x4 a[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            a[u] = buf[hj * kLines + u / 2][slot[u & 1]];
        __builtin_amdgcn_s_waitcnt(kWaitLgkmOnly);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < turns)
            issue(i + 1, 1 - sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const u32x4 r = xa[sb][u];
            u32x4 b;
            b.x = __builtin_amdgcn_alignbyte(r.y, r.x, sh);
            b.y = __builtin_amdgcn_alignbyte(r.z, r.y, sh);
            b.z = __builtin_amdgcn_alignbyte(r.w, r.z, sh);
            b.w = __builtin_amdgcn_alignbyte(xe[sb][u], r.w, sh);
            acc = mfma(a[u], b, acc);
        }
    };
    for (int i = 0; i < turns; i += 2) {
        step(i, std::integral_constant<int, 0>{});
        if (i + 1 < turns)
            step(i + 1, std::integral_constant<int, 1>{});
    }

    if (wave > 0)
        red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int v = 0; v < kMfmaWaves - 1; ++v)
        acc += red[v][lane];
    if (i16 < m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + 4 * g + e;
            if (j < crows)
                y[(int64_t)i16 * ldy + cls + (int64_t)classes * j] =
                    acc[e] + edge_sums[i16 * 16 + 4 * g + e];
        }
    }
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
    const void *fn;
    if (p->mfma_rows == kMfmaRowsPerBlock)
        fn = reinterpret_cast<const void *>(&gemv_mfma<2, 16, kMfmaChunk>);
    else if (p->mfma_rows == kMfmaNarrowRows && m <= kMfmaNarrowShortX)
        fn = reinterpret_cast<const void *>(&gemv_mfma<1, kMfmaNarrowShortX, kMfmaNarrowChunk>);
    else if (p->mfma_rows == kMfmaNarrowRows)
        fn = reinterpret_cast<const void *>(&gemv_mfma<1, 16, kMfmaNarrowChunk>);
    else
        return GEMV_ERR_INVALID_ARG;
    hipError_t e = hipLaunchKernel(fn,
                                   dim3((unsigned)p->mfma_grid_x, (unsigned)p->mfma_splits),
                                   dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

gemv_status launch_mfma_unaligned(gemv_plan_t p, const gemv_segment &seg, const void *X,
                                  int64_t ldx, void *stream, bool *done)
{
    *done = false;
    if (!p->mfma_unaligned_depth)
        return GEMV_OK;
    // Rows r and r + classes start at the same offset from the 16-byte grid.
    const int r8 = (int)(seg.ldw % 8);
    const int classes = r8 == 0 ? 1 : r8 % 4 == 0 ? 2 : r8 % 2 == 0 ? 4 : 8;
    int64_t tiles = 0;
    for (int c = 0; c < classes; ++c)
        tiles += ((p->n - c + classes - 1) / classes + 15) / 16;
    *done = true;
    const uint16_t *w = static_cast<const uint16_t *>(seg.W);
    const uint16_t *x = static_cast<const uint16_t *>(X);
    float *y = seg.Y;
    int n = (int)p->n, k = (int)p->k, ldw = (int)seg.ldw, ldxi = (int)ldx, ldy = (int)seg.ldy,
        m = p->m, cl = classes;
    void *args[] = {&w, &x, &y, &n, &k, &ldw, &ldxi, &ldy, &m, &cl};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemv_mfma_unaligned),
                                   dim3((unsigned)tiles), dim3(kThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
