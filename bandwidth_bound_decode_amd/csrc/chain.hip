// chain.hip - one persistent launch that runs a decode step's dependent GEMVs in order.
//
// The decode-GEMV page ("Decode GEMV at half of HBM bandwidth", "A strong answer", cause 3)
// and the GPU performance chains page ("Launch gaps in a decode step") locate the loss of a
// decode step between kernels: every GEMV launch pays a start, a first-byte latency and a
// drain, during which HBM idles. On MI355X that is ~3 us per launch, ~0.4 ms over the 129
// GEMVs of a Llama-8B step, even with the launches replayed from one graph.
//
// Here one workgroup per CU walks the whole list. A workgroup is W worker waves and one
// controller wave.
//
// Workers only stream weights. Work items are R rows (R = 1 or 2, chosen per link so that
// items spread evenly) of one link; worker wave v of the grid takes items v, v + V, v + 2V,
// ... of every link (V worker waves in all). An item is read in bursts of 8 16-byte loads
// per lane (8 wave steps of one row, or 4 of each of two rows), and every worker keeps
// kDepth bursts in flight: it issues burst b + kDepth as soon as burst b is consumed,
// whichever item or link burst b + kDepth belongs to. So a worker reaching the end of a link
// already has the next link's weights on the way, and it only stops, to wait for that link's
// input, when it is about to multiply them.
//
// Workers read x from LDS and leave their row results in LDS; they never wait on a global
// memory operation except their own weight loads, so nothing drains their load queue.
//
// The controller does everything that has latency and is not weight streaming: it copies
// each link's x into LDS (direct global-to-LDS loads), writes the workgroup's outputs of a
// link to HBM once all of its workers are done with that link, and arrives on the link's
// grid-wide counter. It then polls that counter until every workgroup has arrived - only then
// is link g complete device-wide, the dependency a real decode step has, since link g + 1's
// input is computed from link g's output - and stages link g + 1's x. One arrival and one
// poller per CU keeps the barrier at a few microseconds (thousands of per-wave arrivals on
// device-scope counters cost tens), and the workers' in-flight bursts cover it.
//
// Counters are never cleared: link g's counter gains one per workgroup per launch, and a
// launch waits for the value (epoch + 1) * workgroups (mod 2^32), where epoch counts the
// finished launches. Every wait is bounded: a wait that runs out sets the error flag, the
// workgroup stops, and the launch's last workgroup puts the counters where a complete launch
// would have left them.
//
// Every output row is summed in the same order as the unsplit gemv_fast kernel sums it
// (lane chain over the row's 16-byte vectors in order, then the same DPP tree), so a chain
// is bitwise equal to running its links one by one with unsplit plans.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

constexpr int kLoads = 8;            // 16-byte loads per lane in one weight burst
constexpr int kDepth = 3;            // weight bursts a worker wave keeps in flight
constexpr int kMaxWorkers = 11;      // worker waves per workgroup (plus one controller)
constexpr int kDefaultWorkers = 8;
constexpr int kCtrlBytes = 256;      // LDS control words, ahead of x
constexpr int kXReadyWord = 32;      // x of link g is staged once this word reaches g + 1
constexpr unsigned kAbort = 0xFFFFFFFFu;
constexpr unsigned kDefaultSpinLimit = 1u << 20;

struct LinkDesc {                    // device-side, one per link, read with scalar loads
    const uint16_t *w[GEMV_MAX_SEGMENTS];
    float *y[GEMV_MAX_SEGMENTS];
    int64_t ldw[GEMV_MAX_SEGMENTS];
    int32_t row0[GEMV_MAX_SEGMENTS];   // first row of each segment; INT32_MAX when unused
    const uint16_t *x;
    int32_t n;                         // rows over all segments
    int32_t k;
    int32_t items;                     // ceil(n / rows)
    int32_t rows;                      // rows per item: 1 or 2
    int32_t nvec;                      // whole 16-byte vectors per row (k / 8)
    int32_t span;                      // wave steps per burst and row: 8 / rows
    int32_t bursts;                    // bursts per item
    int32_t xbytes;                    // LDS bytes of x: the wave steps bursts read (and the
                                       // vector of the k % 8 last elements), zero past k
    int32_t per_wave;                  // most items one worker wave has: ceil(items / V)
    int32_t pad;
};

// The descriptor table is read-only during a launch: reading it through the constant
// address space lets the compiler use scalar loads (and the scalar cache).
typedef __attribute__((address_space(4))) const LinkDesc ConstLink;

struct ChainArgs {
    ConstLink *links;
    unsigned *count;      // [nlinks] workgroup arrivals, modulo 2^32
    unsigned *epoch;      // launches completed so far
    unsigned *finished;   // workgroups of this launch that have finished (zero between launches)
    unsigned *error;      // set when a wait gives up
    int32_t nlinks;
    uint32_t spin_limit;
    int32_t res_offset;   // LDS byte offset of the row results
    int32_t pad;
};

// State words of a chain with `nlinks` links: counters, epoch, finished, error (last).
inline size_t chain_state_words(int nlinks) { return (size_t)nlinks + 3; }

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
typedef __attribute__((address_space(1))) const uint16_t global_u16;
typedef __attribute__((address_space(1))) float global_float;

// s_waitcnt operand with lgkmcnt(0) and the vector-memory and export counts left at their
// maxima: waits for this wave's LDS and scalar operations only.
constexpr int kWaitLgkmOnly = 0xC07F;

// Descriptor pointers are loaded from memory, so the compiler cannot infer their address
// space; casting to the global space keeps the loads global (not flat) loads.
__device__ __forceinline__ u32x4 load_w(const uint16_t *p)
{
    return __builtin_nontemporal_load((global_u32x4 *)p);
}

__device__ __forceinline__ float load_elem(const uint16_t *p)
{
    return bf16_to_f32(*(global_u16 *)p);
}

__device__ __forceinline__ const uint16_t *weight_row(ConstLink *L, int row)
{
    const int j = (row >= L->row0[1]) + (row >= L->row0[2]) + (row >= L->row0[3]);
    return L->w[j] + (int64_t)(row - L->row0[j]) * L->ldw[j];
}

__device__ __forceinline__ unsigned *ctrl(unsigned char *lds)
{
    return reinterpret_cast<unsigned *>(lds);
}

__device__ __forceinline__ unsigned uniform(unsigned v)
{
    return (unsigned)__builtin_amdgcn_readfirstlane((int)v);
}

// Position of a worker wave in its sequence of bursts. All fields are wave-uniform.
struct Cursor {
    int g;          // link; nlinks once the wave has no work left
    int item;       // item of link g
    int t;          // ordinal of that item among this wave's items of link g
    int burst;      // burst within the item
    int n, k, items, rows, nvec, span, bursts;   // of link g
};

// Move to the first link at or after g in which worker wave `gw` has an item.
__device__ __forceinline__ void enter(Cursor &c, ConstLink *links, int nlinks, int g, int gw)
{
    while (g < nlinks && gw >= links[g].items)
        ++g;
    c.g = g;
    c.item = gw;
    c.t = 0;
    c.burst = 0;
    ConstLink *L = links + min(g, nlinks - 1);   // past the end: any link's values will do
    c.n = L->n;
    c.k = L->k;
    c.items = L->items;
    c.rows = L->rows;
    c.nvec = L->nvec;
    c.span = L->span;
    c.bursts = L->bursts;
}

__device__ __forceinline__ void advance(Cursor &c, ConstLink *links, int nlinks, int gw,
                                        int total)
{
    if (c.g >= nlinks)
        return;
    if (++c.burst < c.bursts)
        return;
    c.burst = 0;
    ++c.t;
    c.item += total;
    if (c.item < c.items)
        return;
    enter(c, links, nlinks, c.g + 1, gw);
}

// Issue the 8 weight loads of the burst at cursor c into buf. Loads 0..3 read wave steps
// s0..s0+3 of the item's first row; loads 4..7 read steps s0+4..s0+7 of the same row (one
// row per item) or steps s0..s0+3 of the second row. Lanes past the row's last whole vector
// re-read the row's first vector (in bounds; the consumer zeroes them). Past the wave's last
// burst it re-reads one vector of link 0, so every call issues exactly 8 loads and the wait
// counts the compiler derives stay those of a full pipeline.
__device__ __forceinline__ void issue(u32x4 (&buf)[kLoads], const Cursor &c, ConstLink *links,
                                      int nlinks, int lane)
{
    const uint16_t *lo;
    const uint16_t *hi;
    int v0 = 0, vh = 0, limit = 0;
    bool full = false;
    if (c.g < nlinks) {
        ConstLink *L = links + c.g;
        const int ra = c.item * c.rows;
        lo = weight_row(L, ra);
        hi = c.rows == 1 ? lo : weight_row(L, min(ra + 1, c.n - 1));   // past N: re-read
        const int s0 = c.burst * c.span;
        v0 = s0 * kWaveLanes + lane;
        vh = c.rows == 1 ? v0 + 4 * kWaveLanes : v0;
        limit = c.nvec;
        full = (s0 + c.span) * kWaveLanes <= c.nvec;
    } else {
        lo = hi = links[0].w[0];
    }
    if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            buf[j] = load_w(lo + kVecElems * (v0 + kWaveLanes * j));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            buf[4 + j] = load_w(hi + kVecElems * (vh + kWaveLanes * j));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = v0 + kWaveLanes * j;
            buf[j] = load_w(v < limit ? lo + kVecElems * v : lo);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = vh + kWaveLanes * j;
            buf[4 + j] = load_w(v < limit ? hi + kVecElems * v : hi);
        }
    }
}

// Worker wave w has finished every link before g (its results of those are in LDS).
__device__ __forceinline__ void post_done(unsigned char *lds, int w, int g, int lane)
{
    __builtin_amdgcn_s_waitcnt(kWaitLgkmOnly);   // result writes land before the flag
    if (lane == 0)
        __hip_atomic_store(ctrl(lds) + w, (unsigned)g, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until the controller has staged x of link g. False if the launch is aborting.
__device__ bool wait_x(unsigned char *lds, int g, const ChainArgs &a, int lane)
{
    // The controller's waits are bounded and it always either stages x or aborts, so this
    // bound only guards against the controller itself; it is far longer than those waits.
    const uint64_t limit = 64ull * a.spin_limit;
    for (uint64_t spins = 0;; ++spins) {
        const unsigned v = uniform(__hip_atomic_load(ctrl(lds) + kXReadyWord, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v == kAbort)
            return false;
        if (v >= (unsigned)g + 1)
            return true;
        if (spins >= limit) {
            if (lane == 0)
                __hip_atomic_fetch_or(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Elements past the row's last whole vector (k % 8 of them), after all vectors, as the
// unsplit kernel adds them.
__device__ __forceinline__ void row_tail(const Cursor &c, ConstLink *links, unsigned char *lds,
                                      int lane, float &acc0, float &acc1)
{
    if (lane < (c.k & 7)) {
        ConstLink *L = links + c.g;
        const int kk = kVecElems * c.nvec + lane;
        const int ra = c.item * c.rows;
        const float xv = bf16_to_f32(reinterpret_cast<const uint16_t *>(lds + kCtrlBytes)[kk]);
        acc0 = fmaf(load_elem(weight_row(L, ra) + kk), xv, acc0);
        if (c.rows == 2)
            acc1 = fmaf(load_elem(weight_row(L, min(ra + 1, c.n - 1)) + kk), xv, acc1);
    }
}

// Multiply the burst at cursor c (its loads are in buf) into the accumulators; at the end
// of an item, reduce and leave the item's results in LDS. False if the launch is aborting.
__device__ __forceinline__ bool consume(const u32x4 (&buf)[kLoads], const Cursor &c,
                                        ConstLink *links, const ChainArgs &a,
                                        unsigned char *lds, int lane, int w, int workers,
                                        float &acc0, float &acc1)
{
    if (c.burst == 0 && c.t == 0) {           // this wave's first burst of link c.g
        post_done(lds, w, c.g, lane);
        if (!wait_x(lds, c.g, a, lane))
            return false;
    }
    const int s0 = c.burst * c.span;
    const int v0 = s0 * kWaveLanes + lane;
    const int vh = c.rows == 1 ? v0 + 4 * kWaveLanes : v0;
    u32x4 wv[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
        wv[j] = buf[j];
    if ((s0 + c.span) * kWaveLanes > c.nvec) {   // partial burst: clear re-read lanes
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (v0 + kWaveLanes * j >= c.nvec)
                wv[j] = zero;
            if (vh + kWaveLanes * j >= c.nvec)
                wv[4 + j] = zero;
        }
    }
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(lds + kCtrlBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc0 = dot8(wv[j], xs[v0 + kWaveLanes * j], acc0);
    // loads 4..7 continue row 0 (one row per item) or start row 1; selecting values, not
    // the accumulator's address, keeps both accumulators in registers
    const bool one_row = c.rows == 1;
    float hi = one_row ? acc0 : acc1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        hi = dot8(wv[4 + j], xs[vh + kWaveLanes * j], hi);
    acc0 = one_row ? hi : acc0;
    acc1 = one_row ? acc1 : hi;
    if (c.burst == c.bursts - 1) {
        if (c.k & 7)
            row_tail(c, links, lds, lane, acc0, acc1);
        const float r0 = lane63(wave_sum(acc0));
        const float r1 = lane63(wave_sum(acc1));
        float *res = reinterpret_cast<float *>(lds + a.res_offset) + (c.t * workers + w) * c.rows;
        if (lane == 0) {
            res[0] = r0;
            if (c.rows == 2)
                res[1] = r1;
        }
        acc0 = 0.f;
        acc1 = 0.f;
    }
    return true;
}

__device__ __forceinline__ void worker(const ChainArgs &a, unsigned char *lds, int w,
                                       int workers, int lane)
{
    const int gw = (int)blockIdx.x * workers + w;
    const int total = (int)gridDim.x * workers;
    ConstLink *links = a.links;
    const int nlinks = a.nlinks;
    Cursor p, c;
    enter(p, links, nlinks, 0, gw);
    enter(c, links, nlinks, 0, gw);
    u32x4 buf[kDepth][kLoads];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        issue(buf[d], p, links, nlinks, lane);
        advance(p, links, nlinks, gw, total);
    }
    float acc0 = 0.f, acc1 = 0.f;
    bool ok = true;
    // The loop's only exit is at the end of the unrolled body. (An exit in the middle is
    // routed through the loop's back edge by the compiler's control-flow structurizer, and
    // on that path fewer loads are in flight, so the compiler would wait for all of them at
    // the top of every iteration.) A burst slot past the end, or after an abort, is skipped
    // but still refilled.
    for (;;) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (ok && c.g < nlinks) {
                ok = consume(buf[d], c, links, a, lds, lane, w, workers, acc0, acc1);
                advance(c, links, nlinks, gw, total);
            }
            issue(buf[d], p, links, nlinks, lane);
            advance(p, links, nlinks, gw, total);
        }
        if (!ok || c.g >= nlinks)
            break;
    }
    if (ok)
        post_done(lds, w, nlinks, lane);
}

// Copy x of link L into LDS: whole vectors with direct global-to-LDS loads, zeros up to the
// staged length, then the k % 8 trailing elements.
__device__ void stage_x(ConstLink *L, unsigned char *lds, int lane)
{
    const uint16_t *x = L->x;
    const int nv = L->nvec;
    const int k = L->k;
    const int staged = L->xbytes / 16;
    unsigned char *xs = lds + kCtrlBytes;
    for (int c = 0; c * kWaveLanes < nv; ++c) {
        const int v = c * kWaveLanes + lane;
        if (v < nv)
            __builtin_amdgcn_global_load_lds(
                (__attribute__((address_space(1))) void *)(x + kVecElems * v),
                (__attribute__((address_space(3))) void *)(xs + c * kWaveLanes * 16), 16, 0, 0);
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int v = nv + lane; v < staged; v += kWaveLanes)
        reinterpret_cast<u32x4 *>(xs)[v] = zero;
    __builtin_amdgcn_s_waitcnt(0);
    const int rem = k & 7;
    if (rem) {
        if (lane < rem)
            reinterpret_cast<uint16_t *>(xs)[kVecElems * nv + lane] =
                *(global_u16 *)(x + kVecElems * nv + lane);
        __builtin_amdgcn_s_waitcnt(0);
    }
}

// Wait until every worker wave of this workgroup has finished links before `need`. LDS
// polls are short, so this wait allows 16 times as many as the grid-wide one.
__device__ bool wait_workers(unsigned char *lds, unsigned need, int workers, int lane,
                             uint32_t spin_limit)
{
    const uint64_t limit = 16ull * spin_limit;
    for (uint64_t spins = 0;; ++spins) {
        const unsigned v = lane < workers
                               ? __hip_atomic_load(ctrl(lds) + lane, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP)
                               : need;
        if (__ballot(v < need) == 0)
            return true;
        if (spins >= limit)
            return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Wait until every workgroup has arrived on a link counter. The counter's value before
// this launch's arrivals was target - workgroups.
__device__ bool wait_grid(const unsigned *count, unsigned target, unsigned workgroups,
                          uint32_t spin_limit)
{
    const unsigned before = target - workgroups;
    for (uint32_t spins = 0;; ++spins) {
        const unsigned v = uniform(
            __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v - before >= workgroups)
            return true;
        if (spins >= spin_limit)
            return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Write this workgroup's row results of link L to the outputs. Result e of the LDS buffer
// belongs to the wave's item ordinal t = e / (W * rows), worker w and row r of the item.
__device__ void store_results(ConstLink *L, const float *res, int lane, int wg, int workers,
                              int total)
{
    const int rows = L->rows;
    const int n = L->n;
    const int items = L->items;
    const int per = workers * rows;
    const int cnt = L->per_wave * per;
    const int r1 = L->row0[1], r2 = L->row0[2], r3 = L->row0[3];
    for (int e = lane; e < cnt; e += kWaveLanes) {
        const int t = e / per;
        const int wr = e - t * per;
        const int w = rows == 1 ? wr : wr >> 1;
        const int item = wg * workers + w + t * total;
        const int row = item * rows + (wr - w * rows);
        if (item < items && row < n) {
            float *y = L->y[0];
            int base = 0;
            if (row >= r1) { y = L->y[1]; base = r1; }
            if (row >= r2) { y = L->y[2]; base = r2; }
            if (row >= r3) { y = L->y[3]; base = r3; }
            __hip_atomic_store((global_float *)(y + (row - base)), res[e], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__device__ __forceinline__ void controller(const ChainArgs &a, unsigned char *lds, int workers,
                                           int lane)
{
    const unsigned wgs = gridDim.x;
    const int wg = (int)blockIdx.x;
    const int total = (int)wgs * workers;
    const int nlinks = a.nlinks;
    const unsigned epoch = uniform(
        __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const unsigned target = (epoch + 1u) * wgs;
    unsigned *xready = ctrl(lds) + kXReadyWord;
    const float *res = reinterpret_cast<const float *>(lds + a.res_offset);
    bool ok = true;
    stage_x(a.links, lds, lane);
    if (lane == 0)
        __hip_atomic_store(xready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int g = 0; g < nlinks; ++g) {
        if (!wait_workers(lds, (unsigned)g + 1, workers, lane, a.spin_limit)) {
            ok = false;
            break;
        }
        store_results(a.links + g, res, lane, wg, workers, total);
        __builtin_amdgcn_s_waitcnt(0);         // outputs of link g are stored
        if (lane == 0)
            __hip_atomic_fetch_add(a.count + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (g + 1 == nlinks)
            break;
        if (!wait_grid(a.count + g, target, wgs, a.spin_limit)) {
            ok = false;
            break;
        }
        stage_x(a.links + g + 1, lds, lane);
        if (lane == 0)
            __hip_atomic_store(xready, (unsigned)g + 2, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (!ok && lane == 0) {
        __hip_atomic_fetch_or(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(xready, kAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // The last workgroup of the launch advances the epoch. After a timeout some counters
    // hold partial arrivals, so it sets them to the values a complete launch leaves.
    __builtin_amdgcn_s_waitcnt(0);
    unsigned t = 0;
    if (lane == 0)
        t = __hip_atomic_fetch_add(a.finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t = uniform(t);
    if (t == wgs - 1) {
        const unsigned failed = uniform(
            __hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (failed)
            for (int i = lane; i < nlinks; i += kWaveLanes)
                __hip_atomic_store(a.count + i, target, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) {
            __hip_atomic_store(a.epoch, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ void __launch_bounds__((kMaxWorkers + 1) * kWaveLanes) gemv_chain_kernel(ChainArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int lane = (int)(threadIdx.x & (kWaveLanes - 1));
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWaveLanes));
    const int workers = (int)(blockDim.x / kWaveLanes) - 1;
    if (threadIdx.x < kCtrlBytes / 4)
        ctrl(lds)[threadIdx.x] = 0u;
    __syncthreads();
    if (wave == workers)
        controller(a, lds, workers, lane);
    else
        worker(a, lds, wave, workers, lane);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Rows per item for a link: the one that gives the fewest bursts to the busiest worker
// wave (ties: one row, the longer run of steps per burst).
void choose_rows(LinkDesc &d, int64_t total)
{
    int64_t best = -1;
    for (int rows = 1; rows <= 2; ++rows) {
        const int span = kLoads / rows;
        const int64_t items = ceil_div(d.n, rows);
        const int64_t bursts = ceil_div(ceil_div(d.nvec, kWaveLanes), span);
        const int64_t cost = ceil_div(items, total) * bursts;
        if (best < 0 || cost < best) {
            best = cost;
            d.rows = rows;
            d.span = span;
            d.items = (int32_t)items;
            d.bursts = (int32_t)bursts;
            d.per_wave = (int32_t)ceil_div(items, total);
            // every wave step a burst reads, and the vector holding the k % 8 last elements
            const int64_t xvec = std::max<int64_t>(bursts * span * kWaveLanes,
                                                   ceil_div(d.k, kVecElems));
            d.xbytes = (int32_t)(xvec * 16);
        }
    }
}

}  // namespace

struct gemv_chain_s {
    int device;
    LinkDesc *d_links;
    unsigned *d_state;     // counters, epoch, finished, error
    int nlinks;
    int grid;
    int block;
    size_t lds;
    int res_offset;
    unsigned spin_limit;
};

extern "C" gemv_status gemv_chain_create(gemv_chain_t *out, const gemv_chain_link *links,
                                         int nlinks, int device, const gemv_chain_opts *opts)
{
    if (!out)
        return GEMV_ERR_INVALID_ARG;
    *out = nullptr;
    if (!links || nlinks < 1 || device < 0)
        return GEMV_ERR_INVALID_ARG;
    gemv_chain_opts o = {0, 0};
    if (opts)
        o = *opts;
    const int workers = o.waves_per_cu ? o.waves_per_cu : kDefaultWorkers;
    if (workers < 1 || workers > kMaxWorkers)
        return GEMV_ERR_INVALID_ARG;

    std::vector<LinkDesc> host((size_t)nlinks);
    for (int i = 0; i < nlinks; ++i) {
        const gemv_chain_link &l = links[i];
        if (!l.segs || l.nseg < 1 || l.nseg > GEMV_MAX_SEGMENTS || !l.X || l.k < kVecElems ||
            l.k > ((int64_t)1 << 24))
            return GEMV_ERR_INVALID_ARG;
        LinkDesc &d = host[(size_t)i];
        memset(&d, 0, sizeof d);
        int64_t rows = 0;
        for (int j = 0; j < GEMV_MAX_SEGMENTS; ++j) {
            if (j < l.nseg) {
                const gemv_segment &s = l.segs[j];
                if (!s.W || !s.Y || s.n < 1 || s.ldw < l.k)
                    return GEMV_ERR_INVALID_ARG;
                if (!aligned16(s.W) || s.ldw % 8 != 0 || !aligned4(s.Y))
                    return GEMV_ERR_MISALIGNED;
                d.w[j] = static_cast<const uint16_t *>(s.W);
                d.y[j] = s.Y;
                d.ldw[j] = s.ldw;
                d.row0[j] = (int32_t)rows;
                rows += s.n;
                if (rows > ((int64_t)1 << 30))
                    return GEMV_ERR_INVALID_ARG;
            } else {
                d.w[j] = d.w[0];
                d.y[j] = d.y[0];
                d.ldw[j] = d.ldw[0];
                d.row0[j] = INT32_MAX;
            }
        }
        if (!aligned16(l.X))
            return GEMV_ERR_MISALIGNED;
        d.x = static_cast<const uint16_t *>(l.X);
        d.n = (int32_t)rows;
        d.k = (int32_t)l.k;
        d.nvec = (int32_t)(l.k / kVecElems);
    }

    int prev = 0;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_DEVICE);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_DEVICE);
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return record_hip_error(0, GEMV_ERR_DEVICE);

    // One workgroup per CU. Its LDS holds the control words, the longest staged x and the
    // largest per-link result buffer; asking for more than half of a CU's LDS keeps the
    // dispatcher from placing two workgroups on one CU.
    const int64_t total = (int64_t)prop.multiProcessorCount * workers;
    size_t xcap = 0, rcap = 0;
    for (LinkDesc &d : host) {
        choose_rows(d, total);
        xcap = std::max(xcap, (size_t)d.xbytes);
        rcap = std::max(rcap, (size_t)d.per_wave * workers * d.rows * sizeof(float));
    }
    size_t lds = kCtrlBytes + xcap + rcap;
    const size_t half = (size_t)prop.maxSharedMemoryPerMultiProcessor / 2 + 16;
    if (lds < half && half <= prop.sharedMemPerBlock)
        lds = half;
    lds = (lds + 15) & ~(size_t)15;
    if (lds > prop.sharedMemPerBlock)
        return GEMV_ERR_INVALID_ARG;   // x of some link does not fit in LDS

    e = hipSetDevice(device);
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_DEVICE);
    const int block = (workers + 1) * kWaveLanes;
    gemv_chain_s *c = nullptr;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_chain_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    // Every workgroup must be resident at once (they wait on each other).
    int per_cu = 0;
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&gemv_chain_kernel), block, lds);
    if (e == hipSuccess && per_cu < 1)
        e = hipErrorInvalidConfiguration;
    if (e == hipSuccess) {
        c = new (std::nothrow) gemv_chain_s;
        if (!c) {
            (void)hipSetDevice(prev);
            return GEMV_ERR_INVALID_ARG;
        }
        memset(c, 0, sizeof *c);
        c->device = device;
        c->nlinks = nlinks;
        c->grid = prop.multiProcessorCount;
        c->block = block;
        c->lds = lds;
        c->res_offset = (int)(kCtrlBytes + xcap);
        c->spin_limit = o.spin_limit ? o.spin_limit : kDefaultSpinLimit;
        e = hipMalloc(&c->d_links, sizeof(LinkDesc) * (size_t)nlinks);
    }
    if (e == hipSuccess)
        e = hipMalloc(&c->d_state, sizeof(unsigned) * chain_state_words(nlinks));
    if (e == hipSuccess)
        e = hipMemcpy(c->d_links, host.data(), sizeof(LinkDesc) * (size_t)nlinks,
                      hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemset(c->d_state, 0, sizeof(unsigned) * chain_state_words(nlinks));
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        gemv_chain_destroy(c);
        return record_hip_error((int)e, GEMV_ERR_DEVICE);
    }
    *out = c;
    return GEMV_OK;
}

extern "C" gemv_status gemv_chain_run(gemv_chain_t c, void *stream)
{
    if (!c)
        return GEMV_ERR_INVALID_ARG;
    ChainArgs a;
    memset(&a, 0, sizeof a);
    a.links = (ConstLink *)c->d_links;
    a.count = c->d_state;
    a.epoch = a.count + c->nlinks;
    a.finished = a.epoch + 1;
    a.error = a.finished + 1;
    a.nlinks = c->nlinks;
    a.spin_limit = c->spin_limit;
    a.res_offset = c->res_offset;
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemv_chain_kernel),
                                   dim3((unsigned)c->grid), dim3((unsigned)c->block), args,
                                   c->lds, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_DEVICE);
    return GEMV_OK;
}

extern "C" gemv_status gemv_chain_check(gemv_chain_t c)
{
    if (!c)
        return GEMV_ERR_INVALID_ARG;
    int prev = 0;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess)
        e = hipSetDevice(c->device);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    unsigned flag = 0;
    unsigned *err = c->d_state + chain_state_words(c->nlinks) - 1;
    if (e == hipSuccess)
        e = hipMemcpy(&flag, err, sizeof flag, hipMemcpyDeviceToHost);
    if (e == hipSuccess && flag)
        e = hipMemset(err, 0, sizeof flag);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    (void)hipSetDevice(prev);
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_DEVICE);
    return flag ? GEMV_ERR_TIMEOUT : GEMV_OK;
}

extern "C" void gemv_chain_destroy(gemv_chain_t c)
{
    if (!c)
        return;
    int prev = 0;
    bool restore = hipGetDevice(&prev) == hipSuccess && hipSetDevice(c->device) == hipSuccess;
    if (c->d_links)
        (void)hipFree(c->d_links);
    if (c->d_state)
        (void)hipFree(c->d_state);
    if (restore)
        (void)hipSetDevice(prev);
    delete c;
}
