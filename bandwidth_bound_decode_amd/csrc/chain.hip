// chain.hip - one persistent launch that runs a decode step's dependent GEMVs in order.
//
// The decode-GEMV page ("Decode GEMV at half of HBM bandwidth", "A strong answer", cause 3)
// and the GPU performance chains page ("Launch gaps in a decode step") locate the loss of a
// decode step between kernels: every GEMV launch pays a start, a first-byte latency and a
// drain, during which HBM idles. On MI355X that is ~3 us per launch, ~0.4 ms over the 129
// GEMVs of a Llama-8B step, even with the launches replayed from one graph.
//
// Here one grid of resident waves walks the whole list. Work items are R rows of one link;
// wave w takes items w, w + W, w + 2W, ... of every link, so every wave moves through the
// links in order. Before computing its first item of link g a wave waits until all of link
// g-1 is done - the dependency a real decode step has, since link g's input is computed
// from link g-1's output - but it issues that item's first burst of weight loads before it
// waits: weights never depend on the previous result, so HBM keeps streaming across the
// link boundary instead of draining and refilling.
//
// Link completion is a two-level arrival tree with spread addresses, because thousands of
// waves hitting one device-coherent counter serialise on it (measured: ~70 us per link).
// After its last item of link g (and after its output stores completed) every wave adds 1 to
// one of kSlots slot counters; the wave that completes a slot adds 1 to the link's
// second-level counter; the wave that completes that one writes the link's kReleases
// release flags. A waiting wave polls one release flag, shared by few waves. Counters reset
// themselves (the wave that completes one zeroes it) and release flags hold the launch's
// epoch number, so nothing needs clearing between launches or graph replays. A dependency
// wait polls with a bound: a wait that runs out sets the error flag and the wave stops, so
// the launch always ends; the last wave of such a launch clears the counters.
//
// Every output row is summed in the same order as the unsplit gemv_fast kernel sums it
// (lane chain over the row's 16-byte vectors in order, then the same DPP tree), so a chain
// is bitwise equal to running its links one by one with unsplit plans.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

// Tile of a link (batch 1): rows per item R and loads per burst U. Rows of up to 8 wave
// steps are one burst of 8 for a single-row item; longer rows go two per item in bursts of
// 4, as in the standalone kernel's measured defaults.
constexpr int32_t kTileShort = 0;   // R = 1, U = 8
constexpr int32_t kTileLong = 1;    // R = 2, U = 4

struct LinkDesc {                    // device-side, one per link, read with scalar loads
    const uint16_t *w[GEMV_MAX_SEGMENTS];
    float *y[GEMV_MAX_SEGMENTS];
    int64_t ldw[GEMV_MAX_SEGMENTS];
    int32_t row0[GEMV_MAX_SEGMENTS];   // first row of each segment; INT32_MAX when unused
    const uint16_t *x;
    int32_t n;                         // rows over all segments
    int32_t k;
    int32_t items;                     // ceil(n / R)
    int32_t tile;
    int32_t pad[2];
};

// The descriptor table is read-only during a launch: reading it through the constant
// address space lets the compiler use scalar loads (and the scalar cache) for the uniform
// accesses, instead of vector loads in front of every item's first weight load.
typedef __attribute__((address_space(4))) const LinkDesc ConstLink;

constexpr int kSlots = 64;      // first-level arrival counters per link
constexpr int kReleases = 64;   // release flags per link (each polled by W / 64 waves)

struct ChainArgs {
    ConstLink *links;
    unsigned *slots;      // [nlinks][kSlots] first-level arrivals (zero between launches)
    unsigned *level2;     // [nlinks] completed slots (zero between launches)
    unsigned *release;    // [nlinks][kReleases] epoch + 1 once link g is complete
    unsigned *epoch;      // launches completed so far
    unsigned *finished;   // waves of this launch that have finished (zero between launches)
    unsigned *error;      // set when a dependency wait gives up
    int32_t nlinks;
    uint32_t spin_limit;
};

// State words of a chain with `nlinks` links: slots, level2, release flags, epoch,
// finished, error.
inline size_t chain_state_words(int nlinks)
{
    return (size_t)nlinks * (kSlots + 1 + kReleases) + 3;
}

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
typedef __attribute__((address_space(1))) float global_float;

// Descriptor pointers are loaded from memory, so the compiler cannot infer their address
// space; casting to the global space keeps the loads global (not flat) loads.
__device__ __forceinline__ u32x4 load_w(const uint16_t *p)
{
    return __builtin_nontemporal_load((global_u32x4 *)p);
}

__device__ __forceinline__ u32x4 load_x(const uint16_t *p) { return *(global_u32x4 *)p; }

__device__ __forceinline__ float load_elem(const uint16_t *p)
{
    return bf16_to_f32(*(__attribute__((address_space(1))) const uint16_t *)p);
}

__device__ __forceinline__ int segment_of(ConstLink *L, int row)
{
    return (row >= L->row0[1]) + (row >= L->row0[2]) + (row >= L->row0[3]);
}

__device__ __forceinline__ const uint16_t *weight_row(ConstLink *L, int row)
{
    const int j = segment_of(L, row);
    return L->w[j] + (int64_t)(row - L->row0[j]) * L->ldw[j];
}

__device__ __forceinline__ global_float *output_of(ConstLink *L, int row)
{
    const int j = segment_of(L, row);
    return (global_float *)(L->y[j] + (row - L->row0[j]));
}

// Wait until link g-1 has completed. Uniform across the wave. False if the wait gave up.
__device__ bool wait_for_link(const ChainArgs &a, int g, int wave, int lane, unsigned epoch)
{
    const unsigned *flag = a.release + (size_t)(g - 1) * kReleases + (wave % kReleases);
    for (unsigned spins = 0;; ++spins) {
        unsigned v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)__builtin_amdgcn_readfirstlane((int)v) == epoch + 1)
            return true;
        if (spins >= a.spin_limit) {
            if (lane == 0)
                __hip_atomic_fetch_or(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(4);
    }
}

// This wave is done with link g (its output stores have completed): arrive on the tree.
__device__ __forceinline__ void arrive(const ChainArgs &a, int g, int wave, int waves, int lane,
                                       unsigned epoch)
{
    __builtin_amdgcn_s_waitcnt(0);
    if (lane != 0)
        return;
    const int slot = wave % kSlots;
    const unsigned in_slot = (unsigned)(waves / kSlots + (slot < waves % kSlots ? 1 : 0));
    unsigned *slot_word = a.slots + (size_t)g * kSlots + slot;
    const unsigned old = __hip_atomic_fetch_add(slot_word, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 != in_slot)
        return;
    __hip_atomic_store(slot_word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned used = (unsigned)(waves < kSlots ? waves : kSlots);
    const unsigned old2 = __hip_atomic_fetch_add(a.level2 + g, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (old2 + 1 != used)
        return;
    __hip_atomic_store(a.level2 + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = 0; i < kReleases; ++i)
        __hip_atomic_store(a.release + (size_t)g * kReleases + i, epoch + 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// One item: rows [item * R, item * R + R) of link L. With `wait_first` the item's first
// burst of weight loads is issued, then the wave waits for link g-1, then it loads x.
template <int R, int U>
__device__ __forceinline__ bool chain_item(const ChainArgs &a, ConstLink *L, int item,
                                           int lane, bool wait_first, int g, int wave,
                                           unsigned epoch)
{
    const int n = L->n;
    const int k = L->k;
    const int row_first = item * R;
    const uint16_t *wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        wrow[r] = weight_row(L, min(row_first + r, n - 1));   // past N: re-read row N-1
    const uint16_t *xk = L->x;
    const int nvec = k >> 3;
    const int rem = k & 7;
    const int full = nvec >> 6;

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.f;

    int step = 0;
    {
        // First burst: weight loads go out before the dependency wait.
        const int cnt = min(U, full);
        u32x4 wv[U][R];
        u32x4 xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < cnt)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    wv[u][r] = load_w(wrow[r] + 8 * (lane + 64 * u));
        __builtin_amdgcn_sched_barrier(0);
        if (wait_first && !wait_for_link(a, g, wave, lane, epoch))
            return false;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < cnt)
                xv[u] = load_x(xk + 8 * (lane + 64 * u));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < cnt)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[r] = dot8(wv[u][r], xv[u], acc[r]);
        step = cnt;
    }
    for (; step + U <= full; step += U) {
        u32x4 wv[U][R];
        u32x4 xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[u][r] = load_w(wrow[r] + 8 * (lane + 64 * (step + u)));
#pragma unroll
        for (int u = 0; u < U; ++u)
            xv[u] = load_x(xk + 8 * (lane + 64 * (step + u)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = dot8(wv[u][r], xv[u], acc[r]);
    }
    if (step < full) {
        const int rest = full - step;
        u32x4 wv[U][R];
        u32x4 xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < rest)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    wv[u][r] = load_w(wrow[r] + 8 * (lane + 64 * (step + u)));
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < rest)
                xv[u] = load_x(xk + 8 * (lane + 64 * (step + u)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < rest)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[r] = dot8(wv[u][r], xv[u], acc[r]);
    }
    const int v_last = lane + 64 * full;
    if (v_last < nvec) {
        const u32x4 xv = load_x(xk + 8 * v_last);
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = dot8(load_w(wrow[r] + 8 * v_last), xv, acc[r]);
    }
    if (lane < rem) {
        const int kk = 8 * nvec + lane;
        const float xs = load_elem(xk + kk);
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = fmaf(load_elem(wrow[r] + kk), xs, acc[r]);
    }
    float out = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s = lane63(wave_sum(acc[r]));
        if (lane == r)
            out = s;
    }
    if (lane < R && row_first + lane < n)
        __hip_atomic_store(output_of(L, row_first + lane), out, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

__global__ void __launch_bounds__(64) gemv_chain_kernel(ChainArgs a)
{
    const int lane = threadIdx.x;
    const int wave = blockIdx.x;
    const int waves = gridDim.x;
    const unsigned epoch = (unsigned)__builtin_amdgcn_readfirstlane(
        (int)__hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    bool ok = true;
    for (int g = 0; g < a.nlinks && ok; ++g) {
        ConstLink *L = a.links + g;
        const int items = L->items;
        const bool tile_short = L->tile == kTileShort;
        bool first = g > 0;      // the first item of a link waits for the previous link
        for (int item = wave; item < items; item += waves) {
            ok = tile_short ? chain_item<1, 8>(a, L, item, lane, first, g, wave, epoch)
                            : chain_item<2, 4>(a, L, item, lane, first, g, wave, epoch);
            if (!ok)
                break;
            first = false;
        }
        if (ok)
            arrive(a, g, wave, waves, lane, epoch);
    }
    // The last wave of the launch advances the epoch. After a timeout the counters may hold
    // partial arrivals, so it clears them too (all 64 lanes, only on that path).
    __builtin_amdgcn_s_waitcnt(0);
    unsigned t = 0;
    if (lane == 0)
        t = __hip_atomic_fetch_add(a.finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t = (unsigned)__builtin_amdgcn_readfirstlane((int)t);
    if (t == (unsigned)waves - 1) {
        const unsigned failed = (unsigned)__builtin_amdgcn_readfirstlane(
            (int)__hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (failed) {
            const size_t n = (size_t)a.nlinks * (kSlots + 1);   // slots and level2
            for (size_t i = lane; i < n; i += 64)
                __hip_atomic_store(a.slots + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) {
            __hip_atomic_store(a.epoch, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

constexpr int kDefaultWavesPerCU = 8;
constexpr unsigned kDefaultSpinLimit = 1u << 20;   // ~1 s of polling

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

struct gemv_chain_s {
    int device;
    LinkDesc *d_links;
    unsigned *d_state;     // slots, level2, release flags, epoch, finished, error
    int nlinks;
    int grid;
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
    if (o.waves_per_cu < 0)
        return GEMV_ERR_INVALID_ARG;

    std::vector<LinkDesc> host((size_t)nlinks);
    int64_t items_total = 0;
    for (int i = 0; i < nlinks; ++i) {
        const gemv_chain_link &l = links[i];
        if (!l.segs || l.nseg < 1 || l.nseg > GEMV_MAX_SEGMENTS || !l.X || l.k < 1 ||
            l.k > ((int64_t)1 << 30))
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
        const int64_t steps = (l.k + kWaveStep - 1) / kWaveStep;
        const int r = steps <= 8 ? 1 : 2;
        d.x = static_cast<const uint16_t *>(l.X);
        d.n = (int32_t)rows;
        d.k = (int32_t)l.k;
        d.tile = steps <= 8 ? kTileShort : kTileLong;
        d.items = (int32_t)((rows + r - 1) / r);
        items_total += d.items;
        if (items_total > INT32_MAX / 2)
            return GEMV_ERR_INVALID_ARG;
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
    e = hipSetDevice(device);
    if (e != hipSuccess)
        return record_hip_error((int)e, GEMV_ERR_DEVICE);

    // Every wave of the grid must be resident at once (waves wait on each other), so the
    // grid never exceeds what the occupancy calculator says fits.
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(&gemv_chain_kernel), 64, 0);
    int want = o.waves_per_cu ? o.waves_per_cu : kDefaultWavesPerCU;
    gemv_chain_s *c = nullptr;
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
        c->grid = prop.multiProcessorCount * (want < per_cu ? want : per_cu);
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
    const size_t n = (size_t)c->nlinks;
    a.links = (ConstLink *)c->d_links;
    a.slots = c->d_state;
    a.level2 = a.slots + n * kSlots;
    a.release = a.level2 + n;
    a.epoch = a.release + n * kReleases;
    a.finished = a.epoch + 1;
    a.error = a.finished + 1;
    a.nlinks = c->nlinks;
    a.spin_limit = c->spin_limit;
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemv_chain_kernel),
                                   dim3((unsigned)c->grid), dim3(64), args, 0,
                                   static_cast<hipStream_t>(stream));
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
