// calib.hip - the pure-read streaming kernel used to measure the achievable HBM read rate and
// the loaded memory latency on this part (gemv_read_stream in gemv.h).
//
// It is the batch-1 GEMV's weight stream with everything else taken out: one single-wave
// workgroup per row, lane l reading the 16-byte vectors l, l + 64, ... of its row in bursts
// of U loads issued before any is used, nontemporal like the weights, no x, no arithmetic
// beyond folding the words together, no stores. Over a buffer far larger than the caches
// its rate is the ceiling the GEMV can approach; swept over U and resident waves per CU it
// gives bandwidth against bytes in flight, whose linear part is Little's law with the
// loaded latency as the slope (decode-GEMV page, "A strong answer"; GPU performance chains
// page, "Bytes in flight to reach bandwidth").
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

constexpr unsigned kNeverFolded = 0x9E3779B9u;   // stored only if the fold equals it

template <int U>
__global__ void __launch_bounds__(64) read_stream(const uint16_t *buf, int steps, int64_t ld,
                                                  unsigned *sink)
{
    const int lane = threadIdx.x & 63;
    const uint16_t *row = buf + (int64_t)blockIdx.x * ld;
    unsigned acc = 0;
    for (int s = 0; s < steps; s += U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_stream(row + kVecElems * (lane + kWaveLanes * (s + u)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == kNeverFolded)
        *sink = acc;
}

const void *find_read(int u)
{
    switch (u) {
    case 1: return reinterpret_cast<const void *>(&read_stream<1>);
    case 2: return reinterpret_cast<const void *>(&read_stream<2>);
    case 4: return reinterpret_cast<const void *>(&read_stream<4>);
    case 8: return reinterpret_cast<const void *>(&read_stream<8>);
    default: return nullptr;
    }
}

}  // namespace

extern "C" gemv_status gemv_read_stream(const void *buf, int64_t rows, int64_t row_bytes,
                                        int unroll, int waves_per_cu, unsigned *sink,
                                        void *stream)
{
    const void *fn = find_read(unroll);
    if (!buf || !sink || !fn || rows < 1 || rows > INT32_MAX || row_bytes < 1 ||
        row_bytes % ((int64_t)kWaveLanes * 16 * unroll) != 0 ||
        row_bytes / 2 / kWaveStep > INT32_MAX || waves_per_cu < 0 ||
        waves_per_cu > kMaxWavesPerCU)
        return GEMV_ERR_INVALID_ARG;
    if (((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u))
        return GEMV_ERR_MISALIGNED;
    // At most waves_per_cu single-wave workgroups per CU: the smallest LDS reservation per
    // workgroup that admits that many and no more (as the GEMV plans' caps do).
    size_t lds = 0;
    if (waves_per_cu > 0 && waves_per_cu < kMaxWavesPerCU)
        lds = ((size_t)kLdsPerCU / (size_t)(waves_per_cu + 1) / 512 + 1) * 512;
    if (lds > 64 * 1024) {
        static std::atomic<bool> raised[9];
        if (!raised[unroll].load(std::memory_order_acquire)) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kLdsPerCU / 2 + 1024);
            if (e != hipSuccess)
                return record_hip_error((int)e, GEMV_ERR_DEVICE);
            raised[unroll].store(true, std::memory_order_release);
        }
    }
    const uint16_t *b = static_cast<const uint16_t *>(buf);
    int steps = (int)(row_bytes / 2 / kWaveStep);
    int64_t ld = row_bytes / 2;
    void *args[] = {&b, &steps, &ld, &sink};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)rows), dim3(kWaveLanes), args, lds,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}
