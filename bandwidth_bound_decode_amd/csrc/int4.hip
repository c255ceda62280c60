// int4.hip - batch-1 GEMV with INT4 weights, dequantized in registers.
//
// The decode-GEMV page's INT4 follow-up: a quarter of the weight bytes, so the same kernel
// needs proportionally fewer bytes in flight, but every byte now needs unpacking, and that
// must happen while the next loads are outstanding. Format (signed two's-complement nibbles,
// element k in the low nibble of byte k/2 when k is even, one bf16 scale per 128 elements
// of a row) is the one declared in gemv.h.
//
// A wave owns R rows: lane l takes the 16-byte packed vectors l, l + 64, ... of each (32
// weights each, inside one 128-element group), issuing U of them per row, their group
// scales and the four 16-byte x vectors they meet before using any. Every x vector serves
// R rows, and when x fits (2K bytes <= 64 KiB) the workgroup stages it in LDS first, so the
// vector-memory path carries weights and scales only: x is 4 bytes per packed weight byte,
// and loading it per wave measured up to 1.5x slower (probe sweep at the Llama shapes).
// Per 32-bit word (8 weights):
//   - (word << 4) & 0xF0F0F0F0 puts the even-indexed nibbles, and word & 0xF0F0F0F0 the
//     odd-indexed ones, in the top half of a byte each; read as a signed byte that is 16 v,
//     exactly;
//   - each signed byte converts to fp32 (one instruction with a byte select), and the top
//     halves of two such floats are the bf16 pair (16 v_2i, 16 v_2i+1), exactly, which
//     v_dot2c_f32_bf16 multiplies by the x pair (x_2i, x_2i+1);
// so the 32 products of a vector form one fp32 chain, p = sum 16 v x, and the group scale
// then enters once: acc = fma(p, scale / 16, acc). No product is formed inexactly (16 v has
// 4 significant bits, x 8) and no offset is subtracted after the fact, so the error analysis
// of the bf16 path carries over unchanged.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

// bf16 pair (16 v_2i, 16 v_2i+1) for pair i of a packed word, from its even/odd bytes.
template <int I>
__device__ __forceinline__ unsigned int4_pair(unsigned even, unsigned odd)
{
    const float lo = (float)(int8_t)(even >> (8 * I));
    const float hi = (float)(int8_t)(odd >> (8 * I));
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// p + sum of the 8 products of packed word d with the x vector half xd (4 bf16 pairs).
__device__ __forceinline__ float int4_dot8(unsigned d, u32x4 xd, float p)
{
    const unsigned even = (d << 4) & 0xF0F0F0F0u;
    const unsigned odd = d & 0xF0F0F0F0u;
    const unsigned x0 = xd.x, x1 = xd.y, x2 = xd.z, x3 = xd.w;
    p = dot2(int4_pair<0>(even, odd), x0, p);
    p = dot2(int4_pair<1>(even, odd), x1, p);
    p = dot2(int4_pair<2>(even, odd), x2, p);
    p = dot2(int4_pair<3>(even, odd), x3, p);
    return p;
}

// U vectors per lane per burst; R rows per wave (sharing every x vector); XLDS: the
// workgroup first copies x (2K bytes) into LDS and the waves read it from there, which takes
// the x traffic (four 16-byte x vectors per 16-byte weight vector) off the vector-memory
// path. The rows of a workgroup are consecutive: wave w owns rows R*(blockIdx.x*waves + w)
// and on.
template <int U, int R, bool XLDS>
__global__ void __launch_bounds__(512)
    gemv_int4(const uint8_t *wq, const uint16_t *scales, const uint16_t *x, float *y, int n,
              int vecs, int ldq, int lds)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char xs[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int waves = (int)(blockDim.x >> 6);
    const int row0 = (blockIdx.x * waves + wave) * R;
    if constexpr (XLDS) {
        const unsigned char *xb = reinterpret_cast<const unsigned char *>(x);
        for (int off = 16 * (int)threadIdx.x; off < 64 * vecs; off += 16 * (int)blockDim.x)
            *reinterpret_cast<u32x4 *>(xs + off) = *reinterpret_cast<const u32x4 *>(xb + off);
        __syncthreads();
    }
    // Rows past N (only in the last workgroup) are clamped onto row N-1 and never stored.
    const uint8_t *wr[R];
    const uint16_t *sr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, n - 1);
        wr[r] = wq + (int64_t)row * ldq;
        sr[r] = scales + (int64_t)row * lds;
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.f;
    for (int s0 = 0; s0 < vecs; s0 += 64 * U) {
        u32x4 wv[U][R], xv[U][4];
        unsigned short sv[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(s0 + lane + 64 * u, vecs - 1);   // clamped into the row
#pragma unroll
            for (int r = 0; r < R; ++r) {
                wv[u][r] =
                    __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr[r] + 16 * v));
                sv[u][r] = sr[r][v >> 2];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (XLDS)
                    xv[u][j] = *reinterpret_cast<const u32x4 *>(xs + 64 * v + 16 * j);
                else
                    xv[u][j] = load_cached(x + 32 * v + 8 * j);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // the burst's loads before the first unpack
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = s0 + lane + 64 * u < vecs;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const unsigned w0 = wv[u][r].x, w1 = wv[u][r].y, w2 = wv[u][r].z,
                               w3 = wv[u][r].w;
                float p = int4_dot8(w0, xv[u][0], 0.f);
                p = int4_dot8(w1, xv[u][1], p);
                p = int4_dot8(w2, xv[u][2], p);
                p = int4_dot8(w3, xv[u][3], p);
                const float scale = bf16_to_f32(sv[u][r]) * 0.0625f;   // exact: a power of two
                const float next = fmaf(p, scale, acc[r]);
                acc[r] = in ? next : acc[r];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float sum = lane63(wave_sum(acc[r]));
        if (lane == 0 && row0 + r < n)
            y[row0 + r] = sum;
    }
}

template <int U, int R, bool XLDS>
const void *int4_kernel()
{
    return reinterpret_cast<const void *>(&gemv_int4<U, R, XLDS>);
}

// Compiled (U, R, x in LDS) combinations; the plan picks among them.
const void *find_int4(int u, int r, bool xlds)
{
    if (xlds) {
        if (r == 1)
            return u == 1 ? int4_kernel<1, 1, true>() : u == 2 ? int4_kernel<2, 1, true>()
                 : u == 4 ? int4_kernel<4, 1, true>() : nullptr;
        if (r == 2)
            return u == 1 ? int4_kernel<1, 2, true>() : u == 2 ? int4_kernel<2, 2, true>()
                                                             : nullptr;
        return nullptr;
    }
    if (r == 1)
        return u == 1 ? int4_kernel<1, 1, false>() : u == 2 ? int4_kernel<2, 1, false>()
             : u == 4 ? int4_kernel<4, 1, false>() : nullptr;
    if (r == 2)
        return u == 1 ? int4_kernel<1, 2, false>() : u == 2 ? int4_kernel<2, 2, false>()
                                                           : nullptr;
    return nullptr;
}

}  // namespace

namespace bbd {

gemv_status launch_int4(gemv_plan_t p, const void *Wq, int64_t ldq, const void *S, int64_t lds,
                        const void *X, float *Y, void *stream)
{
    const bool xlds = p->lds_bytes > 0;
    const void *fn = find_int4(p->unroll, p->rows_per_wave, xlds);
    if (!fn)
        return GEMV_ERR_INVALID_ARG;
    const uint8_t *wq = static_cast<const uint8_t *>(Wq);
    const uint16_t *sc = static_cast<const uint16_t *>(S);
    const uint16_t *x = static_cast<const uint16_t *>(X);
    int n = (int)p->n, vecs = (int)(p->k / kInt4VecElems), ldqi = (int)ldq, ldsi = (int)lds;
    void *args[] = {&wq, &sc, &x, &Y, &n, &vecs, &ldqi, &ldsi};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p->grid_x), dim3((unsigned)p->block_threads),
                                   args, (size_t)p->lds_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
