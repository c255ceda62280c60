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
//   - v_cvt_off_f32_i4 turns the signed nibble in bits 3:0 of its operand into v / 16 in
//     fp32, exactly; with a byte select it reads the even-indexed nibbles straight from the
//     word's bytes, and from the word shifted right by 4 the odd-indexed ones;
//   - the top halves of two such floats are the bf16 pair (v_2i / 16, v_2i+1 / 16), exactly,
//     which v_dot2c_f32_bf16 multiplies by the x pair (x_2i, x_2i+1);
// so the 32 products of a vector form one fp32 chain, p = sum (v / 16) x, and the group
// scale then enters once: acc = fma(p, 16 scale, acc). No product is formed inexactly (v / 16
// has 4 significant bits, x 8) and no offset is subtracted after the fact, so the error
// analysis of the bf16 path carries over unchanged.
//
// That unpack costs 17 VALU instructions per 8 weights (one shift, 8 conversions, 4 packs,
// 4 dot products), which at the HBM rate is most of a CU's VALU issue. When x is staged in
// LDS the kernel first tries a cheaper exact form (13 per 8 weights) built on fp16:
//   - x is staged per 32-element vector as fp16 x * 2^s, with s chosen per vector so that
//     its largest magnitude lands in [2^15, 2^16); the 2^-s goes into that vector's scale
//     multiplier. The conversion works on the bit patterns (exponent rebased by a packed
//     saturating subtract, then shifted into place), and every element must come out as a
//     normal fp16 or zero, i.e. within 2^29 of its vector's largest. If one does not, or x
//     holds an inf or NaN, the whole workgroup stages bf16 x instead and runs the form
//     above;
//   - per packed word, with t = word >> 8 and n' = nibble ^ 8 = v + 8, (word & 0x000F000F)
//     ^ 0x64086408 is the fp16 pair (1024 + n'_0, 1024 + n'_4) and (word & 0x00F000F0) ^
//     0x54805480 the pair (64 + n'_1, 64 + n'_5) (the high nibble lands where an fp16 near
//     64 has a unit step); one v_bitop3 each, the XOR doing the offset and the exponent at
//     once. The same on t gives elements 2, 6 and 3, 7. One packed fp16 add of -1032 (or
//     -72) leaves (v, v') exactly;
//   - v_dot2c_f32_f16 multiplies each pair by its staged x pair ((x_0, x_4) 2^s, ...), so
//     every product is v x 2^s, exact in fp32 (4 and 8 significant bits); the vector then
//     enters as fma(p, scale * 2^-s, acc). A power-of-two scale changes no rounding, and
//     the chain has as many steps as the bf16 form's, so the same depth bound holds.
// x staging is done once per workgroup, so workgroups loop over row blocks to spread it
// over more rows.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device.h"
#include "plan.h"

namespace {

using namespace bbd;

// bf16 pair (v_2i / 16, v_2i+1 / 16) for pair i of a packed word d, t = d >> 4. Byte i of d
// holds element 2i in its low nibble and byte i of t element 2i + 1: bit-field extracts of
// bytes fold into the conversions' byte selects.
template <int I>
__device__ __forceinline__ unsigned int4_pair(unsigned d, unsigned t)
{
    const float lo = __builtin_amdgcn_cvt_off_f32_i4(__builtin_amdgcn_ubfe(d, 8 * I, 8));
    const float hi = __builtin_amdgcn_cvt_off_f32_i4(__builtin_amdgcn_ubfe(t, 8 * I, 8));
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// d >> 4 as a value of its own. Written plainly, the compiler folds the shift into each odd
// element's extract (a shift per element instead of a byte select on one shifted word).
__device__ __forceinline__ unsigned shifted_by_4(unsigned d)
{
    unsigned t;
    asm("v_lshrrev_b32 %0, 4, %1" : "=v"(t) : "v"(d));
    return t;
}

// p + sum of the 8 products (v / 16) x of packed word d with the x vector half xd (4 bf16
// pairs).
__device__ __forceinline__ float int4_dot8(unsigned d, u32x4 xd, float p)
{
    const unsigned t = shifted_by_4(d);
    const unsigned x0 = xd.x, x1 = xd.y, x2 = xd.z, x3 = xd.w;
    p = dot2(int4_pair<0>(d, t), x0, p);
    p = dot2(int4_pair<1>(d, t), x1, p);
    p = dot2(int4_pair<2>(d, t), x2, p);
    p = dot2(int4_pair<3>(d, t), x3, p);
    return p;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// p + sum of the 8 products of packed word d with the staged fp16 pairs of its x block:
// xd = ((x0, x4), (x1, x5), (x2, x6), (x3, x7)), each times the vector's 2^s.
__device__ __forceinline__ float int4_dot8_f16(unsigned d, u32x4 xd, float p)
{
    const unsigned t = d >> 8;
    const half2v lo_off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2v hi_off = {(_Float16)-72.0f, (_Float16)-72.0f};
    const half2v a = __builtin_bit_cast(half2v, (d & 0x000F000Fu) ^ 0x64086408u) + lo_off;
    const half2v b = __builtin_bit_cast(half2v, (d & 0x00F000F0u) ^ 0x54805480u) + hi_off;
    const half2v c = __builtin_bit_cast(half2v, (t & 0x000F000Fu) ^ 0x64086408u) + lo_off;
    const half2v e = __builtin_bit_cast(half2v, (t & 0x00F000F0u) ^ 0x54805480u) + hi_off;
    const unsigned x0 = xd.x, x1 = xd.y, x2 = xd.z, x3 = xd.w;
    p = __builtin_amdgcn_fdot2(a, __builtin_bit_cast(half2v, x0), p, false);
    p = __builtin_amdgcn_fdot2(b, __builtin_bit_cast(half2v, x1), p, false);
    p = __builtin_amdgcn_fdot2(c, __builtin_bit_cast(half2v, x2), p, false);
    p = __builtin_amdgcn_fdot2(e, __builtin_bit_cast(half2v, x3), p, false);
    return p;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(unsigned v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ unsigned as_u32(u16x2 v) { return __builtin_bit_cast(unsigned, v); }

// Stage one 32-element x vector (16 words of bf16 pairs, element 2i in the low half of word
// i) as the fp16 pairs int4_dot8_f16 expects, scaled by the vector's 2^s; *mult = 2^-s.
// Returns false when an element is not exactly a normal fp16 (or zero) after scaling, or
// the vector holds an inf or NaN, or its largest element is below 2^-96.
__device__ __forceinline__ bool stage_vec_f16(const unsigned (&w)[16], unsigned (&out)[16],
                                              float *mult)
{
    // Magnitude patterns: the largest, and the smallest nonzero one (minus 1; 0 wraps).
    u16x2 amax = {0, 0}, amin = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const u16x2 a = as_u16x2(w[i] & 0x7FFF7FFFu);
        amax = __builtin_elementwise_max(amax, a);
        amin = __builtin_elementwise_min(amin, a - (u16x2){1, 1});
    }
    const unsigned big = max((unsigned)amax.x, (unsigned)amax.y);
    const unsigned small = min((unsigned)amin.x, (unsigned)amin.y);   // 0xFFFF: all zero
    const unsigned e = big >> 7;                     // biased exponent of the largest
    bool ok = big < 0x7F80u && (big == 0 || e >= 31);
    // fp16 exponent field of an element = its bf16 one - (e - 30): the largest gets 30.
    const unsigned d = e >= 30 ? (e - 30) << 7 : 0;
    ok = ok && (big == 0 || small + 1 >= d + 0x80);
    const u16x2 dd = {(unsigned short)d, (unsigned short)d};
    unsigned h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const u16x2 a = as_u16x2(w[i] & 0x7FFF7FFFu);
        const unsigned t = as_u32(__builtin_elementwise_sub_sat(a, dd));   // zeros stay 0
        h[i] = (t << 3) | (w[i] & 0x80008000u);
    }
    // word i holds elements 2i, 2i+1; pairs are (x0, x4), (x1, x5), (x2, x6), (x3, x7)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[4 * j + 0] = __builtin_amdgcn_perm(h[4 * j + 2], h[4 * j], 0x05040100u);
        out[4 * j + 1] = __builtin_amdgcn_perm(h[4 * j + 2], h[4 * j], 0x07060302u);
        out[4 * j + 2] = __builtin_amdgcn_perm(h[4 * j + 3], h[4 * j + 1], 0x05040100u);
        out[4 * j + 3] = __builtin_amdgcn_perm(h[4 * j + 3], h[4 * j + 1], 0x07060302u);
    }
    *mult = big == 0 ? 1.f : __uint_as_float((e - 15) << 23);   // 2^(e - 142) = 2^-s
    return ok;
}

// One burst of a wave's R rows: U packed vectors per lane and row (lane l takes vectors
// l, l + 64, ... of each row, from s0 on) with their group scales, and, when x is not staged
// in LDS, the four 16-byte x blocks of each (their latency is as long as the weights').
template <int U, int R, bool XLDS>
struct Burst {
    u32x4 w[U][R];
    unsigned short s[U][R];
    u32x4 xg[XLDS ? 1 : U][4];
};

template <int U, int R, bool XLDS>
__device__ __forceinline__ void load_burst(Burst<U, R, XLDS> &b, const uint8_t *const (&wr)[R],
                                           const uint16_t *const (&sr)[R], const uint16_t *x,
                                           int s0, int vecs, int lane)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int v = min(s0 + lane + 64 * u, vecs - 1);   // clamped into the row
#pragma unroll
        for (int r = 0; r < R; ++r) {
            b.w[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr[r] + 16 * v));
            b.s[u][r] = sr[r][v >> 2];
        }
        if constexpr (!XLDS) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b.xg[u][j] = load_cached(x + 32 * v + 8 * j);
        }
    }
}

// Multiply a loaded burst into the R accumulators. F16: the x blocks are the fp16 pairs of
// stage_vec_f16 in LDS with the vector multipliers after them; otherwise bf16 (LDS when
// XLDS). Staged x is read from LDS only when its vector is about to be used.
template <int U, int R, bool XLDS, bool F16>
__device__ __forceinline__ void use_burst(const Burst<U, R, XLDS> &b, const unsigned char *xs,
                                          int s0, int vecs, int lane, float (&acc)[R])
{
    const float *mults = reinterpret_cast<const float *>(xs + 64 * vecs);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool in = s0 + lane + 64 * u < vecs;
        u32x4 xv[4];
        float mv = 1.f;
        if constexpr (XLDS) {
            const int v = min(s0 + lane + 64 * u, vecs - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xv[j] = *reinterpret_cast<const u32x4 *>(xs + 64 * v + 16 * j);
            if constexpr (F16)
                mv = mults[v];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xv[j] = b.xg[u][j];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const unsigned w0 = b.w[u][r].x, w1 = b.w[u][r].y, w2 = b.w[u][r].z,
                           w3 = b.w[u][r].w;
            float p, scale;
            if constexpr (F16) {
                p = int4_dot8_f16(w0, xv[0], 0.f);
                p = int4_dot8_f16(w1, xv[1], p);
                p = int4_dot8_f16(w2, xv[2], p);
                p = int4_dot8_f16(w3, xv[3], p);
                scale = bf16_to_f32(b.s[u][r]) * mv;   // exact: mv is a power of two
            } else {
                p = int4_dot8(w0, xv[0], 0.f);
                p = int4_dot8(w1, xv[1], p);
                p = int4_dot8(w2, xv[2], p);
                p = int4_dot8(w3, xv[3], p);
                scale = bf16_to_f32(b.s[u][r]) * 16.f;   // exact: a power of two
            }
            const float next = fmaf(p, scale, acc[r]);
            acc[r] = in ? next : acc[r];
        }
    }
}

template <int R>
__device__ __forceinline__ void row_pointers(const uint8_t *wq, const uint16_t *scales, int n,
                                             int ldq, int lds, int row0,
                                             const uint8_t *(&wr)[R], const uint16_t *(&sr)[R])
{
    // Rows past N (only in the last row block) are clamped onto row N-1 and never stored.
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, n - 1);
        wr[r] = wq + (int64_t)row * ldq;
        sr[r] = scales + (int64_t)row * lds;
    }
}

// The rows of the workgroup's row blocks b0, b0 + stride, ..., the first burst of the first
// block already loaded in `first`.
template <int U, int R, bool XLDS, bool F16>
__device__ __forceinline__ void int4_blocks(Burst<U, R, XLDS> &first, const uint8_t *wq,
                                            const uint16_t *scales, const unsigned char *xs,
                                            const uint16_t *x, float *y, int n, int vecs,
                                            int ldq, int lds, int b0, int stride, int blocks,
                                            int waves, int wave, int lane)
{
    for (int b = b0; b < blocks; b += stride) {
        const int row0 = (b * waves + wave) * R;
        const uint8_t *wr[R];
        const uint16_t *sr[R];
        row_pointers<R>(wq, scales, n, ldq, lds, row0, wr, sr);
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = 0.f;
        for (int s0 = 0; s0 < vecs; s0 += 64 * U) {
            if (b != b0 || s0 != 0) {
                load_burst<U, R, XLDS>(first, wr, sr, x, s0, vecs, lane);
                __builtin_amdgcn_sched_barrier(0);   // the burst's loads before the unpack
            }
            use_burst<U, R, XLDS, F16>(first, xs, s0, vecs, lane, acc);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sum = lane63(wave_sum(acc[r]));
            if (lane == 0 && row0 + r < n)
                y[row0 + r] = sum;
        }
    }
}

// U vectors per lane per burst; R rows per wave (sharing every x vector); up to MAXW waves
// per workgroup. XLDS: the workgroup stages x in LDS (fp16 when exact, else bf16), which
// takes the x traffic (four 16-byte x blocks per 16-byte weight vector) off the
// vector-memory path. Row block b holds rows b*waves*R and on, wave w its rows w*R + r;
// workgroups take row blocks blockIdx.x, + gridDim.x, ... so the staging serves them all.
// Each thread issues its x loads, then its first weight burst, then waits for x alone:
// vector loads return in order, so the weights stream while x is converted.
template <int U, int R, bool XLDS, int MAXW, bool TRY_F16>
__global__ void __launch_bounds__(64 * MAXW)
    gemv_int4(const uint8_t *wq, const uint16_t *scales, const uint16_t *x, float *y, int n,
              int vecs, int ldq, int lds, int blocks)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char xs[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int waves = (int)(blockDim.x >> 6);
    const int b0 = blockIdx.x;
    Burst<U, R, XLDS> first;
    if constexpr (XLDS && !TRY_F16) {
        // bf16 x copied into LDS; the first weight burst goes out right behind its loads
        const int t = (int)threadIdx.x;
        const int nthreads = (int)blockDim.x;
        const unsigned char *xb = reinterpret_cast<const unsigned char *>(x);
        // 16-byte copies held per thread: the plans give long rows (K = 14336: 28 KiB of x
        // over 512 threads) U >= 4 and K = 4096 rows (8 KiB over 256-512 threads) U <= 2;
        // any x beyond goes through the loop after the burst.
        constexpr int kMaxCopy = U >= 4 ? 4 : 2;
        // Unconditional loads from clamped offsets (past the end they re-read the last 16
        // bytes): loads under a branch, even a workgroup-uniform one, are each waited for
        // before the join.
        u32x4 cp[kMaxCopy];
#pragma unroll
        for (int i = 0; i < kMaxCopy; ++i) {
            const int off = min(16 * (t + i * nthreads), 64 * vecs - 16);
            cp[i] = *reinterpret_cast<const u32x4 *>(xb + off);
        }
        __builtin_amdgcn_sched_barrier(0);   // x's loads go out before the weights'
        {
            const uint8_t *wr[R];
            const uint16_t *sr[R];
            row_pointers<R>(wq, scales, n, ldq, lds, (b0 * waves + wave) * R, wr, sr);
            load_burst<U, R, XLDS>(first, wr, sr, x, 0, vecs, lane);
        }
#pragma unroll
        for (int i = 0; i < kMaxCopy; ++i) {
            const int off = 16 * (t + i * nthreads);
            if (off < 64 * vecs)
                *reinterpret_cast<u32x4 *>(xs + off) = cp[i];
        }
        for (int off = 16 * (t + kMaxCopy * nthreads); off < 64 * vecs; off += 16 * nthreads)
            *reinterpret_cast<u32x4 *>(xs + off) = *reinterpret_cast<const u32x4 *>(xb + off);
        __syncthreads();
        int4_blocks<U, R, XLDS, false>(first, wq, scales, xs, x, y, n, vecs, ldq, lds, b0,
                                       gridDim.x, blocks, waves, wave, lane);
        return;
    } else if constexpr (!XLDS) {
        const uint8_t *wr[R];
        const uint16_t *sr[R];
        row_pointers<R>(wq, scales, n, ldq, lds, (b0 * waves + wave) * R, wr, sr);
        load_burst<U, R, XLDS>(first, wr, sr, x, 0, vecs, lane);
        __builtin_amdgcn_sched_barrier(0);
        int4_blocks<U, R, XLDS, false>(first, wq, scales, xs, x, y, n, vecs, ldq, lds, b0,
                                       gridDim.x, blocks, waves, wave, lane);
        return;
    } else {
        // Each thread stages whole vectors: fp16 pairs at xs + 64 v, multipliers after x.
        // The vectors of the first pass are loaded before the first weight burst.
        float *mults = reinterpret_cast<float *>(xs + 64 * vecs);
        const int t = (int)threadIdx.x;
        const int nthreads = (int)blockDim.x;
        unsigned w[16];
        {   // clamped rather than predicated, for the same reason as the bf16 copy above
            const u32x4 *src = reinterpret_cast<const u32x4 *>(x + 32 * min(t, vecs - 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 v = src[j];
                w[4 * j] = v.x;
                w[4 * j + 1] = v.y;
                w[4 * j + 2] = v.z;
                w[4 * j + 3] = v.w;
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // x's loads go out before the weights'
        {
            const uint8_t *wr[R];
            const uint16_t *sr[R];
            row_pointers<R>(wq, scales, n, ldq, lds, (b0 * waves + wave) * R, wr, sr);
            load_burst<U, R, XLDS>(first, wr, sr, x, 0, vecs, lane);
        }
        bool ok = true;
        for (int v = t; v < vecs; v += nthreads) {
            if (v != t) {                                   // later passes: load here
                const u32x4 *src = reinterpret_cast<const u32x4 *>(x + 32 * v);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 q = src[j];
                    w[4 * j] = q.x;
                    w[4 * j + 1] = q.y;
                    w[4 * j + 2] = q.z;
                    w[4 * j + 3] = q.w;
                }
            }
            unsigned out[16];
            float m;
            ok = stage_vec_f16(w, out, &m) && ok;
            u32x4 *dst = reinterpret_cast<u32x4 *>(xs + 64 * v);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dst[j] = u32x4{out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]};
            mults[v] = m;
        }
        const bool f16 = !__syncthreads_or(!ok);
        if (f16) {
            int4_blocks<U, R, XLDS, true>(first, wq, scales, xs, x, y, n, vecs, ldq, lds, b0,
                                          gridDim.x, blocks, waves, wave, lane);
        } else {                         // some element of x: back to the bf16 copy
            const unsigned char *xb = reinterpret_cast<const unsigned char *>(x);
            for (int off = 16 * t; off < 64 * vecs; off += 16 * nthreads)
                *reinterpret_cast<u32x4 *>(xs + off) = *reinterpret_cast<const u32x4 *>(xb + off);
            __syncthreads();
            int4_blocks<U, R, XLDS, false>(first, wq, scales, xs, x, y, n, vecs, ldq, lds, b0,
                                           gridDim.x, blocks, waves, wave, lane);
        }
    }
}

template <int U, int R, bool XLDS, bool F16>
const void *int4_kernel(int waves)
{
    if constexpr (!XLDS && U == 7) {   // x in registers: too many for 16-wave workgroups
        return waves > 8 ? nullptr
                         : reinterpret_cast<const void *>(&gemv_int4<U, R, XLDS, 8, false>);
    } else {
        return waves > 8 ? reinterpret_cast<const void *>(&gemv_int4<U, R, XLDS, 16, F16>)
                         : reinterpret_cast<const void *>(&gemv_int4<U, R, XLDS, 8, F16>);
    }
}

template <bool XLDS, bool F16>
const void *int4_tile(int u, int r, int waves)
{
    if (r == 1)
        return u == 1   ? int4_kernel<1, 1, XLDS, F16>(waves)
             : u == 2 ? int4_kernel<2, 1, XLDS, F16>(waves)
             : u == 4 ? int4_kernel<4, 1, XLDS, F16>(waves)
             : u == 7 ? int4_kernel<7, 1, XLDS, F16>(waves)
                      : nullptr;
    if (r == 2)
        return u == 1   ? int4_kernel<1, 2, XLDS, F16>(waves)
             : u == 2 ? int4_kernel<2, 2, XLDS, F16>(waves)
                      : nullptr;
    return nullptr;
}

// Compiled (U, R, x in LDS, fp16 staging tried, waves per workgroup up to 8 or 16).
const void *find_int4(int u, int r, bool xlds, bool f16, int waves)
{
    if (!xlds)
        return int4_tile<false, false>(u, r, waves);
    return f16 ? int4_tile<true, true>(u, r, waves) : int4_tile<true, false>(u, r, waves);
}

}  // namespace

namespace bbd {

gemv_status launch_int4(gemv_plan_t p, const void *Wq, int64_t ldq, const void *S, int64_t lds,
                        const void *X, float *Y, void *stream)
{
    const bool xlds = p->lds_bytes > 0;
    const int64_t vecs64 = p->k / kInt4VecElems;
    // The launch's dynamic LDS is exactly the staged x (64-byte pairs and a 4-byte
    // multiplier per vector); anything else is a plan this kernel was not sized for.
    if (xlds && (int64_t)p->lds_bytes != vecs64 * (64 + 4))
        return GEMV_ERR_INVALID_ARG;
    const void *fn = find_int4(p->unroll, p->rows_per_wave, xlds, p->int4_fp16 != 0,
                               p->waves_per_block);
    if (!fn)
        return GEMV_ERR_INVALID_ARG;
    const uint8_t *wq = static_cast<const uint8_t *>(Wq);
    const uint16_t *sc = static_cast<const uint16_t *>(S);
    const uint16_t *x = static_cast<const uint16_t *>(X);
    int n = (int)p->n, vecs = (int)(p->k / kInt4VecElems), ldqi = (int)ldq, ldsi = (int)lds;
    int blocks = (int)((p->n + (int64_t)p->rows_per_wave * p->waves_per_block - 1) /
                       ((int64_t)p->rows_per_wave * p->waves_per_block));
    void *args[] = {&wq, &sc, &x, &Y, &n, &vecs, &ldqi, &ldsi, &blocks};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p->grid_x), dim3((unsigned)p->block_threads),
                                   args, (size_t)p->lds_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMV_OK : record_hip_error((int)e, GEMV_ERR_DEVICE);
}

}  // namespace bbd
