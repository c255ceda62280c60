// device.h - device helpers shared by the gfx950 GEMV kernels (gemv.hip, chain.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace bbd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Element access goes through by-value scalars: clang mis-lowers __builtin_bit_cast
// applied directly to an ext_vector element (it reads element 0).
__device__ __forceinline__ float dot2(unsigned w, unsigned x, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, x), acc, false);
}

__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc)
{
    unsigned w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    unsigned x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
    acc = dot2(w0, x0, acc);
    acc = dot2(w1, x1, acc);
    acc = dot2(w2, x2, acc);
    acc = dot2(w3, x3, acc);
    return acc;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((unsigned)b << 16);
}

__device__ __forceinline__ u32x4 load_stream(const uint16_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ u32x4 load_cached(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v)
{
    // Lanes outside ROW_MASK keep `old` = 0, so adding the result leaves them unchanged.
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK,
                                                      0xF, false));
}

// Sum of the 64 lane values, valid in lane 63. Fixed tree, hence deterministic.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]: pairs
    v += dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]: quads
    v += dpp<0x141, 0xF>(v);  // row_half_mirror: 8 lanes
    v += dpp<0x140, 0xF>(v);  // row_mirror: 16 lanes (a full DPP row)
    v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ float lane63(float v)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace bbd
