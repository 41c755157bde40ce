// moe_device.h -- device helpers shared by the gfx950 kernels of the fused MoE forward pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 moe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float moe_f32x4 __attribute__((ext_vector_type(4)));
typedef float moe_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t moe_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t moe_u32x2 __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64

// bf16 bit pattern -> f32 (exact).
__device__ __forceinline__ float moe_bf16_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// f32 -> bf16 bit pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t moe_f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t moe_pack_bf16x2(float lo, float hi)
{
    return moe_f32_to_bf16(lo) | (moe_f32_to_bf16(hi) << 16);
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16) on one wave.
// Lane l supplies A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16] and holds
// D[4*(l/16) + r][l%16], r = 0..3.
__device__ __forceinline__ moe_f32x4 moe_mfma_16x16x32(moe_u32x4 a, moe_u32x4 b, moe_f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(moe_bf16x8, a),
                                                   __builtin_bit_cast(moe_bf16x8, b), c, 0, 0, 0);
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16) on one wave: twice the work of the 16x16x32
// form in the same issue time on gfx950.  Lane l supplies A[l%32][8*(l/32) .. +8] and
// B[8*(l/32) .. +8][l%32] and holds D[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15.
__device__ __forceinline__ moe_f32x16 moe_mfma_32x32x16(moe_u32x4 a, moe_u32x4 b, moe_f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(moe_bf16x8, a),
                                                   __builtin_bit_cast(moe_bf16x8, b), c, 0, 0, 0);
}

// Element type of the pass's activations, weights and outputs: DT 0 = bf16, 1 = f16 (both
// 16-bit patterns in uint16_t).  The MFMA forms of the two types share lane layouts.
typedef _Float16 moe_f16x8 __attribute__((ext_vector_type(8)));

template <int DT>
__device__ __forceinline__ moe_f32x4 moe_mma16(moe_u32x4 a, moe_u32x4 b, moe_f32x4 c)
{
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(moe_f16x8, a),
                                                      __builtin_bit_cast(moe_f16x8, b), c, 0, 0,
                                                      0);
    else
        return moe_mfma_16x16x32(a, b, c);
}

template <int DT>
__device__ __forceinline__ moe_f32x16 moe_mma32(moe_u32x4 a, moe_u32x4 b, moe_f32x16 c)
{
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(moe_f16x8, a),
                                                      __builtin_bit_cast(moe_f16x8, b), c, 0, 0,
                                                      0);
    else
        return moe_mfma_32x32x16(a, b, c);
}

// two f32 -> one word of two 16-bit values (lo in the low half), round to nearest even
template <int DT>
__device__ __forceinline__ uint32_t moe_pack2(float lo, float hi)
{
    if constexpr (DT == 1)
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    else
        return moe_pack_bf16x2(lo, hi);
}

// 16-bit pattern (low half of b) -> f32, exact
template <int DT>
__device__ __forceinline__ float moe_to_f32(uint32_t b)
{
    if constexpr (DT == 1)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu));
    else
        return moe_bf16_to_f32(b & 0xffffu);
}

// Ordering a wave's LDS traffic without a workgroup barrier.
__device__ __forceinline__ void moe_wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
