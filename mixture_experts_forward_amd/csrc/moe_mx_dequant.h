// moe_mx_dequant.h -- OCP MX FP4 (e2m1 codes, one E8M0 scale per 32 elements) to bf16 on gfx950,
// shared by the MXFP4 weight-streaming, row-tiled and 256 x 256 tile kernels.
#pragma once

#include "moe_device.h"

namespace moe_mx {

// E8M0 scale byte -> f32: 2^(s-127) (s = 0 is the subnormal 2^-127, s = 255 is NaN)
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    const uint32_t bits = s == 0u ? 0x00400000u : (s == 255u ? 0x7FC00000u : s << 23);
    return __uint_as_float(bits);
}

// one word of four code bytes -> eight bf16 (two per byte, low nibble first), times scale:
// v_cvt_scalef32_pk_bf16_fp4 converts one byte per call (exact: an e2m1 value has at most two
// significant bits)
__device__ __forceinline__ moe_u32x4 dequant8(uint32_t w, float scale)
{
    moe_u32x4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return o;
}

}  // namespace moe_mx
