// moe_fp8_quant.h -- the OCP e4m3 encoder of the per-1 x 128 activation quantiser, shared by the
// standalone quantiser kernels (moe_quant.hip) and the FP8 GEMMs that quantise their activation
// rows themselves (moe_fp8_kernel.h), so both give the same codes.
#pragma once

#include "moe_device.h"

namespace moe {

// f32 -> e4m3 code, round to nearest even, magnitudes from 448 up saturate to 448 (0x7E), NaN
// -> 0x7F.  Normal range (|v| >= 2^-6): the e4m3 code is the f32 exponent rebiased (127 -> 7)
// and the top 3 mantissa bits, plus one when the 20 dropped bits are above half or exactly
// half with an odd code (a carry out of the mantissa steps the exponent, which is the next
// e4m3 value).  Below 2^-6 the codes are the subnormals m * 2^-9: m = rint(|v| * 512) (exact
// scaling, rint rounds half to even; m = 8 is the code of 2^-6).
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t code;
    if (!(a < 448.0f)) {
        code = a != a ? 0x7Fu : 0x7Eu;
    } else if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const uint32_t ab = __float_as_uint(a);
        const uint32_t base = ((((ab >> 23) - 127u + 7u)) << 3) | ((ab >> 20) & 7u);
        const uint32_t rest = ab & 0xFFFFFu;
        code = base + ((rest > 0x80000u || (rest == 0x80000u && (base & 1u))) ? 1u : 0u);
    }
    return code | sign;
}

// The codes of v0..v3 as bytes 0..3 of a word, equal to e4m3_code of each.  Below 464 in
// magnitude (448 is the largest code; the quantiser's quotients never exceed 448 by more than
// rounding) gfx950's v_cvt_pk_fp8_f32 rounds every f32 exactly as e4m3_code does (checked
// against it on all 2^32 bit patterns); from 464 up it gives NaN where e4m3_code saturates,
// so such lanes, and NaN, take e4m3_code.
__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3)
{
    const float m = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
    if (m < 464.0f) {  // false for NaN too
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
    }
    return e4m3_code(v0) | (e4m3_code(v1) << 8) | (e4m3_code(v2) << 16) | (e4m3_code(v3) << 24);
}

}  // namespace moe
