// moe_quant.hip -- bf16 activations -> OCP e4m3 codes with one f32 scale per 1 x 128 group, the
// a / a_scale operand pair of the block-scaled FP8 grouped GEMM (TileOPs "MoE" page,
// MoEGroupedGemmFP8Fwd: a_scale [.., ceil_div(K, 128)] f32).
//
// Two sources: rows of x, and SiLU(gate) * up of gate-up GEMM rows (bf16, then quantised).
//
// Per group: s = amax / 448 (448 = the largest finite e4m3 magnitude; s = 1 for an all-zero
// group), code = e4m3 nearest to x / s, ties to the even code.  Both divisions are IEEE f32.
// 16 lanes own one group (8 consecutive elements each: one 16-byte load, one 8-byte store); the
// group's amax is a 16-lane butterfly of maxima.  HBM-bound: 2 bytes in, 1 + 4/128 out per
// element.
#include "moe_device.h"
#include "moe_fp8_quant.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;

// Source rows: SRC_ROWS, row r of x; SRC_SWIGLU, h = bf16( SiLU(x[r, k]) * x[r, K + k] ) of a
// gate-up row x [M, 2K].
enum { SRC_ROWS = 0, SRC_SWIGLU = 2 };

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_quant_fp8(const uint16_t *__restrict__ x, int M,
                                                        int K, uint8_t *__restrict__ q,
                                                        float *__restrict__ scale)
{
    const int G = (K + 127) / 128;
    const long long gid = (long long)blockIdx.x * (kThreads / 16) + threadIdx.x / 16;
    if (gid >= (long long)M * G)  // whole 16-lane groups leave together
        return;
    const int row = (int)(gid / G), g = (int)(gid % G);
    const int sub = threadIdx.x & 15;
    const int k = 128 * g + 8 * sub;  // first of this lane's 8 elements
    const bool in = k < K;            // K % 8 == 0: a lane's 8 are all in or all out
    float v[8];
    if (in) {
        const size_t stride = MODE == SRC_SWIGLU ? 2 * (size_t)K : (size_t)K;
        const moe_u32x4 raw = *reinterpret_cast<const moe_u32x4 *>(x + (size_t)row * stride + k);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
        if (MODE == SRC_SWIGLU) {
            const moe_u32x4 rup =
                *reinterpret_cast<const moe_u32x4 *>(x + (size_t)row * stride + K + k);
            const uint32_t u[4] = {rup.x, rup.y, rup.z, rup.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u0 = __uint_as_float(u[i] << 16), u1 = __uint_as_float(u[i] & 0xFFFF0000u);
                const float g0 = v[2 * i], g1 = v[2 * i + 1];
                // h rounded to bf16 as the 16-bit passes store it, then quantised
                v[2 * i] = moe_bf16_to_f32(moe_f32_to_bf16(g0 / (1.0f + __expf(-g0)) * u0));
                v[2 * i + 1] =
                    moe_bf16_to_f32(moe_f32_to_bf16(g1 / (1.0f + __expf(-g1)) * u1));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
        amax = fmaxf(amax, __shfl_xor(amax, d, 16));
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
    if (sub == 0)
        scale[(size_t)row * G + g] = s;
    if (!in)
        return;
    const uint32_t lo = moe::e4m3_pack4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
    const uint32_t hi = moe::e4m3_pack4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    moe_u32x2 packed;
    packed.x = lo;
    packed.y = hi;
    *reinterpret_cast<moe_u32x2 *>(q + (size_t)row * K + k) = packed;
}

}  // namespace

namespace moe {

void launch_quant_fp8(const uint16_t *x, int M, int K, uint8_t *q, float *scale,
                      hipStream_t stream)
{
    const long long groups = (long long)M * ((K + 127) / 128);
    const long long blocks = (groups + kThreads / 16 - 1) / (kThreads / 16);
    hipLaunchKernelGGL(k_quant_fp8<SRC_ROWS>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       x, M, K, q, scale);
}

void launch_quant_fp8_swiglu(const uint16_t *gu, int M, int K, uint8_t *q, float *scale,
                             hipStream_t stream)
{
    const long long groups = (long long)M * ((K + 127) / 128);
    const long long blocks = (groups + kThreads / 16 - 1) / (kThreads / 16);
    hipLaunchKernelGGL(k_quant_fp8<SRC_SWIGLU>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, gu, M, K, q, scale);
}

}  // namespace moe
