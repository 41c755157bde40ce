// moe_gemm_fp8.hip -- launches of the block-scaled FP8 grouped GEMM (moe_fp8_kernel.h).
#include "moe_fp8_kernel.h"
#include "moe_internal.h"

namespace {

template <int BM, int NTW, int STAGES>
void launch_one(const moe_fp8::Fp8Problem &p, hipStream_t stream)
{
    const int n_blocks = (p.N + 64 * NTW - 1) / (64 * NTW);
    const int m_tiles = (p.max_m + BM - 1) / BM;
    const int tiles = p.E * n_blocks * m_tiles;
    hipLaunchKernelGGL((moe_fp8::k_fp8_gemm<BM, NTW, STAGES>), dim3(moe_fp8::fp8_grid(tiles)),
                       dim3(64 * moe_fp8::kWaves), 0, stream, p, n_blocks, m_tiles);
}

}  // namespace

namespace moe {

void launch_fp8_gemm(const uint8_t *a, const float *a_scale, const uint8_t *b,
                     const float *b_scale, const int32_t *masked_m, int E, int max_m, int N,
                     int K, uint16_t *out, hipStream_t stream)
{
    moe_fp8::Fp8Problem p;
    p.a = a;
    p.a_scale = a_scale;
    p.b = b;
    p.b_scale = b_scale;
    p.masked_m = masked_m;
    p.out = out;
    p.E = E;
    p.max_m = max_m;
    p.N = N;
    p.K = K;
    p.KB = K / 128;
    p.NB = (N + 127) / 128;
    launch_one<64, 1, 3>(p, stream);
}

}  // namespace moe
