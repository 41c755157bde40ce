// moe_combine.hip -- deterministic weighted combine of the expert output rows.
//
// out[t, c] = bf16( sum_{j<k} w[t,j] * y[t*k + j, c]  (+ ys[t, c]) ), j ascending, f32 sums
// (f16 in and out for the f16 pass)
// (TileOPs "MoE" page, MoEPostPermuteFwd: expert_output, topk_weights [T,K] f32; the shared
// expert of FusedMoESharedExpertFwd is added with weight one).  Routes whose id is outside
// [0, E) are skipped.  The expert GEMMs write y indexed by route, so a token's k rows are
// contiguous and each 16-byte load covers eight columns (the FP8 pass, whose rows stay in expert
// order, passes the row of each route instead).  Every output row is written, so the
// output needs no clear beforehand (the aiter MI308 decoding PR drops its output clear for the
// same reason).
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;

template <int DT>
__global__ __launch_bounds__(kThreads) void k_combine(
    const uint16_t *__restrict__ y, const int32_t *__restrict__ ids,
    const float *__restrict__ weights, const uint16_t *__restrict__ ys, uint16_t *__restrict__ out,
    int H, int k, int E, const int32_t *__restrict__ row_of_route)
{
    const int t = blockIdx.x;
    const int c = (blockIdx.y * kThreads + threadIdx.x) * 8;
    if (c >= H)
        return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // routes in groups of kGroup: the group's row loads are all issued before any is summed, so
    // their latencies overlap; the sums still run in j order
    constexpr int kGroup = 8;
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        moe_u32x4 v[kGroup];
        float w[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int j = j0 + u;
            w[u] = 0.0f;
            v[u] = moe_u32x4{0u, 0u, 0u, 0u};
            if (j < k) {
                const size_t r = (size_t)t * k + j;
                const int e = ids[r];
                if (e >= 0 && e < E) {
                    w[u] = weights[r];
                    const size_t yr = row_of_route ? (size_t)row_of_route[r] : r;
                    // each expert row is read once: non-temporal, so the stream of them does
                    // not evict what L2 holds for other work (DeepSeek-V3 prefill: 105 -> 93 us)
                    v[u] = __builtin_nontemporal_load(
                        reinterpret_cast<const moe_u32x4 *>(y + yr * H + c));
                }
            }
        }
        // a skipped route adds 0 * 0 = +0, which leaves the sum as it is (the sum starts at +0
        // and never becomes -0)
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += w[u] * moe_to_f32<DT>(v[u][q]);
                acc[2 * q + 1] += w[u] * moe_to_f32<DT>(v[u][q] >> 16);
            }
        }
    }
    if (ys) {
        const moe_u32x4 v = *reinterpret_cast<const moe_u32x4 *>(ys + (size_t)t * H + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += moe_to_f32<DT>(v[q]);
            acc[2 * q + 1] += moe_to_f32<DT>(v[q] >> 16);
        }
    }
    moe_u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = moe_pack2<DT>(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<moe_u32x4 *>(out + (size_t)t * H + c) = o;
}

}  // namespace

namespace moe {

void launch_combine(const uint16_t *y, const int32_t *ids, const float *weights,
                    const uint16_t *ys, uint16_t *out, int T, int H, int k, int E, int dtype,
                    hipStream_t stream, const int32_t *row_of_route)
{
    const dim3 grid(T, (H / 8 + kThreads - 1) / kThreads);
    if (dtype == 1)
        hipLaunchKernelGGL(k_combine<1>, grid, dim3(kThreads), 0, stream, y, ids, weights, ys,
                           out, H, k, E, row_of_route);
    else
        hipLaunchKernelGGL(k_combine<0>, grid, dim3(kThreads), 0, stream, y, ids, weights, ys,
                           out, H, k, E, row_of_route);
}

}  // namespace moe
