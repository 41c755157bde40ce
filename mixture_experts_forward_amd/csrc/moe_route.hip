// moe_route.hip -- routing kernel: one wave per token, four tokens per workgroup.
#include "moe_internal.h"
#include "moe_route_dev.h"

namespace {

constexpr int kWaves = 4;
constexpr int kMaxExperts = 1024;

template <int SLOTS>
__global__ __launch_bounds__(64 * kWaves) void k_route(
    const float *__restrict__ gating, const float *__restrict__ bias, int T, int E, int k,
    int sigmoid, int renormalize, int n_group, int topk_group, float rsf,
    int32_t *__restrict__ ids_out, float *__restrict__ weights_out)
{
    __shared__ float s_key[kWaves][kMaxExperts];
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * kWaves + wv;
    if (t >= T)
        return;  // whole wave; no workgroup barrier follows
    moe_route_dev::route_token<SLOTS>(gating, bias, t, E, k, sigmoid, renormalize, n_group,
                                      topk_group, rsf, s_key[wv], threadIdx.x & 63, ids_out,
                                      weights_out, nullptr);
}

}  // namespace

namespace moe {

void launch_route(const float *gating, const float *bias, int T, int E, int k, int sigmoid,
                  int renormalize, int n_group, int topk_group, float rsf, int32_t *ids,
                  float *weights, hipStream_t stream)
{
    const dim3 grid((T + kWaves - 1) / kWaves), block(64 * kWaves);
#define MOE_ROUTE_CASE(S)                                                                        \
    hipLaunchKernelGGL(k_route<S>, grid, block, 0, stream, gating, bias, T, E, k, sigmoid,       \
                       renormalize, n_group, topk_group, rsf, ids, weights)
    if (E <= 64)
        MOE_ROUTE_CASE(1);
    else if (E <= 128)
        MOE_ROUTE_CASE(2);
    else if (E <= 256)
        MOE_ROUTE_CASE(4);
    else if (E <= 512)
        MOE_ROUTE_CASE(8);
    else
        MOE_ROUTE_CASE(16);
#undef MOE_ROUTE_CASE
}

}  // namespace moe
