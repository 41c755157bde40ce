// moe_masked.hip -- route ids of the masked layout (TileOPs "MoE" page, MoEGroupedGemmFwd with
// a: [E, layout.max_m, K] and layout_metadata [E]).
//
// Row q = e * max_m + i of the flattened [E * max_m] row blocks belongs to expert e when
// i < masked_m[e] and to no expert (-1) otherwise.  With these ids as single-route tokens, the
// align/sort and the grouped GEMMs of the routed pass compute the masked MLP unchanged.
#include "moe_internal.h"

namespace {

__global__ __launch_bounds__(256) void k_masked_ids(const int32_t *__restrict__ masked_m, int E,
                                                    int max_m, int32_t *__restrict__ ids)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)E * max_m)
        return;
    const int e = (int)(q / max_m);
    const int i = (int)(q - (int64_t)e * max_m);
    const int m = min(max(masked_m[e], 0), max_m);
    ids[q] = i < m ? e : -1;
}

}  // namespace

namespace moe {

void launch_masked_ids(const int32_t *masked_m, int E, int max_m, int32_t *ids,
                       hipStream_t stream)
{
    const int64_t rows = (int64_t)E * max_m;
    if (rows == 0)
        return;
    hipLaunchKernelGGL(k_masked_ids, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                       masked_m, E, max_m, ids);
}

}  // namespace moe
