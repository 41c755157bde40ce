// moe_stream_read.hip -- the HBM streaming-read kernel the benchmark reports as context: the
// read rate one GPU's CUs reach on a plain sequential stream, the practical ceiling for the
// weight-streaming expert GEMMs (whose bytes are almost all one read of each touched expert's
// weights).
//
// One workgroup of 8 waves per CU.  The grid sweeps the buffer in 8 KB blocks, block q read
// by workgroup q % grid (lane l taking its 16 bytes at 16 * l), so at any moment the grid's
// requests cover a contiguous window of a few MB spread over every HBM channel.  Each lane
// keeps kDepth non-temporal 16-byte loads in flight (like the expert weight loads); the loaded
// words are folded into one word per workgroup so the loads cannot be dropped.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 512;
constexpr int kDepth = 4;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kThreads) void k_stream_read(const moe_u32x4 *__restrict__ src,
                                                          size_t n16, uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kThreads;  // 16-byte units per sweep step
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kDepth - 1) * stride < n16; i += kDepth * stride) {
        moe_u32x4 v[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            v[d] = __builtin_nontemporal_load(src + i + (size_t)d * stride);
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    for (; i < n16; i += stride) {
        const moe_u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // one word per workgroup: the xor of its lanes' words (wave reduction, then LDS)
    __shared__ uint32_t part[kThreads / 64];
    for (int off = 32; off > 0; off >>= 1)
        acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < kThreads / 64; ++w)
            x ^= part[w];
        sink[blockIdx.x] = x;
    }
}

}  // namespace

namespace moe {

int stream_read_grid()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    return n;
}

void launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const moe_u32x4 *>(buf), bytes / 16, sink);
}

}  // namespace moe
