// moe_noalloc.hip -- fused_moe_fwd_noalloc: fused_moe_fwd with its workspace in a fixed
// device array of the library instead of caller memory, for callers that cannot allocate.
//
// The array lives once per GPU for the life of the process.  Its host-side name is not a device
// address, so on the first call on each device (with that device current) the entry point
// looks up the array's device address with hipGetSymbolAddress and keeps it per device; only
// that address is ever handed to kernels.  Nothing here allocates.  The kernels clear what they
// need themselves (the align step zeroes the tile counters of the 256 x 256 GEMM; every other
// workspace region is written before it is read), so the array's contents from an earlier call
// do not matter.  Calls on one GPU share the array: calls that can overlap race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up once per device), or NULL
// if the HIP runtime reports an error.
void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return nullptr;
        g_ptr[dev] = ptr;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" int fused_moe_fwd_noalloc(const uint16_t *hidden_states, const float *gating_output,
                                     const uint16_t *w_gate_up, const uint16_t *w_down,
                                     const float *correction_bias, const moe_params_t *p,
                                     uint16_t *out, int32_t *topk_ids_out,
                                     float *topk_weights_out, void *stream)
{
    const size_t need = fused_moe_workspace_bytes(p, 0);
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_WORKSPACE;
    if (need == 0)  // T = 0 or arguments fused_moe_fwd rejects: its own status, nothing launched
        return fused_moe_fwd(hidden_states, gating_output, w_gate_up, w_down, correction_bias, p,
                             out, topk_ids_out, topk_weights_out, nullptr, 0, stream);
    void *ws = scratch_ptr();
    if (ws == nullptr)
        return MOE_ERR_LAUNCH;
    return fused_moe_fwd(hidden_states, gating_output, w_gate_up, w_down, correction_bias, p,
                         out, topk_ids_out, topk_weights_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                         stream);
}
