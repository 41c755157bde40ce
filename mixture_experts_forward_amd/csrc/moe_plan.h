// moe_plan.h -- host-only planning of a fused MoE call: argument checks, path choice, tile
// choice and the workspace layout.  No HIP call is made here, so every check runs (and can be
// tested) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;
constexpr int kMaxGroups = 64;
constexpr int kSortedBlockM = 16;  // row tile of the weight-streaming GEMMs
constexpr int kAlignChunk = 1024;   // routes per chunk of the chunked align/sort
// Workgroup slots (CUs x resident workgroups) whose K-split partial tiles the shared expert's
// workspace holds; on a device with more, the split uses fewer parts.
constexpr int kMaxSplitSlots = 256;

// Ints of device scratch the chunked align/sort needs for P routes and E experts (0: P fits one
// workgroup, which needs none).
inline size_t align_scratch_ints(int P, int E, bool balanced = false)
{
    return P > kAlignChunk
               ? (size_t)((P + kAlignChunk - 1) / kAlignChunk + (balanced ? 1 : 0)) * E
               : 0;
}

enum KernelKind {
    KERNEL_WS = 0,
    KERNEL_TILED = 1,
    KERNEL_WIDE = 3,
    KERNEL_MX = 4,
    KERNEL_MX_TILED = 5,
    KERNEL_MX_WIDE = 6
};

// Weight format of the routed experts: 16-bit (bf16 / f16) or MXFP4.
enum WeightFormat { WEIGHTS_16BIT = 0, WEIGHTS_MXFP4 = 1 };

struct TileChoice {
    int kind;  // KernelKind
    int nt, mt, ksplit, stages;
};

struct Plan {
    int path;           // MOE_PATH_DIRECT or MOE_PATH_SORTED (resolved)
    int T, H, E, F, k, S, P;
    int dtype;          // MOE_DTYPE_*
    int block_m;        // sorted path
    bool balanced;      // sorted path: routes spread evenly over each expert's tiles
    int slots;          // rows of the padded sorted order
    int tiles_cap;
    TileChoice gate_up, down, shared_gate_up, shared_down;
    int shared_slot_eighths;  // share of the resident slots the shared expert's GEMMs take
    // byte offsets into the workspace
    size_t off_ids, off_weights, off_sorted, off_offsets, off_tile_expert, off_inverse,
        off_n_tiles, off_sched, off_align, off_h, off_y, off_hs, off_ys, off_partial;
    size_t partial_bytes;  // bytes at off_partial (shared expert's K-split tiles)
    size_t total;
};

// Size checks common to every fused entry point (T, H, E, F, k, path).
int check_dims(const moe_params_t *p);
// Routing attribute checks (scoring, grouping, bias).
int check_routing(const moe_params_t *p, int bias_given);
int check_shared(int32_t shared_inter);

// Fills *plan for a valid p (checks must have passed).  S = shared_inter (0 = none).
void make_plan(const moe_params_t *p, int32_t S, Plan *plan, int wfmt = WEIGHTS_16BIT);

}  // namespace moe
