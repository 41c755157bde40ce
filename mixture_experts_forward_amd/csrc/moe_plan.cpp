// moe_plan.cpp -- host-only argument checks, path/tile choice and workspace layout.
#include "moe_plan.h"

namespace moe {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int check_dims(const moe_params_t *p)
{
    if (!p)
        return MOE_ERR_NULL;
    if (p->num_tokens < 0 || p->hidden <= 0 || p->num_experts <= 0 || p->inter <= 0 ||
        p->top_k <= 0 || p->top_k > p->num_experts)
        return MOE_ERR_SHAPE;
    if (p->top_k > kMaxTopK || p->num_experts > kMaxExperts)
        return MOE_ERR_UNSUPPORTED;
    if (p->hidden % 64 != 0 || p->inter % 64 != 0)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)p->num_tokens * p->top_k >= (1ll << 30))
        return MOE_ERR_UNSUPPORTED;
    if (p->path != MOE_PATH_AUTO && p->path != MOE_PATH_DIRECT && p->path != MOE_PATH_SORTED)
        return MOE_ERR_UNSUPPORTED;
    if (p->path == MOE_PATH_DIRECT && p->num_tokens * p->top_k > MOE_DIRECT_MAX_ROUTES)
        return MOE_ERR_UNSUPPORTED;
    if (p->dtype != MOE_DTYPE_BF16 && p->dtype != MOE_DTYPE_F16)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_routing(const moe_params_t *p, int bias_given)
{
    if (!p)
        return MOE_ERR_NULL;
    if (p->scoring != MOE_SCORING_SOFTMAX && p->scoring != MOE_SCORING_SIGMOID)
        return MOE_ERR_UNSUPPORTED;
    if (p->renormalize != 0 && p->renormalize != 1)
        return MOE_ERR_UNSUPPORTED;
    const int ng = p->num_expert_group, tg = p->topk_group;
    if (ng < 1 || ng > kMaxGroups || tg < 1 || tg > ng || p->num_experts % ng != 0)
        return MOE_ERR_UNSUPPORTED;
    if (p->top_k > tg * (p->num_experts / ng))
        return MOE_ERR_UNSUPPORTED;
    if (p->scoring == MOE_SCORING_SOFTMAX && (bias_given || ng > 1))
        return MOE_ERR_UNSUPPORTED;
    if (!(p->routed_scaling_factor == p->routed_scaling_factor))  // NaN
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_shared(int32_t S)
{
    if (S < 0)
        return MOE_ERR_SHAPE;
    if (S > 0 && S % 64 != 0)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

void make_plan(const moe_params_t *p, int32_t S, Plan *pl, int wfmt)
{
    pl->T = p->num_tokens;
    pl->H = p->hidden;
    pl->E = p->num_experts;
    pl->F = p->inter;
    pl->k = p->top_k;
    pl->S = S;
    pl->P = pl->T * pl->k;
    pl->dtype = p->dtype;
    const int P = pl->P;
    const double mean_rows = (double)P / (double)pl->E;
    if (p->path == MOE_PATH_AUTO)
        pl->path = (P <= MOE_DIRECT_MAX_ROUTES && mean_rows <= 8.0) ? MOE_PATH_DIRECT
                                                                   : MOE_PATH_SORTED;
    else
        pl->path = p->path;
    // Kernel and tile by routed rows per expert, T*k/E (density tiers, as the FlashInfer
    // BF16-activation PR picks its route tiles); shapes measured on MI355X.  Few rows per
    // expert (decode): the weight-streaming kernel, one 16-column tile per wave for gate-up,
    // two for down, K split over four waves, 16-row passes.  Tens of rows (batch): the
    // row-tiled kernel, activation tile shared through LDS, 64-row tiles.  Hundreds (prefill):
    // the 256 x 256 tile kernel, both operands loaded straight into LDS.  The dense shared
    // expert: the 256 x 256 tile kernel for both GEMMs, the tiles past the last whole round
    // over the CUs split along K.
    if (pl->path == MOE_PATH_DIRECT) {
        pl->gate_up = {KERNEL_WS, 1, 1, 4, 3};
        pl->down = {KERNEL_WS, 2, 1, P <= 64 ? 4 : 2, P <= 64 ? 2 : 3};
    } else if (mean_rows <= 8.0) {
        pl->gate_up = {KERNEL_WS, 1, 1, 4, 3};
        pl->down = {KERNEL_WS, 2, 1, 4, 2};
    } else if (mean_rows <= 64.0) {
        // the down GEMM's short K loop keeps one k-step ahead once the tiles are well filled,
        // with four 16-column tiles per wave (qwen3-235b batch, 32 rows per expert: two tiles
        // two steps ahead 0.341, one step ahead 0.330, four tiles one step ahead 0.310 ms);
        // sparser tiles need the deeper prefetch (Kimi-K2 at 512 tokens, 11 rows: 1.03 ms with
        // two tiles two steps ahead, 1.07 one step ahead, 1.10 with four tiles).  The gate-up
        // GEMM takes two 16-column tiles (32 gate and 32 up rows per wave) one k-step ahead:
        // with the expert-major tile order, 16 rows per expert at DeepSeek-V3 and Kimi-K2
        // dimensions 2.765 -> 2.736 and 2.479 -> 2.439 ms per pass against one tile two steps
        // ahead, Qwen3-235B batch unchanged
        pl->gate_up = {KERNEL_TILED, 2, 4, 1, 2};
        pl->down = mean_rows >= 24.0 ? TileChoice{KERNEL_TILED, 4, 4, 1, 2}
                                     : TileChoice{KERNEL_TILED, 2, 4, 1, 3};
    } else {
        pl->gate_up = {KERNEL_WIDE, 0, 16, 1, 2};
        pl->down = {KERNEL_WIDE, 0, 16, 1, 2};
    }
    if (wfmt == WEIGHTS_MXFP4) {
        // MXFP4 weights (W4A16): the weight-streaming form with 16-row passes up to 8 routed
        // rows per expert, the row-tiled form (64-row tiles, each weight byte feeding 64 rows)
        // up to 64 (48 with grouped routing), the 256 x 256 tile with the codes dequantised
        // into its MFMA operands above (both K, H and F, whole groups of 256).  256 x 256
        // against 64-row tiles, Qwen3-235B dimensions (softmax routing): 56 rows per expert
        // 0.795 against 0.658 ms, 64 rows 0.829 against 0.759, 80 and 96 rows even; DeepSeek-V3
        // and Kimi-K2 dimensions with grouped routing, whose busiest experts take hundreds of
        // rows (the 256-row tile streams their weights once per 256 rows): 64 rows 2.91 against
        // 3.13 ms and 2.79 against 3.07.  The row-tiled down GEMM keeps one k-step ahead (its K
        // loop is short: Qwen3-235B batch 0.515 -> 0.503 ms, 16 rows per expert at Kimi-K2 and
        // DeepSeek-V3 dimensions 1.593 -> 1.565 and 1.636 -> 1.607 ms against two steps ahead).
        if (pl->path == MOE_PATH_DIRECT || mean_rows <= 8.0) {
            pl->gate_up = {KERNEL_MX, 1, 1, 2, 3};
            pl->down = {KERNEL_MX, 2, 1, 2, 3};
        } else if (mean_rows > (p->num_expert_group > 1 ? 48.0 : 64.0) && pl->H % 256 == 0 &&
                   pl->F % 256 == 0) {
            pl->gate_up = {KERNEL_MX_WIDE, 0, 16, 1, 2};
            pl->down = {KERNEL_MX_WIDE, 0, 16, 1, 2};
        } else {
            pl->gate_up = {KERNEL_MX_TILED, 1, 4, 1, 3};
            pl->down = {KERNEL_MX_TILED, 2, 4, 1, 2};
        }
    }
    pl->shared_gate_up = {KERNEL_WIDE, 0, 16, 1, 2};
    pl->shared_down = {KERNEL_WIDE, 0, 16, 1, 2};
    // The shared expert's GEMMs take three eighths of the resident workgroup slots, and the
    // fused entry runs them on a second stream beside the routed GEMMs, which fill the rest
    // (Kimi-K2 at 512 tokens, align + routed GEMMs + shared expert: one stream 3.494 ms; two
    // streams with the shared GEMMs on all slots 3.452, on 2/8 3.360, 3/8 3.338, 4/8 3.382).
    // The stage-by-stage form uses the same share, so both give the same bits.
    pl->shared_slot_eighths = S > 0 ? 3 : 0;
    pl->block_m = (pl->gate_up.kind == KERNEL_WS || pl->gate_up.kind == KERNEL_MX)
                      ? kSortedBlockM
                      : 16 * pl->gate_up.mt;
    // 256-row tiles: an expert's routes spread evenly over its tiles, so that the tiles of a
    // heavy expert (which read the same weight rows) run at the same pace and share those
    // rows in L2, instead of a ragged last tile streaming them on its own
    pl->balanced = pl->gate_up.kind == KERNEL_WIDE || pl->gate_up.kind == KERNEL_MX_WIDE;
    pl->slots = P + pl->E * (pl->block_m - 1);
    pl->tiles_cap = P / pl->block_m + pl->E;

    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    pl->off_ids = take((size_t)P * 4);
    pl->off_weights = take((size_t)P * 4);
    if (pl->path == MOE_PATH_SORTED) {
        pl->off_sorted = take((size_t)pl->slots * 4);
        pl->off_offsets = take((size_t)(pl->E + 1) * 4);
        pl->off_tile_expert = take((size_t)pl->tiles_cap * 4);
        pl->off_inverse = take((size_t)P * 4);
        pl->off_n_tiles = take(4);
        // per-XCD tile ranges of the 256 x 256 tile kernel (moe_internal.h's TileSchedule)
        pl->off_sched = pl->balanced ? take(2 * 4 * 9) : 0;
        const size_t scratch = align_scratch_ints(P, pl->E, pl->balanced);
        pl->off_align = scratch ? take(scratch * 4) : 0;
        pl->off_h = take((size_t)pl->slots * pl->F * 2);
    } else {
        pl->off_sorted = pl->off_offsets = pl->off_tile_expert = pl->off_inverse = 0;
        pl->off_sched = 0;
        pl->off_n_tiles = pl->off_align = 0;
        pl->off_h = take((size_t)P * pl->F * 2);
    }
    pl->off_y = take((size_t)P * pl->H * 2);
    if (S > 0) {
        pl->off_hs = take((size_t)pl->T * S * 2);
        pl->off_ys = take((size_t)pl->T * pl->H * 2);
        // f32 partial tiles of the shared expert's K-split 256 x 256 tiles: at most one per
        // workgroup slot (kMaxSplitSlots slots of 256 x 256 f32)
        pl->partial_bytes = (size_t)kMaxSplitSlots * 256 * 256 * 4;
        pl->off_partial = take(pl->partial_bytes);
    } else {
        pl->off_hs = pl->off_ys = 0;
        pl->off_partial = 0;
        pl->partial_bytes = 0;
    }
    pl->total = o;
}

}  // namespace moe
