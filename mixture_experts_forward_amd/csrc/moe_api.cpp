// moe_api.cpp -- the extern "C" entry points declared in include/moe.h.
//
// Each entry point validates everything on the host first (moe_plan.cpp), then enqueues its
// kernels on the caller's stream and returns; no host synchronisation, no device->host copy,
// no allocation.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"
#include "moe_plan.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// A roctx range around one entry point's enqueue, so that a profiler's marker trace shows which
// kernels each forward call launched (a no-op unless a profiler is attached).
struct TraceRange {
    explicit TraceRange(const char *name) { roctxRangePushA(name); }
    ~TraceRange() { roctxRangePop(); }
    TraceRange(const TraceRange &) = delete;
    TraceRange &operator=(const TraceRange &) = delete;
};

// the plan reserves 2 * 4 * 9 bytes for the sorted path's tile schedule
static_assert(sizeof(moe::TileSchedule) <= 2 * 4 * 9, "tile schedule fits its workspace slot");

int launch_status()
{
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

template <typename T>
T *ws_at(void *ws, size_t off)
{
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// Everything one expert-part stage needs.
struct Ctx {
    const uint16_t *hidden, *w_gate_up, *w_down, *s_gu, *s_d;
    const int32_t *ids;
    const float *weights;
    uint16_t *out;
    void *ws;
    hipStream_t stream;
    // MXFP4 expert weights (codes, scales), when the plan uses them
    const uint8_t *gu_q = nullptr, *gu_s = nullptr, *d_q = nullptr, *d_s = nullptr;
};

// The GEMM problems of a plan (sorted layout, when used, lives in the workspace).
moe::GemmProblem gate_up_problem(const moe::Plan &pl, const Ctx &c)
{
    moe::GemmProblem g = {};
    g.act = c.hidden;
    g.weight = c.w_gate_up;
    g.out = ws_at<uint16_t>(c.ws, pl.off_h);
    g.topk_ids = c.ids;
    g.K = pl.H;
    g.n_out = pl.F;
    g.top_k = pl.k;
    g.P = pl.P;
    g.num_experts = pl.E;
    g.dtype = pl.dtype;
    g.wq = c.gu_q;
    g.wscale = c.gu_s;
    if (pl.path == MOE_PATH_SORTED) {
        g.sorted_ids = ws_at<int32_t>(c.ws, pl.off_sorted);
        g.offsets = ws_at<int32_t>(c.ws, pl.off_offsets);
        g.tile_expert = ws_at<int32_t>(c.ws, pl.off_tile_expert);
        g.sched = pl.off_sched ? ws_at<moe::TileSchedule>(c.ws, pl.off_sched) : nullptr;
        const bool per_expert =
            pl.gate_up.kind == moe::KERNEL_WS || pl.gate_up.kind == moe::KERNEL_MX;
        g.num_groups = per_expert ? pl.E : pl.tiles_cap;
    } else {
        g.num_groups = pl.P <= 64 ? pl.P : pl.E;  // per route (direct) or per expert (scan)
    }
    return g;
}

moe::GemmProblem down_problem(const moe::Plan &pl, const Ctx &c)
{
    moe::GemmProblem g = gate_up_problem(pl, c);
    g.act = ws_at<uint16_t>(c.ws, pl.off_h);
    g.weight = c.w_down;
    g.wq = c.d_q;
    g.wscale = c.d_s;
    g.out = ws_at<uint16_t>(c.ws, pl.off_y);
    g.K = pl.F;
    g.n_out = pl.H;
    return g;
}

moe::GemmProblem shared_problem(const moe::Plan &pl, const Ctx &c, bool gate_up)
{
    moe::GemmProblem g = {};
    const moe::TileChoice &t = gate_up ? pl.shared_gate_up : pl.shared_down;
    g.act = gate_up ? c.hidden : ws_at<uint16_t>(c.ws, pl.off_hs);
    g.weight = gate_up ? c.s_gu : c.s_d;
    g.out = ws_at<uint16_t>(c.ws, gate_up ? pl.off_hs : pl.off_ys);
    g.K = gate_up ? pl.H : pl.S;
    g.n_out = gate_up ? pl.S : pl.H;
    g.top_k = 1;
    g.rows = pl.T;
    g.num_experts = 1;
    g.dtype = pl.dtype;
    g.num_groups = (pl.T + 16 * t.mt - 1) / (16 * t.mt);
    g.slot_eighths = pl.shared_slot_eighths;
    if (pl.off_partial) {
        g.partial = ws_at<float>(c.ws, pl.off_partial);
        g.partial_bytes = pl.partial_bytes;
    }
    return g;
}

moe::WsTile ws_tile(const moe::TileChoice &t) { return moe::WsTile{t.nt, t.mt, t.ksplit, t.stages}; }

bool launch_gemm(bool gate_up, const moe::GemmProblem &g, moe::RowSource src,
                 const moe::TileChoice &t, hipStream_t stream)
{
    if (t.kind == moe::KERNEL_TILED)
        return moe::launch_tiled(gate_up, g, src, ws_tile(t), stream);
    if (t.kind == moe::KERNEL_WIDE)
        return moe::launch_wide(gate_up, g, src, stream);
    if (t.kind == moe::KERNEL_MX)
        return moe::launch_mx(gate_up, g, src, ws_tile(t), stream);
    if (t.kind == moe::KERNEL_MX_TILED)
        return moe::launch_mx_tiled(gate_up, g, src, ws_tile(t), stream);
    if (t.kind == moe::KERNEL_MX_WIDE)
        return moe::launch_wide_mx(gate_up, g, src, stream);
    return gate_up ? moe::launch_gate_up(g, src, ws_tile(t), stream)
                   : moe::launch_down(g, src, ws_tile(t), stream);
}

int run_stage(int stage, const moe::Plan &pl, const Ctx &c)
{
    const moe::RowSource src = pl.path == MOE_PATH_SORTED ? moe::ROWS_SORTED
                               : pl.P <= 64                ? moe::ROWS_DIRECT
                                                           : moe::ROWS_SCAN;
    switch (stage) {
    case MOE_STAGE_ALIGN:
        if (pl.path == MOE_PATH_SORTED)
            moe::launch_align_sort(c.ids, pl.P, pl.E, pl.block_m,
                                   ws_at<int32_t>(c.ws, pl.off_sorted),
                                   ws_at<int32_t>(c.ws, pl.off_offsets),
                                   ws_at<int32_t>(c.ws, pl.off_tile_expert),
                                   ws_at<int32_t>(c.ws, pl.off_inverse),
                                   ws_at<int32_t>(c.ws, pl.off_n_tiles),
                                   pl.off_align ? ws_at<int32_t>(c.ws, pl.off_align) : nullptr,
                                   c.stream,
                                   pl.off_sched ? ws_at<moe::TileSchedule>(c.ws, pl.off_sched)
                                                : nullptr,
                                   pl.balanced);
        break;
    case MOE_STAGE_GATE_UP:
        if (!launch_gemm(true, gate_up_problem(pl, c), src, pl.gate_up, c.stream))
            return MOE_ERR_LAUNCH;
        break;
    case MOE_STAGE_DOWN:
        if (!launch_gemm(false, down_problem(pl, c), src, pl.down, c.stream))
            return MOE_ERR_LAUNCH;
        break;
    case MOE_STAGE_SHARED:
        if (pl.S <= 0)
            return MOE_ERR_UNSUPPORTED;
        if (!launch_gemm(true, shared_problem(pl, c, true), moe::ROWS_DENSE, pl.shared_gate_up,
                         c.stream) ||
            !launch_gemm(false, shared_problem(pl, c, false), moe::ROWS_DENSE, pl.shared_down,
                         c.stream))
            return MOE_ERR_LAUNCH;
        break;
    case MOE_STAGE_COMBINE:
        moe::launch_combine(ws_at<uint16_t>(c.ws, pl.off_y), c.ids, c.weights,
                            pl.S > 0 ? ws_at<uint16_t>(c.ws, pl.off_ys) : nullptr, c.out, pl.T,
                            pl.H, pl.k, pl.E, pl.dtype, c.stream);
        break;
    default:
        return MOE_ERR_UNSUPPORTED;
    }
    return launch_status();
}

// Routed experts (+ shared expert) and the combine, with the routing already in ids/weights
// (and, if first_stage is past MOE_STAGE_ALIGN, the sorted layout already in the workspace).
int experts_impl(const moe::Plan &pl, const Ctx &c, int first_stage = MOE_STAGE_ALIGN)
{
    for (int stage = first_stage; stage <= MOE_STAGE_COMBINE; ++stage) {
        if (stage == MOE_STAGE_SHARED && pl.S == 0)
            continue;
        const int st = run_stage(stage, pl, c);
        if (st != MOE_OK)
            return st;
    }
    return MOE_OK;
}

// A second stream per device for the shared expert's GEMMs, with the two events that fork it
// from and join it to the caller's stream.  Created on first use (default priority,
// non-blocking), kept until the process ends.  The mutex is held over a whole fork-join
// enqueue, so calls from several host threads never interleave their records and waits on
// these shared events.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// The side stream of the device of `stream` (g_side_mu held), or nullptr if it cannot be made.
SideStream *side_stream_locked(hipStream_t stream)
{
    int dev = 0;
    if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    SideStream &ss = g_side[dev];
    if (ss.stream && ss.fork && ss.join)
        return &ss;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess))
        return nullptr;
    bool ok = true;
    if (!ss.stream)
        ok = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) == hipSuccess;
    if (ok && !ss.fork)
        ok = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess;
    if (ok && !ss.join)
        ok = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
    if (cur != dev)
        (void)hipSetDevice(cur);
    (void)hipGetLastError();
    return ok ? &ss : nullptr;
}

// MXFP4 weights (the plan of the bf16 pass with the MXFP4 GEMM for both expert GEMMs):
// bf16 activations, H and F multiples of 128 (whole 128-element k-steps)
int mx_check(const moe_params_t *p)
{
    int st = moe::check_dims(p);
    if (st != MOE_OK)
        return st;
    if (p->dtype != MOE_DTYPE_BF16 || p->hidden % 128 != 0 || p->inter % 128 != 0)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int fused_impl(const uint16_t *hidden, const float *gating, const uint16_t *w_gate_up,
               const uint16_t *w_down, const float *bias, const uint16_t *s_gu,
               const uint16_t *s_d, int32_t S, const moe_params_t *p, uint16_t *out,
               int32_t *ids_out, float *weights_out, void *ws, size_t ws_bytes, void *stream)
{
    int st = moe::check_dims(p);
    if (st != MOE_OK)
        return st;
    if ((st = moe::check_routing(p, bias != nullptr)) != MOE_OK)
        return st;
    if ((st = moe::check_shared(S)) != MOE_OK)
        return st;
    if (p->num_tokens == 0)
        return MOE_OK;  // empty tensors may have NULL data pointers
    if (!hidden || !gating || !w_gate_up || !w_down || !out)
        return MOE_ERR_NULL;
    if (S > 0 && (!s_gu || !s_d))
        return MOE_ERR_NULL;
    moe::Plan pl;
    moe::make_plan(p, S, &pl);
    if (!ws)
        return MOE_ERR_NULL;
    if (ws_bytes < pl.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(hidden) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(out) ||
        !aligned16(ws) || (S > 0 && (!aligned16(s_gu) || !aligned16(s_d))))
        return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);

    int32_t *ids = ids_out ? ids_out : ws_at<int32_t>(ws, pl.off_ids);
    float *weights = weights_out ? weights_out : ws_at<float>(ws, pl.off_weights);
    const Ctx c = {hidden, w_gate_up, w_down, s_gu, s_d, ids, weights, out, ws, s};
    const int sigmoid = p->scoring == MOE_SCORING_SIGMOID;
    auto route = [&] {
        moe::launch_route(gating, bias, pl.T, pl.E, pl.k, sigmoid, p->renormalize,
                          p->num_expert_group, p->topk_group, p->routed_scaling_factor, ids,
                          weights, s);
    };
    if (S > 0) {
        // The shared expert needs only hidden_states: it forks off before the routing and
        // runs on the side stream, on its share of the CUs, beside route, align and the
        // routed GEMMs; the combine (which adds its rows) waits for it.  Without a side
        // stream the same kernels run in order on the caller's stream.
        std::lock_guard<std::mutex> lock(g_side_mu);
        if (SideStream *ss = side_stream_locked(s)) {
            if (hipEventRecord(ss->fork, s) != hipSuccess ||
                hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess)
                return MOE_ERR_LAUNCH;
            Ctx side = c;
            side.stream = ss->stream;
            int st = run_stage(MOE_STAGE_SHARED, pl, side);
            // the side stream is joined back whatever happens (a capture stays whole)
            const bool rec = hipEventRecord(ss->join, ss->stream) == hipSuccess;
            if (st == MOE_OK) {
                route();
                for (int stage : {MOE_STAGE_ALIGN, MOE_STAGE_GATE_UP, MOE_STAGE_DOWN})
                    if (st == MOE_OK)
                        st = run_stage(stage, pl, c);
            }
            if (!rec || hipStreamWaitEvent(s, ss->join, 0) != hipSuccess)
                return MOE_ERR_LAUNCH;
            return st == MOE_OK ? run_stage(MOE_STAGE_COMBINE, pl, c) : st;
        }
    }
    route();
    return experts_impl(pl, c);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK:
        return "ok";
    case MOE_ERR_NULL:
        return "a required pointer is NULL";
    case MOE_ERR_SHAPE:
        return "invalid size (non-positive dimension or top_k > num_experts)";
    case MOE_ERR_UNSUPPORTED:
        return "unsupported combination of arguments";
    case MOE_ERR_WORKSPACE:
        return "workspace too small";
    case MOE_ERR_LAUNCH:
        return "kernel launch failed";
    default:
        return "unknown status";
    }
}

int moe_check_params(const moe_params_t *p, int correction_bias_given, int32_t shared_inter)
{
    int st = moe::check_dims(p);
    if (st == MOE_OK)
        st = moe::check_routing(p, correction_bias_given);
    if (st == MOE_OK)
        st = moe::check_shared(shared_inter);
    return st;
}

int moe_route(const float *gating_output, const float *correction_bias, const moe_params_t *p,
              int32_t *topk_ids, float *topk_weights, void *stream)
{
    if (!p)
        return MOE_ERR_NULL;
    if (p->num_tokens < 0 || p->num_experts <= 0 || p->top_k <= 0 ||
        p->top_k > p->num_experts)
        return MOE_ERR_SHAPE;
    if (p->top_k > moe::kMaxTopK || p->num_experts > moe::kMaxExperts)
        return MOE_ERR_UNSUPPORTED;
    int st = moe::check_routing(p, correction_bias != nullptr);
    if (st != MOE_OK)
        return st;
    if (p->num_tokens == 0)
        return MOE_OK;
    if (!gating_output || !topk_ids || !topk_weights)
        return MOE_ERR_NULL;
    moe::launch_route(gating_output, correction_bias, p->num_tokens, p->num_experts, p->top_k,
                      p->scoring == MOE_SCORING_SIGMOID, p->renormalize, p->num_expert_group,
                      p->topk_group, p->routed_scaling_factor, topk_ids, topk_weights,
                      static_cast<hipStream_t>(stream));
    return launch_status();
}

namespace {

// moe_align_sort's argument checks shared with its workspace query
int align_args(int32_t T, int32_t k, int32_t E, int32_t block_m)
{
    if (T < 0 || k < 1 || E < 1)
        return MOE_ERR_SHAPE;
    if (E > moe::kMaxExperts || block_m < 1 || block_m > 1024 || (int64_t)T * k >= (1ll << 30))
        return MOE_ERR_UNSUPPORTED;
    if (((int64_t)T * k + (int64_t)E * (block_m - 1)) >= (1ll << 31))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

size_t moe_align_sort_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t block_m)
{
    if (align_args(T, k, E, block_m) != MOE_OK)
        return 0;
    return moe::align_scratch_ints(T * k, E) * 4;
}

int moe_align_sort(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                   int32_t *sorted_route_ids, int32_t *expert_offsets, int32_t *tile_expert,
                   int32_t *inverse_pos, int32_t *n_tiles, void *workspace,
                   size_t workspace_bytes, void *stream)
{
    int st = align_args(T, k, E, block_m);
    if (st != MOE_OK)
        return st;
    if (!sorted_route_ids || !expert_offsets || !tile_expert || !n_tiles ||
        (T > 0 && (!topk_ids || !inverse_pos)))
        return MOE_ERR_NULL;
    const size_t need = moe::align_scratch_ints(T * k, E) * 4;
    if (need > 0) {
        if (workspace_bytes < need)
            return MOE_ERR_WORKSPACE;
        if (!workspace)
            return MOE_ERR_NULL;
        if (((uintptr_t)workspace & 3u) != 0)
            return MOE_ERR_UNSUPPORTED;
    }
    moe::launch_align_sort(topk_ids, T * k, E, block_m, sorted_route_ids, expert_offsets,
                           tile_expert, inverse_pos, n_tiles,
                           need > 0 ? static_cast<int32_t *>(workspace) : nullptr,
                           static_cast<hipStream_t>(stream));
    return launch_status();
}

size_t fused_moe_workspace_bytes(const moe_params_t *p, int32_t shared_inter)
{
    if (moe::check_dims(p) != MOE_OK || moe::check_shared(shared_inter) != MOE_OK)
        return 0;
    if (p->num_tokens == 0)
        return 0;
    moe::Plan pl;
    moe::make_plan(p, shared_inter, &pl);
    return pl.total;
}

int fused_moe_fwd(const uint16_t *hidden_states, const float *gating_output,
                  const uint16_t *w_gate_up, const uint16_t *w_down,
                  const float *correction_bias, const moe_params_t *p, uint16_t *out,
                  int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                  size_t workspace_bytes, void *stream)
{
    const TraceRange range("fused_moe_fwd");
    return fused_impl(hidden_states, gating_output, w_gate_up, w_down, correction_bias, nullptr,
                      nullptr, 0, p, out, topk_ids_out, topk_weights_out, workspace,
                      workspace_bytes, stream);
}

int fused_moe_shared_fwd(const uint16_t *hidden_states, const float *gating_output,
                         const uint16_t *w_gate_up, const uint16_t *w_down,
                         const float *correction_bias, const uint16_t *shared_w_gate_up,
                         const uint16_t *shared_w_down, int32_t shared_inter,
                         const moe_params_t *p, uint16_t *out, int32_t *topk_ids_out,
                         float *topk_weights_out, void *workspace, size_t workspace_bytes,
                         void *stream)
{
    const TraceRange range("fused_moe_shared_fwd");
    if (shared_inter == 0)
        return MOE_ERR_SHAPE;
    return fused_impl(hidden_states, gating_output, w_gate_up, w_down, correction_bias,
                      shared_w_gate_up, shared_w_down, shared_inter, p, out, topk_ids_out,
                      topk_weights_out, workspace, workspace_bytes, stream);
}

size_t fused_moe_mxfp4_workspace_bytes(const moe_params_t *p)
{
    if (mx_check(p) != MOE_OK || p->num_tokens == 0)
        return 0;
    moe::Plan pl;
    moe::make_plan(p, 0, &pl, moe::WEIGHTS_MXFP4);
    return pl.total;
}

int fused_moe_mxfp4_fwd(const uint16_t *hidden_states, const float *gating_output,
                        const uint8_t *w_gate_up_q, const uint8_t *w_gate_up_scale,
                        const uint8_t *w_down_q, const uint8_t *w_down_scale,
                        const float *correction_bias, const moe_params_t *p, uint16_t *out,
                        int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    const TraceRange range("fused_moe_mxfp4_fwd");
    int st = mx_check(p);
    if (st != MOE_OK)
        return st;
    if ((st = moe::check_routing(p, correction_bias != nullptr)) != MOE_OK)
        return st;
    if (p->num_tokens == 0)
        return MOE_OK;
    if (!hidden_states || !gating_output || !w_gate_up_q || !w_gate_up_scale || !w_down_q ||
        !w_down_scale || !out || !workspace)
        return MOE_ERR_NULL;
    moe::Plan pl;
    moe::make_plan(p, 0, &pl, moe::WEIGHTS_MXFP4);
    if (workspace_bytes < pl.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(hidden_states) || !aligned16(w_gate_up_q) || !aligned16(w_down_q) ||
        !aligned4(w_gate_up_scale) || !aligned4(w_down_scale) || !aligned16(out) ||
        !aligned16(workspace))
        return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t *ids = topk_ids_out ? topk_ids_out : ws_at<int32_t>(workspace, pl.off_ids);
    float *weights = topk_weights_out ? topk_weights_out : ws_at<float>(workspace, pl.off_weights);
    Ctx c = {hidden_states, nullptr, nullptr, nullptr, nullptr, ids, weights, out, workspace, s};
    c.gu_q = w_gate_up_q;
    c.gu_s = w_gate_up_scale;
    c.d_q = w_down_q;
    c.d_s = w_down_scale;
    moe::launch_route(gating_output, correction_bias, pl.T, pl.E, pl.k,
                      p->scoring == MOE_SCORING_SIGMOID, p->renormalize, p->num_expert_group,
                      p->topk_group, p->routed_scaling_factor, ids, weights, s);
    return experts_impl(pl, c);
}

// ---- the FP8 pass: routed rows quantised per 1 x 128 group, block-scaled FP8 expert GEMMs on
// the contiguous (tight, expert-ordered) layout
// The direct form (T * k <= 64 routes, one launch per GEMM straight from topk_ids) or the
// sorted one (align, quantisers, contiguous GEMMs).
struct Fp8Pass {
    int T, H, E, F, k, P;
    bool direct;
    size_t off_ids, off_weights, off_sorted, off_offsets, off_tile_expert, off_inverse,
        off_n_tiles, off_align, off_aq, off_as, off_gu, off_hq, off_hs, off_h, off_y, total;
};

constexpr int kFp8DirectMaxRoutes = 64;

static bool fp8_direct_fits(const moe_params_t *p)
{
    return p->num_tokens * p->top_k <= kFp8DirectMaxRoutes &&
           moe::fp8_direct_shape_ok(p->hidden) && moe::fp8_direct_shape_ok(p->inter);
}

static int fp8_check(const moe_params_t *p)
{
    int st = moe::check_dims(p);
    if (st != MOE_OK)
        return st;
    if (p->dtype != MOE_DTYPE_BF16 || p->hidden % 128 != 0 || p->inter % 128 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (p->path == MOE_PATH_DIRECT && p->num_tokens > 0 && !fp8_direct_fits(p))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

static void fp8_plan(const moe_params_t *p, Fp8Pass *f)
{
    f->T = p->num_tokens;
    f->H = p->hidden;
    f->E = p->num_experts;
    f->F = p->inter;
    f->k = p->top_k;
    f->P = f->T * f->k;
    // AUTO: direct while the routes are few, both absolutely and per expert
    f->direct = p->path == MOE_PATH_DIRECT ||
                (p->path == MOE_PATH_AUTO && fp8_direct_fits(p) && f->P <= 8 * f->E);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = (o + bytes + 255) / 256 * 256;
        return at;
    };
    const size_t P = f->P;
    f->off_ids = take(P * 4);
    f->off_weights = take(P * 4);
    if (f->direct) {
        f->off_sorted = f->off_offsets = f->off_tile_expert = f->off_inverse = 0;
        f->off_n_tiles = f->off_align = f->off_aq = f->off_as = f->off_gu = 0;
        f->off_hq = f->off_hs = 0;
        f->off_h = take(P * f->F * 2);
        f->off_y = take(P * f->H * 2);
        f->total = o;
        return;
    }
    f->off_h = 0;
    f->off_sorted = take(P * 4);                      // block_m 1: no padding slots
    f->off_offsets = take((size_t)(f->E + 1) * 4);
    f->off_tile_expert = take((P + f->E) * 4);
    f->off_inverse = take(P * 4);
    f->off_n_tiles = take(4);
    const size_t scratch = moe::align_scratch_ints(f->P, f->E);
    f->off_align = scratch ? take(scratch * 4) : 0;
    f->off_aq = take((size_t)f->T * f->H);  // each token's x row quantised once
    f->off_as = take((size_t)f->T * (f->H / 128) * 4);
    f->off_gu = take(P * 2 * f->F * 2);
    f->off_hq = take(P * f->F);
    f->off_hs = take(P * (f->F / 128) * 4);
    f->off_y = take(P * f->H * 2);
    f->total = o;
}

// One stage of the FP8 pass's expert part (the routing in ids / weights).
static void fp8_stage(int stage, const Fp8Pass &f, const uint16_t *hidden, const uint8_t *w_gu,
               const float *s_gu, const uint8_t *w_d, const float *s_d, const int32_t *ids,
               const float *weights, uint16_t *out, void *ws, hipStream_t s)
{
    if (f.direct) {
        uint16_t *h = ws_at<uint16_t>(ws, f.off_h);
        uint16_t *y = ws_at<uint16_t>(ws, f.off_y);
        switch (stage) {
        case MOE_STAGE_GATE_UP:
            moe::launch_fp8_direct(true, hidden, ids, f.P, f.k, f.E, w_gu, s_gu, f.F, f.H, h, s);
            break;
        case MOE_STAGE_DOWN:
            moe::launch_fp8_direct(false, h, ids, f.P, f.k, f.E, w_d, s_d, f.H, f.F, y, s);
            break;
        case MOE_STAGE_COMBINE:  // y row of route (t, j) is t * k + j
            moe::launch_combine(y, ids, weights, nullptr, out, f.T, f.H, f.k, f.E,
                                MOE_DTYPE_BF16, s);
            break;
        default:  // MOE_STAGE_ALIGN: nothing to do
            break;
        }
        return;
    }
    int32_t *sorted = ws_at<int32_t>(ws, f.off_sorted);
    int32_t *offsets = ws_at<int32_t>(ws, f.off_offsets);
    int32_t *inverse = ws_at<int32_t>(ws, f.off_inverse);
    uint8_t *aq = ws_at<uint8_t>(ws, f.off_aq);
    float *as = ws_at<float>(ws, f.off_as);
    uint16_t *gu = ws_at<uint16_t>(ws, f.off_gu);
    uint8_t *hq = ws_at<uint8_t>(ws, f.off_hq);
    float *hs = ws_at<float>(ws, f.off_hs);
    uint16_t *y = ws_at<uint16_t>(ws, f.off_y);
    switch (stage) {
    case MOE_STAGE_ALIGN:
        // expert order, tight (block 1): rows [offsets[e], offsets[e+1]) are expert e's routes;
        // then every token's x row quantised once (a route's row is its token's)
        moe::launch_align_sort(ids, f.P, f.E, 1, sorted, offsets,
                               ws_at<int32_t>(ws, f.off_tile_expert), inverse,
                               ws_at<int32_t>(ws, f.off_n_tiles),
                               f.off_align ? ws_at<int32_t>(ws, f.off_align) : nullptr, s);
        moe::launch_quant_fp8(hidden, f.T, f.H, aq, as, s);
        break;
    case MOE_STAGE_GATE_UP:
        // contiguous row q (the route sorted[q]) reads its token's codes, sorted[q] / k
        moe::launch_fp8_gemm_contig(aq, as, w_gu, s_gu, offsets, f.E, f.P, 2 * f.F, f.H, gu, s,
                                    sorted, f.k);
        break;
    case MOE_STAGE_DOWN:
        moe::launch_quant_fp8_swiglu(gu, f.P, f.F, hq, hs, s);
        moe::launch_fp8_gemm_contig(hq, hs, w_d, s_d, offsets, f.E, f.P, f.H, f.F, y, s);
        break;
    case MOE_STAGE_COMBINE:
        moe::launch_combine(y, ids, weights, nullptr, out, f.T, f.H, f.k, f.E, MOE_DTYPE_BF16, s,
                            inverse);
        break;
    default:
        break;
    }
}

int fused_moe_experts_fwd(const uint16_t *hidden_states, const uint16_t *w_gate_up,
                          const uint16_t *w_down, const int32_t *topk_ids,
                          const float *topk_weights, const moe_params_t *p, uint16_t *out,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    const TraceRange range("fused_moe_experts_fwd");
    int st = moe::check_dims(p);
    if (st != MOE_OK)
        return st;
    if (p->num_tokens == 0)
        return MOE_OK;
    if (!hidden_states || !w_gate_up || !w_down || !topk_ids || !topk_weights || !out)
        return MOE_ERR_NULL;
    moe::Plan pl;
    moe::make_plan(p, 0, &pl);
    if (!workspace)
        return MOE_ERR_NULL;
    if (workspace_bytes < pl.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(hidden_states) || !aligned16(w_gate_up) || !aligned16(w_down) ||
        !aligned16(out) || !aligned16(workspace))
        return MOE_ERR_UNSUPPORTED;
    const Ctx c = {hidden_states, w_gate_up, w_down, nullptr, nullptr, topk_ids, topk_weights,
                   out, workspace, static_cast<hipStream_t>(stream)};
    return experts_impl(pl, c);
}

int fused_moe_experts_stage(int stage, const uint16_t *hidden_states, const uint16_t *w_gate_up,
                            const uint16_t *w_down, const int32_t *topk_ids,
                            const float *topk_weights, const uint16_t *shared_w_gate_up,
                            const uint16_t *shared_w_down, int32_t shared_inter,
                            const moe_params_t *p, uint16_t *out, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    int st = moe::check_dims(p);
    if (st != MOE_OK)
        return st;
    if ((st = moe::check_shared(shared_inter)) != MOE_OK)
        return st;
    if (stage < MOE_STAGE_ALIGN || stage > MOE_STAGE_COMBINE ||
        (stage == MOE_STAGE_SHARED && shared_inter == 0))
        return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0)
        return MOE_OK;
    const bool need_x = stage == MOE_STAGE_GATE_UP || stage == MOE_STAGE_SHARED;
    if (!workspace || !topk_ids || (need_x && !hidden_states) ||
        (stage == MOE_STAGE_GATE_UP && !w_gate_up) || (stage == MOE_STAGE_DOWN && !w_down) ||
        (stage == MOE_STAGE_SHARED && (!shared_w_gate_up || !shared_w_down)) ||
        (stage == MOE_STAGE_COMBINE && (!topk_weights || !out)))
        return MOE_ERR_NULL;
    moe::Plan pl;
    moe::make_plan(p, shared_inter, &pl);
    if (workspace_bytes < pl.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace) || (hidden_states && !aligned16(hidden_states)) ||
        (w_gate_up && !aligned16(w_gate_up)) || (w_down && !aligned16(w_down)) ||
        (out && !aligned16(out)) || (shared_w_gate_up && !aligned16(shared_w_gate_up)) ||
        (shared_w_down && !aligned16(shared_w_down)))
        return MOE_ERR_UNSUPPORTED;
    const Ctx c = {hidden_states, w_gate_up, w_down, shared_w_gate_up, shared_w_down, topk_ids,
                   topk_weights, out, workspace, static_cast<hipStream_t>(stream)};
    return run_stage(stage, pl, c);
}

int fused_moe_mxfp4_stage(int stage, const uint16_t *hidden_states, const uint8_t *w_gate_up_q,
                          const uint8_t *w_gate_up_scale, const uint8_t *w_down_q,
                          const uint8_t *w_down_scale, const int32_t *topk_ids,
                          const float *topk_weights, const moe_params_t *p, uint16_t *out,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    int st = mx_check(p);
    if (st != MOE_OK)
        return st;
    if (stage < MOE_STAGE_ALIGN || stage > MOE_STAGE_COMBINE || stage == MOE_STAGE_SHARED)
        return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0)
        return MOE_OK;
    if (!workspace || !topk_ids || (stage == MOE_STAGE_GATE_UP && !hidden_states) ||
        (stage == MOE_STAGE_GATE_UP && (!w_gate_up_q || !w_gate_up_scale)) ||
        (stage == MOE_STAGE_DOWN && (!w_down_q || !w_down_scale)) ||
        (stage == MOE_STAGE_COMBINE && (!topk_weights || !out)))
        return MOE_ERR_NULL;
    moe::Plan pl;
    moe::make_plan(p, 0, &pl, moe::WEIGHTS_MXFP4);
    if (workspace_bytes < pl.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace) || (hidden_states && !aligned16(hidden_states)) ||
        (w_gate_up_q && !aligned16(w_gate_up_q)) || (w_down_q && !aligned16(w_down_q)) ||
        !aligned4(w_gate_up_scale) || !aligned4(w_down_scale) || (out && !aligned16(out)))
        return MOE_ERR_UNSUPPORTED;
    Ctx c = {hidden_states, nullptr, nullptr, nullptr, nullptr, topk_ids, topk_weights, out,
             workspace, static_cast<hipStream_t>(stream)};
    c.gu_q = w_gate_up_q;
    c.gu_s = w_gate_up_scale;
    c.d_q = w_down_q;
    c.d_s = w_down_scale;
    return run_stage(stage, pl, c);
}

size_t fused_moe_fp8_workspace_bytes(const moe_params_t *p)
{
    if (fp8_check(p) != MOE_OK || p->num_tokens == 0)
        return 0;
    Fp8Pass f;
    fp8_plan(p, &f);
    return f.total;
}

int fused_moe_fp8_fwd(const uint16_t *hidden_states, const float *gating_output,
                      const uint8_t *w_gate_up, const float *w_gate_up_scale,
                      const uint8_t *w_down, const float *w_down_scale,
                      const float *correction_bias, const moe_params_t *p, uint16_t *out,
                      int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    const TraceRange range("fused_moe_fp8_fwd");
    int st = fp8_check(p);
    if (st != MOE_OK)
        return st;
    if ((st = moe::check_routing(p, correction_bias != nullptr)) != MOE_OK)
        return st;
    if (p->num_tokens == 0)
        return MOE_OK;
    if (!hidden_states || !gating_output || !w_gate_up || !w_gate_up_scale || !w_down ||
        !w_down_scale || !out || !workspace)
        return MOE_ERR_NULL;
    Fp8Pass f;
    fp8_plan(p, &f);
    if (workspace_bytes < f.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(hidden_states) || !aligned16(w_gate_up) || !aligned16(w_down) ||
        !aligned16(out) || !aligned16(workspace) || ((uintptr_t)w_gate_up_scale & 3u) ||
        ((uintptr_t)w_down_scale & 3u))
        return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = workspace;
    int32_t *ids = topk_ids_out ? topk_ids_out : ws_at<int32_t>(ws, f.off_ids);
    float *weights = topk_weights_out ? topk_weights_out : ws_at<float>(ws, f.off_weights);
    moe::launch_route(gating_output, correction_bias, f.T, f.E, f.k,
                      p->scoring == MOE_SCORING_SIGMOID, p->renormalize, p->num_expert_group,
                      p->topk_group, p->routed_scaling_factor, ids, weights, s);
    for (int stage : {MOE_STAGE_ALIGN, MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_COMBINE})
        fp8_stage(stage, f, hidden_states, w_gate_up, w_gate_up_scale, w_down, w_down_scale, ids,
                  weights, out, ws, s);
    return launch_status();
}

int fused_moe_fp8_stage(int stage, const uint16_t *hidden_states, const uint8_t *w_gate_up,
                        const float *w_gate_up_scale, const uint8_t *w_down,
                        const float *w_down_scale, const int32_t *topk_ids,
                        const float *topk_weights, const moe_params_t *p, uint16_t *out,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    int st = fp8_check(p);
    if (st != MOE_OK)
        return st;
    if (stage < MOE_STAGE_ALIGN || stage > MOE_STAGE_COMBINE || stage == MOE_STAGE_SHARED)
        return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens == 0)
        return MOE_OK;
    Fp8Pass f;
    fp8_plan(p, &f);
    const int x_stage = f.direct ? MOE_STAGE_GATE_UP : MOE_STAGE_ALIGN;
    if (!workspace || !topk_ids || (stage == x_stage && !hidden_states) ||
        (stage == MOE_STAGE_GATE_UP && (!w_gate_up || !w_gate_up_scale)) ||
        (stage == MOE_STAGE_DOWN && (!w_down || !w_down_scale)) ||
        (stage == MOE_STAGE_COMBINE && (!topk_weights || !out)))
        return MOE_ERR_NULL;
    if (workspace_bytes < f.total)
        return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace) || (hidden_states && !aligned16(hidden_states)) ||
        (w_gate_up && !aligned16(w_gate_up)) || (w_down && !aligned16(w_down)) ||
        (out && !aligned16(out)) || ((uintptr_t)w_gate_up_scale & 3u) ||
        ((uintptr_t)w_down_scale & 3u))
        return MOE_ERR_UNSUPPORTED;
    fp8_stage(stage, f, hidden_states, w_gate_up, w_gate_up_scale, w_down, w_down_scale,
              topk_ids, topk_weights, out, workspace, static_cast<hipStream_t>(stream));
    return launch_status();
}

}  // extern "C"

// ---------------------------------------------------------------- masked layout

namespace {

// The masked rows as a routed problem: E * max_m single-route tokens, sorted path.
int masked_plan(int32_t E, int32_t max_m, int32_t H, int32_t F, moe::Plan *pl)
{
    if (E < 1 || max_m < 0 || H < 1 || F < 1)
        return MOE_ERR_SHAPE;
    if ((int64_t)E * max_m >= (1ll << 30))
        return MOE_ERR_UNSUPPORTED;
    moe_params_t p = {};
    p.num_tokens = E * max_m;
    p.hidden = H;
    p.num_experts = E;
    p.inter = F;
    p.top_k = 1;
    p.scoring = MOE_SCORING_SOFTMAX;
    p.renormalize = 0;
    p.num_expert_group = 1;
    p.topk_group = 1;
    p.routed_scaling_factor = 1.0f;
    p.path = MOE_PATH_SORTED;
    const int st = moe::check_dims(&p);
    if (st != MOE_OK)
        return st;
    if (max_m > 0)
        moe::make_plan(&p, 0, pl);
    return MOE_OK;
}

// The routed plan's workspace up to (not including) its expert-output rows: the masked pass
// writes those rows straight to out.
size_t masked_bytes(const moe::Plan &pl) { return pl.off_y; }

int masked_run(int first, int last, const uint16_t *a, const int32_t *masked_m,
               const uint16_t *w_gate_up, const uint16_t *w_down, int32_t E, int32_t max_m,
               int32_t H, int32_t F, uint16_t *out, void *ws, size_t ws_bytes, void *stream)
{
    moe::Plan pl;
    int st = masked_plan(E, max_m, H, F, &pl);
    if (st != MOE_OK)
        return st;
    if (max_m == 0)
        return MOE_OK;
    const bool align = first <= MOE_STAGE_ALIGN, gate_up = first <= MOE_STAGE_GATE_UP &&
                                                           last >= MOE_STAGE_GATE_UP;
    const bool down = last >= MOE_STAGE_DOWN;
    if (!ws || (align && !masked_m) || (gate_up && (!a || !w_gate_up)) ||
        (down && (!w_down || !out)))
        return MOE_ERR_NULL;
    if (ws_bytes < masked_bytes(pl))
        return MOE_ERR_WORKSPACE;
    if (!aligned16(ws) || (a && !aligned16(a)) || (w_gate_up && !aligned16(w_gate_up)) ||
        (w_down && !aligned16(w_down)) || (out && !aligned16(out)))
        return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t *ids = ws_at<int32_t>(ws, pl.off_ids);
    const Ctx c = {a, w_gate_up, w_down, nullptr, nullptr, ids, nullptr, out, ws, s};
    if (align) {
        moe::launch_masked_ids(masked_m, E, max_m, ids, s);
        if ((st = run_stage(MOE_STAGE_ALIGN, pl, c)) != MOE_OK)
            return st;
    }
    if (gate_up && (st = run_stage(MOE_STAGE_GATE_UP, pl, c)) != MOE_OK)
        return st;
    if (down) {
        moe::GemmProblem g = down_problem(pl, c);
        g.out = out;  // row q of the flattened blocks is written in place
        if (!launch_gemm(false, g, moe::ROWS_SORTED, pl.down, s))
            return MOE_ERR_LAUNCH;
    }
    return launch_status();
}

}  // namespace

extern "C" {

size_t fused_moe_masked_workspace_bytes(int32_t E, int32_t max_m, int32_t H, int32_t F)
{
    moe::Plan pl;
    if (masked_plan(E, max_m, H, F, &pl) != MOE_OK || max_m == 0)
        return 0;
    return masked_bytes(pl);
}

int fused_moe_masked_fwd(const uint16_t *a, const int32_t *masked_m, const uint16_t *w_gate_up,
                         const uint16_t *w_down, int32_t E, int32_t max_m, int32_t H, int32_t F,
                         uint16_t *out, void *workspace, size_t workspace_bytes, void *stream)
{
    const TraceRange range("fused_moe_masked_fwd");
    return masked_run(MOE_STAGE_ALIGN, MOE_STAGE_DOWN, a, masked_m, w_gate_up, w_down, E, max_m,
                      H, F, out, workspace, workspace_bytes, stream);
}

int fused_moe_masked_stage(int stage, const uint16_t *a, const int32_t *masked_m,
                           const uint16_t *w_gate_up, const uint16_t *w_down, int32_t E,
                           int32_t max_m, int32_t H, int32_t F, uint16_t *out, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    if (stage != MOE_STAGE_ALIGN && stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN)
        return MOE_ERR_UNSUPPORTED;
    return masked_run(stage, stage, a, masked_m, w_gate_up, w_down, E, max_m, H, F, out,
                      workspace, workspace_bytes, stream);
}

int moe_grouped_gemm_fp8(const uint8_t *a, const float *a_scale, const uint8_t *b,
                         const float *b_scale, const int32_t *masked_m, int32_t E, int32_t max_m,
                         int32_t N, int32_t K, uint16_t *out, void *stream)
{
    if (E < 1 || max_m < 0 || N < 1 || K < 1)
        return MOE_ERR_SHAPE;
    // the launch covers E * ceil(max_m / 64) row tiles per 256-column block
    if (N % 64 != 0 || K % 128 != 0 || (int64_t)E * max_m >= (1ll << 30) ||
        (int64_t)E * N >= (1ll << 30) ||
        (int64_t)E * ((max_m + 63) / 64) * ((N + 255) / 256) >= (1ll << 30))
        return MOE_ERR_UNSUPPORTED;
    if (max_m == 0)
        return MOE_OK;
    if (!a || !a_scale || !b || !b_scale || !masked_m || !out)
        return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out) || ((uintptr_t)a_scale & 3u) ||
        ((uintptr_t)b_scale & 3u))
        return MOE_ERR_UNSUPPORTED;
    moe::launch_fp8_gemm(a, a_scale, b, b_scale, masked_m, E, max_m, N, K, out,
                         static_cast<hipStream_t>(stream));
    return launch_status();
}

int moe_grouped_gemm_fp8_contiguous(const uint8_t *a, const float *a_scale, const uint8_t *b,
                                    const float *b_scale, const int32_t *expert_offsets,
                                    int32_t E, int32_t P, int32_t N, int32_t K, uint16_t *out,
                                    void *stream)
{
    if (E < 1 || P < 0 || N < 1 || K < 1)
        return MOE_ERR_SHAPE;
    // the launch covers at most (ceil(P / 64) + E) row tiles per 256-column block
    if (N % 64 != 0 || K % 128 != 0 || E > 1024 || P >= (1 << 30) ||
        (int64_t)E * N >= (1ll << 30) ||
        ((int64_t)(P + 63) / 64 + E) * ((N + 255) / 256) >= (1ll << 30))
        return MOE_ERR_UNSUPPORTED;
    if (P == 0)
        return MOE_OK;
    if (!a || !a_scale || !b || !b_scale || !expert_offsets || !out)
        return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out) || ((uintptr_t)a_scale & 3u) ||
        ((uintptr_t)b_scale & 3u) || ((uintptr_t)expert_offsets & 3u))
        return MOE_ERR_UNSUPPORTED;
    moe::launch_fp8_gemm_contig(a, a_scale, b, b_scale, expert_offsets, E, P, N, K, out,
                                static_cast<hipStream_t>(stream));
    return launch_status();
}

int moe_quant_fp8(const uint16_t *x, int32_t M, int32_t K, uint8_t *q, float *scale,
                  void *stream)
{
    if (M < 0 || K < 1)
        return MOE_ERR_SHAPE;
    if (K % 8 != 0 || (int64_t)M * ((K + 127) / 128) >= (1ll << 34))
        return MOE_ERR_UNSUPPORTED;
    if (M == 0)
        return MOE_OK;
    if (!x || !q || !scale)
        return MOE_ERR_NULL;
    if (!aligned16(x) || ((uintptr_t)q & 7u) || ((uintptr_t)scale & 3u))
        return MOE_ERR_UNSUPPORTED;
    moe::launch_quant_fp8(x, M, K, q, scale, static_cast<hipStream_t>(stream));
    return launch_status();
}

int moe_stream_read_sink_words(void) { return moe::stream_read_grid(); }

int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (bytes == 0)
        return MOE_OK;
    if (!buf || !sink)
        return MOE_ERR_NULL;
    if (!aligned16(buf) || bytes % 16 != 0)
        return MOE_ERR_UNSUPPORTED;
    moe::launch_stream_read(buf, bytes, sink, moe::stream_read_grid(),
                            static_cast<hipStream_t>(stream));
    return launch_status();
}

}  // extern "C"
