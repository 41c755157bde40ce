// moe_gemm_ws.hip -- launches of the weight-streaming grouped GEMM (moe_ws_kernel.h).
#include "moe_ws_kernel.h"

namespace {

using moe::GemmProblem;

template <bool GATE_UP, int SRC, int NT, int MT, int KSPLIT, int STAGES, int SEGK>
void launch_seg(const GemmProblem &g, hipStream_t stream)
{
    const dim3 grid((g.n_out + 16 * NT - 1) / (16 * NT), g.num_groups);
    if (g.dtype == 1)
        hipLaunchKernelGGL((moe_ws::k_ws_gemm<GATE_UP, SRC, NT, MT, KSPLIT, STAGES, 1, SEGK>),
                           grid, dim3(64 * KSPLIT), 0, stream, g);
    else
        hipLaunchKernelGGL((moe_ws::k_ws_gemm<GATE_UP, SRC, NT, MT, KSPLIT, STAGES, 0, SEGK>),
                           grid, dim3(64 * KSPLIT), 0, stream, g);
}

// Weight rows a multiple of 4 KB apart stream faster in 256-byte row segments (two k-steps per
// load, one segment in flight: as many bytes ahead as two k-steps of the one-k-step form).
// The form needs every wave's K range to hold whole segments.  Its first compute waits for a
// whole segment, so it pays only on grids of several workgroups per resident slot (MI355X,
// qwen3-30b gate-up: 6144 workgroups 108 -> 106.5 us; one token, 384 workgroups: 19.3 -> 20.6).
constexpr long long kSeg2MinWorkgroups = 2048;
template <bool GATE_UP, int SRC, int NT, int MT, int KSPLIT, int STAGES>
void launch_one(const GemmProblem &g, hipStream_t stream)
{
    const long long wgs = (long long)((g.n_out + 16 * NT - 1) / (16 * NT)) * g.num_groups;
    const bool seg2 = STAGES == 3 && (g.K * 2) % 4096 == 0 && (g.K / 64) % (2 * KSPLIT) == 0 &&
                      wgs >= kSeg2MinWorkgroups;
    if (seg2)
        launch_seg<GATE_UP, SRC, NT, MT, KSPLIT, 2, 2>(g, stream);
    else
        launch_seg<GATE_UP, SRC, NT, MT, KSPLIT, STAGES, 1>(g, stream);
}

// Instantiated tile shapes, per direction.  Every shape the host plan may pick must be
// listed here, and nothing else.
template <bool GATE_UP, int SRC>
bool dispatch(const GemmProblem &g, moe::WsTile t, hipStream_t s)
{
#define MOE_WS_CASE(NT_, MT_, KS_, ST_)                                                          \
    if (t.nt == NT_ && t.mt == MT_ && t.ksplit == KS_ && t.stages == ST_) {                      \
        launch_one<GATE_UP, SRC, NT_, MT_, KS_, ST_>(g, s);                                      \
        return true;                                                                             \
    }
    if constexpr (GATE_UP) {
        MOE_WS_CASE(1, 1, 4, 3)
    } else {
        MOE_WS_CASE(2, 1, 4, 2)
        MOE_WS_CASE(2, 1, 2, 3)
    }
#undef MOE_WS_CASE
    return false;
}

}  // namespace

namespace moe {

static bool launch_any(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
                       hipStream_t stream)
{
    if (gate_up) {
        switch (src) {
        case ROWS_SORTED:
            return dispatch<true, ROWS_SORTED>(g, tile, stream);
        case ROWS_DIRECT:
            return dispatch<true, ROWS_DIRECT>(g, tile, stream);
        case ROWS_SCAN:
            return dispatch<true, ROWS_SCAN>(g, tile, stream);
        default:
            return false;
        }
    }
    switch (src) {
    case ROWS_SORTED:
        return dispatch<false, ROWS_SORTED>(g, tile, stream);
    case ROWS_DIRECT:
        return dispatch<false, ROWS_DIRECT>(g, tile, stream);
    case ROWS_SCAN:
        return dispatch<false, ROWS_SCAN>(g, tile, stream);
    default:
        return false;
    }
}

bool launch_gate_up(const GemmProblem &g, RowSource src, WsTile tile, hipStream_t stream)
{
    return launch_any(true, g, src, tile, stream);
}

bool launch_down(const GemmProblem &g, RowSource src, WsTile tile, hipStream_t stream)
{
    return launch_any(false, g, src, tile, stream);
}

}  // namespace moe
