// moe_gemm_mx.hip -- launches of the MXFP4-weight GEMM (moe_mx_kernel.h).
#include "moe_mx_kernel.h"

namespace {

using moe::GemmProblem;

template <bool GATE_UP, int SRC, int NT, int KSPLIT, int STAGES>
void launch_one(const GemmProblem &g, hipStream_t stream)
{
    const dim3 grid((g.n_out + 16 * NT - 1) / (16 * NT), g.num_groups);
    hipLaunchKernelGGL((moe_mx::k_mx_gemm<GATE_UP, SRC, NT, KSPLIT, STAGES>), grid,
                       dim3(64 * KSPLIT), 0, stream, g);
}

// Instantiated shapes (NT 16-column tiles per workgroup, KSPLIT waves, STAGES), per
// direction: those the host plan picks.
template <bool GATE_UP, int SRC>
bool dispatch(const GemmProblem &g, moe::WsTile t, hipStream_t s)
{
#define MOE_MX_CASE(NT_, KS_, ST_)                                                               \
    if (t.nt == NT_ && t.ksplit == KS_ && t.stages == ST_) {                                     \
        launch_one<GATE_UP, SRC, NT_, KS_, ST_>(g, s);                                           \
        return true;                                                                             \
    }
    if constexpr (GATE_UP) {
        MOE_MX_CASE(1, 2, 3)
    } else {
        MOE_MX_CASE(2, 2, 3)
    }
#undef MOE_MX_CASE
    return false;
}

template <bool GATE_UP>
bool by_source(const GemmProblem &g, moe::RowSource src, moe::WsTile t, hipStream_t s)
{
    switch (src) {
    case moe::ROWS_SORTED:
        return dispatch<GATE_UP, moe::ROWS_SORTED>(g, t, s);
    case moe::ROWS_DIRECT:
        return dispatch<GATE_UP, moe::ROWS_DIRECT>(g, t, s);
    case moe::ROWS_SCAN:
        return dispatch<GATE_UP, moe::ROWS_SCAN>(g, t, s);
    default:
        return false;
    }
}

template <bool GATE_UP, int NTW, int STAGES>
void launch_tiled_one(const GemmProblem &g, hipStream_t stream)
{
    const int n_blocks = (g.n_out + 16 * NTW * 4 - 1) / (16 * NTW * 4);
    const int m_tiles = g.num_groups;
    const int blocks = moe_tiled::tiled_grid(n_blocks, m_tiles);
    hipLaunchKernelGGL((moe_mx::k_mx_tiled<GATE_UP, NTW, STAGES>), dim3(blocks), dim3(256), 0,
                       stream, g, n_blocks, m_tiles);
}

}  // namespace

namespace moe {

bool launch_mx_tiled(bool gate_up, const GemmProblem &g, RowSource src, WsTile t,
                     hipStream_t stream)
{
    if (src != ROWS_SORTED || t.mt != 4)
        return false;
#define MOE_MXT_CASE(G_, NTW_, ST_)                                                              \
    if (gate_up == G_ && t.nt == NTW_ && t.stages == ST_) {                                      \
        launch_tiled_one<G_, NTW_, ST_>(g, stream);                                              \
        return true;                                                                             \
    }
    MOE_MXT_CASE(true, 1, 3)
    MOE_MXT_CASE(false, 2, 2)
#undef MOE_MXT_CASE
    return false;
}


bool launch_mx(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
               hipStream_t stream)
{
    return gate_up ? by_source<true>(g, src, tile, stream) : by_source<false>(g, src, tile, stream);
}

}  // namespace moe
