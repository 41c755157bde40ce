// moe_gemm_tiled.hip -- launches of the row-tiled grouped GEMM (moe_tiled_kernel.h).
#include "moe_tiled_kernel.h"

namespace {

using moe::GemmProblem;

template <bool GATE_UP, int SRC, int BM, int NTW, int STAGES>
void launch_one(const GemmProblem &g, hipStream_t stream)
{
    const int n_blocks = (g.n_out + 16 * NTW * moe_tiled::kWaves - 1) /
                         (16 * NTW * moe_tiled::kWaves);
    const int m_tiles = g.num_groups;
    const int blocks = moe_tiled::tiled_grid(n_blocks, m_tiles);
    if (g.dtype == 1)
        hipLaunchKernelGGL((moe_tiled::k_tiled_gemm<GATE_UP, SRC, BM, NTW, STAGES, 1>),
                           dim3(blocks), dim3(64 * moe_tiled::kWaves), 0, stream, g, n_blocks,
                           m_tiles);
    else
        hipLaunchKernelGGL((moe_tiled::k_tiled_gemm<GATE_UP, SRC, BM, NTW, STAGES, 0>),
                           dim3(blocks), dim3(64 * moe_tiled::kWaves), 0, stream, g, n_blocks,
                           m_tiles);
}

// Instantiated tile shapes (BM rows, NTW 16-column tiles per wave, STAGES), per direction:
// those the host plan picks.
template <bool GATE_UP, int SRC>
bool dispatch(const GemmProblem &g, moe::WsTile t, hipStream_t s)
{
#define MOE_TILED_CASE(BM_, NTW_, ST_)                                                           \
    if (t.mt * 16 == BM_ && t.nt == NTW_ && t.stages == ST_) {                                   \
        launch_one<GATE_UP, SRC, BM_, NTW_, ST_>(g, s);                                          \
        return true;                                                                             \
    }
    if constexpr (GATE_UP) {
        MOE_TILED_CASE(64, 2, 2)
    } else {
        MOE_TILED_CASE(64, 2, 3)
        MOE_TILED_CASE(64, 4, 2)
    }
#undef MOE_TILED_CASE
    return false;
}

}  // namespace

namespace moe {

bool launch_tiled(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
                  hipStream_t stream)
{
    if (src != ROWS_SORTED)
        return false;
    return gate_up ? dispatch<true, ROWS_SORTED>(g, tile, stream)
                   : dispatch<false, ROWS_SORTED>(g, tile, stream);
}

}  // namespace moe
