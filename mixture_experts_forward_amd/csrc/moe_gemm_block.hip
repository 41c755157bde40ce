// moe_gemm_block.hip -- launches of the 128-row block GEMM (moe_block_kernel.h).
#include "moe_block_kernel.h"

namespace {

using moe::GemmProblem;

// Workgroups of `kernel` resident on one CU (found once per instantiation).
template <typename Kernel>
int per_cu(Kernel kernel)
{
    static const int n = [&] {
        int blocks = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 64 * moe_block::kWaves,
                                                         0) != hipSuccess || blocks < 1)
            blocks = 1;
        return blocks;
    }();
    return n;
}

int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    return n;
}

template <bool GATE_UP, int SRC, int TN, int STAGES, int DT>
void launch_typed(const GemmProblem &g, hipStream_t stream)
{
    const auto kernel = moe_block::k_block_gemm<GATE_UP, SRC, TN, STAGES, DT>;
    const int cols = GATE_UP ? 16 * TN : 32 * TN;  // output columns per workgroup
    const int n_blocks = (g.n_out + cols - 1) / cols;
    const int m_tiles = g.num_groups;
    // sorted rows: one tile per workgroup; dense rows: one workgroup per resident slot
    const int slots = SRC == moe::ROWS_DENSE ? per_cu(kernel) * device_cus() : (1 << 30);
    const int grid = moe_block::block_grid(n_blocks * m_tiles, slots);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * moe_block::kWaves), 0, stream, g, n_blocks,
                       m_tiles);
}

template <bool GATE_UP, int SRC, int TN, int STAGES>
void launch_one(const GemmProblem &g, hipStream_t stream)
{
    if (g.dtype == 1)
        launch_typed<GATE_UP, SRC, TN, STAGES, 1>(g, stream);
    else
        launch_typed<GATE_UP, SRC, TN, STAGES, 0>(g, stream);
}

// Instantiated shapes (TN 16-row weight tiles per wave, STAGES).
template <bool GATE_UP, int SRC>
bool dispatch(const GemmProblem &g, moe::WsTile t, hipStream_t s)
{
#define MOE_BLOCK_CASE(TN_, ST_)                                                                 \
    if (t.nt == TN_ && t.stages == ST_) {                                                        \
        launch_one<GATE_UP, SRC, TN_, ST_>(g, s);                                                \
        return true;                                                                             \
    }
    MOE_BLOCK_CASE(4, 2)
    MOE_BLOCK_CASE(4, 3)
    MOE_BLOCK_CASE(8, 2)
#undef MOE_BLOCK_CASE
    return false;
}

}  // namespace

namespace moe {

bool launch_block(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
                  hipStream_t stream)
{
    if (src != ROWS_SORTED && src != ROWS_DENSE)
        return false;
    if (gate_up)
        return src == ROWS_SORTED ? dispatch<true, ROWS_SORTED>(g, tile, stream)
                                  : dispatch<true, ROWS_DENSE>(g, tile, stream);
    return src == ROWS_SORTED ? dispatch<false, ROWS_SORTED>(g, tile, stream)
                              : dispatch<false, ROWS_DENSE>(g, tile, stream);
}

}  // namespace moe
