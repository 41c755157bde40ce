// moe_gemm_wide.hip -- launches of the 256 x 256 tile GEMM (moe_wide_kernel.h).
#include <algorithm>

#include "moe_wide_kernel.h"

namespace {

using moe::GemmProblem;

// Workgroups of `kernel` resident on one CU (found once per instantiation).
template <typename Kernel>
int per_cu(Kernel kernel)
{
    static const int n = [&] {
        int blocks = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, moe_wide::kThreads,
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

template <bool GATE_UP, int SRC, int DT>
void launch_typed(const GemmProblem &g_in, hipStream_t stream)
{
    const auto kernel = moe_wide::k_wide_gemm<GATE_UP, SRC, 3, DT>;
    const int cols = GATE_UP ? moe_wide::kBW / 2 : moe_wide::kBW;  // output columns per tile
    const int n_blocks = (g_in.n_out + cols - 1) / cols;
    const int m_tiles = g_in.num_groups;
    // dense rows, and sorted rows with a schedule: one workgroup per resident slot; sorted rows
    // without one: one tile per workgroup
    const bool persistent = SRC == moe::ROWS_DENSE || g_in.sched != nullptr;
    int slots = persistent ? per_cu(kernel) * device_cus() : (1 << 30);
    if (SRC == moe::ROWS_DENSE && g_in.slot_eighths > 0)  // a share of the chip, the rest
        slots = std::max(moe_wide::kXcds,                 // left to work on another stream
                         slots * g_in.slot_eighths / 8 / moe_wide::kXcds * moe_wide::kXcds);
    const int total = n_blocks * m_tiles;
    GemmProblem g = g_in;
    g.split_tiles = g.split_parts = 0;
    if (SRC == moe::ROWS_DENSE && g.partial != nullptr) {
        // the tiles past the last whole round over the slots (all of them if there are fewer
        // tiles than slots) are split along K so the last round keeps every slot busy
        const int n_split = total < slots ? total : total % slots;
        int q = n_split > 0 ? slots / n_split : 0;
        q = std::min(q, g.K / moe_wide::kStep);
        q = std::min<long long>(q, (long long)(g.partial_bytes /
                                               ((size_t)n_split * moe::kWidePartialBytes + 1)));
        if (n_split > 0 && q >= 2) {
            g.split_tiles = n_split;
            g.split_parts = q;
        } else {
            g.partial = nullptr;
        }
    }
    const int units = g.partial ? moe_wide::wide_split_units(total, g.split_tiles, g.split_parts)
                                : total;
    const int grid = moe_wide::wide_grid(units, slots);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(moe_wide::kThreads), 0, stream, g, n_blocks,
                       m_tiles);
    if (g.partial) {
        const int c8 = (GATE_UP ? moe_wide::kBW / 2 : moe_wide::kBW) / 8;
        const int threads = g.split_tiles * moe_wide::kBM * c8;
        hipLaunchKernelGGL((moe_wide::k_wide_reduce<GATE_UP, DT>), dim3((threads + 255) / 256),
                           dim3(256), 0, stream, g, n_blocks, m_tiles, total);
    }
}

template <bool GATE_UP, int SRC>
void launch_one(const GemmProblem &g, hipStream_t stream)
{
    if (g.dtype == 1)
        launch_typed<GATE_UP, SRC, 1>(g, stream);
    else
        launch_typed<GATE_UP, SRC, 0>(g, stream);
}

template <bool GATE_UP>
void launch_mx_typed(const GemmProblem &g, hipStream_t stream)
{
    const auto kernel = moe_wide::k_wide_mx<GATE_UP>;
    const int cols = GATE_UP ? moe_wide::kBW / 2 : moe_wide::kBW;
    const int n_blocks = (g.n_out + cols - 1) / cols;
    const int m_tiles = g.num_groups;
    const int grid = moe_wide::wide_grid(n_blocks * m_tiles, per_cu(kernel) * device_cus());
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(moe_wide::kThreads), 0, stream, g, n_blocks,
                       m_tiles);
}

}  // namespace

namespace moe {

bool launch_wide_mx(bool gate_up, const GemmProblem &g, RowSource src, hipStream_t stream)
{
    // sorted rows with a schedule; K a multiple of 256 (whole scale groups of 4 k-steps)
    if (src != ROWS_SORTED || g.sched == nullptr || g.K % 256 != 0)
        return false;
    if (gate_up)
        launch_mx_typed<true>(g, stream);
    else
        launch_mx_typed<false>(g, stream);
    return true;
}

bool launch_wide(bool gate_up, const GemmProblem &g, RowSource src, hipStream_t stream)
{
    if (src == ROWS_SORTED) {
        if (gate_up)
            launch_one<true, ROWS_SORTED>(g, stream);
        else
            launch_one<false, ROWS_SORTED>(g, stream);
        return true;
    }
    if (src == ROWS_DENSE) {
        if (gate_up)
            launch_one<true, ROWS_DENSE>(g, stream);
        else
            launch_one<false, ROWS_DENSE>(g, stream);
        return true;
    }
    return false;
}

}  // namespace moe
