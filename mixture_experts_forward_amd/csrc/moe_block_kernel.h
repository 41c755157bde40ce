// moe_block_kernel.h -- 128-row block GEMM of the MoE experts for compute-heavy shapes
// (prefill experts with hundreds of routed rows, the dense shared expert).
//
// Same math as moe_ws_kernel.h (gate-up with the SiLU(gate)*up epilogue, or down).  Built for
// MFMA throughput while still streaming the weights once per 128-row tile:
//   - a workgroup (4 waves, 2 x 2) owns a 128-row tile and BW = 32*TN weight rows; wave
//     (wm, wn) computes rows [64*wm, 64*wm+64) x weight rows [16*TN*wn, 16*TN*(wn+1)) with
//     4 x TN accumulators of v_mfma_f32_16x16x32_bf16 -- every operand read from LDS feeds TN
//     (or 4) MFMAs;
//   - both operand tiles of a 64-element k-step (128 rows x 128 B activations, BW rows x 128 B
//     weights) are loaded cooperatively, each wave instruction covering 8 rows x 128 B (whole
//     lines), STAGES-1 k-steps ahead in registers, and written to a double-buffered,
//     XOR-swizzled LDS tile -- one barrier per k-step.  Weights use ordinary cached loads: the
//     row tiles of one expert re-read them from L2 (non-temporal loads measured slower here);
//   - for gate-up, a wave's weight rows are TN/2 gate tiles and the TN/2 up tiles of the same
//     columns, so SiLU(gate)*up is applied in registers;
//   - tiles are numbered so that workgroups sharing data are neighbours, and blocks are dealt
//     round-robin to the 8 XCDs, each XCD taking a contiguous range of tile numbers per round
//     (see k_block_gemm).  Sorted rows are numbered expert by expert -- column block by
//     column block, the expert's row tiles within -- and all tiles of one expert start their K
//     loop at the same k-step; dense rows number the row tiles of a column block
//     consecutively, which start at the same k-step.  Different experts / column blocks start
//     at different k-steps, spreading the requests over the HBM channels.
//   - the same kernel runs on a plain grid (one tile per workgroup: sorted rows, where that
//     measured faster) or a persistent one (one workgroup per resident slot, walking the
//     tiles in rounds: dense rows, whose row tiles then run in step and share each weight
//     k-slice through L2).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe_block {

using moe::GemmProblem;

constexpr int kWaves = 4;
constexpr int kXcds = 8;
constexpr int kBM = 128;

// Grid of a launch: the resident workgroup slots (a multiple of 8), or fewer when the launch
// has fewer tiles (total_cap: an upper bound of the tile count).
inline int block_grid(int total_cap, int slots)
{
    const int cap = (total_cap + kXcds - 1) / kXcds * kXcds;
    const int s = slots / kXcds * kXcds;
    return cap < kXcds ? kXcds : (s < kXcds ? kXcds : (cap < s ? cap : s));
}

__device__ __forceinline__ moe_u32x4 load_cached(const uint16_t *p)
{
    return *reinterpret_cast<const moe_u32x4 *>(p);
}

// slot of 16-byte chunk c of row r in a swizzled 8-slot row
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Number of tiles of a launch: sorted rows -> the routing's row tiles (read from the layout)
// x column blocks; dense rows -> m_tiles x column blocks.
template <int SRC>
__device__ __forceinline__ int block_total(const GemmProblem &g, int n_blocks, int m_tiles)
{
    if (SRC == moe::ROWS_SORTED)
        return g.offsets[g.num_experts] / kBM * n_blocks;
    return m_tiles * n_blocks;
}

// Tile number t -> (column block, row tile, expert).  Sorted rows: expert-major (an expert's
// tiles are consecutive, column block by column block, its row tiles within); t / n_blocks
// falls inside the expert's own row tiles, so tile_expert names it.  Dense rows: row tiles of
// a column block consecutive.
template <int SRC>
__device__ __forceinline__ void block_decode(const GemmProblem &g, int t, int n_blocks,
                                             int m_tiles, int &nblk, int &mtile, int &expert)
{
    if (SRC == moe::ROWS_SORTED) {
        expert = g.tile_expert[t / n_blocks];
        const int t0 = g.offsets[expert] / kBM;
        const int te = g.offsets[expert + 1] / kBM - t0;
        const int local = t - t0 * n_blocks;
        nblk = local / te;
        mtile = t0 + local % te;
    } else {
        nblk = t / m_tiles;
        mtile = t % m_tiles;
        expert = 0;
    }
}

// One 128-row x BW-weight-row tile: K loop and epilogue.
template <bool GATE_UP, int SRC, int TN, int STAGES, int DT>
__device__ __forceinline__ void block_tile(const GemmProblem &g, int nblk, int mtile, int expert,
                                           moe_u32x4 (*s_x)[kBM * 8],
                                           moe_u32x4 (*s_w)[32 * TN * 8])
{
    constexpr int BW = 32 * TN;        // weight rows per workgroup
    constexpr int XL = kBM / 32;       // activation loads per thread per k-step
    constexpr int WL = BW / 32;        // weight loads per thread per k-step
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;
    const int row0 = mtile * kBM;
    const int n_rows = SRC == moe::ROWS_SORTED ? kBM : min(kBM, g.rows - row0);
    const int K = g.K;
    // output columns of this workgroup: gate-up BW/2 (gate and up rows), down BW
    const int cols_per_wg = GATE_UP ? BW / 2 : BW;
    const int col_wg = nblk * cols_per_wg;

    // ---- cooperative loads: thread covers chunk tid%8 of rows tid/8 + 32*i
    const int lrow = tid >> 3, lchunk = tid & 7;
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const uint16_t *W = g.weight + (size_t)expert * w_rows * K;
    const uint16_t *wld[WL];
#pragma unroll
    for (int i = 0; i < WL; ++i) {
        const int r = lrow + 32 * i;  // weight row within the workgroup's BW rows
        // gate-up: rows [0, BW/2) are gate rows of the workgroup's columns, [BW/2, BW) the
        // up rows of the same columns
        const int c = col_wg + (GATE_UP ? r % (BW / 2) : r);
        const bool ok = c < g.n_out;
        const int src = (GATE_UP && r >= BW / 2) ? c + g.n_out : c;
        wld[i] = W + (size_t)(ok ? src : 0) * K + 8 * lchunk;
    }
    const uint16_t *xld[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int r = lrow + 32 * i;
        int src = -1;
        if (SRC == moe::ROWS_SORTED) {
            const int route = g.sorted_ids[row0 + r];
            if (route >= 0)
                src = GATE_UP ? route / g.top_k : row0 + r;
        } else if (r < n_rows) {
            src = row0 + r;
        }
        // an unused row reads row 0: its column of the result is never stored
        xld[i] = g.act + (size_t)(src < 0 ? 0 : src) * K + 8 * lchunk;
    }

    // ---- operand rows of this wave
    // weight tile n of wave wn: gate-up: n < TN/2 -> gate rows 16*(TN/2)*wn + 16*n of the gate
    // half; n >= TN/2 -> the matching up rows.  down: rows 16*TN*wn + 16*n.
    int wrow0[TN];
#pragma unroll
    for (int n = 0; n < TN; ++n) {
        if (GATE_UP) {
            const int hn = n % (TN / 2);
            const int base = 16 * (TN / 2) * wn + 16 * hn;
            wrow0[n] = (n < TN / 2) ? base : BW / 2 + base;
        } else {
            wrow0[n] = 16 * TN * wn + 16 * n;
        }
    }
    const int rr = lane & 15, rq = lane >> 4;

    // K-loop start: the same for workgroups that share tiles through L2 (they then read each
    // k-slice at about the same time): per expert (sorted rows), else per column block
    const int nk = K / 64;
    const unsigned rkey = SRC == moe::ROWS_SORTED ? expert : nblk;
    const int rot = (int)((rkey * 7u) % (unsigned)nk);

    moe_f32x4 acc[4][TN];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
            acc[m][n] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

    moe_u32x4 wraw[STAGES][WL], xraw[STAGES][XL];
    // rows past the last column read row 0 of the expert: their (never stored) columns are the
    // only ones they affect, so loads and LDS stores stay unconditional
    auto load = [&](int st, int i) {
        const int k = ((i + rot) % nk) * 64;
#pragma unroll
        for (int j = 0; j < WL; ++j)
            wraw[st][j] = load_cached(wld[j] + k);
#pragma unroll
        for (int j = 0; j < XL; ++j)
            xraw[st][j] = load_cached(xld[j] + k);
    };
    auto compute = [&](int st, int i) {
        moe_u32x4 *xb = s_x[i & 1];
        moe_u32x4 *wb = s_w[i & 1];
#pragma unroll
        for (int j = 0; j < WL; ++j)
            wb[swz(lrow + 32 * j, lchunk)] = wraw[st][j];
#pragma unroll
        for (int j = 0; j < XL; ++j)
            xb[swz(lrow + 32 * j, lchunk)] = xraw[st][j];
        __syncthreads();
        moe_u32x4 a[TN][2];
#pragma unroll
        for (int n = 0; n < TN; ++n) {
            const int r = wrow0[n] + rr;
            a[n][0] = wb[swz(r, rq)];
            a[n][1] = wb[swz(r, rq + 4)];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = 64 * wm + 16 * m + rr;
            const moe_u32x4 b0 = xb[swz(r, rq)];
            const moe_u32x4 b1 = xb[swz(r, rq + 4)];
            // the two halves of k are issued TN MFMAs apart: no back-to-back dependency
#pragma unroll
            for (int n = 0; n < TN; ++n)
                acc[m][n] = moe_mma16<DT>(a[n][0], b0, acc[m][n]);
#pragma unroll
            for (int n = 0; n < TN; ++n)
                acc[m][n] = moe_mma16<DT>(a[n][1], b1, acc[m][n]);
        }
    };

    // Software pipeline, STAGES-1 k-steps in flight.  The steady state is branch-free so that
    // the compiler's wait counts stay exact: past the end, the prefetch wraps to an early
    // k-step (in bounds, never consumed).
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        load(st, st);
    int i = 0;
    for (; i + STAGES <= nk; i += STAGES) {
#pragma unroll
        for (int st = 0; st < STAGES; ++st) {
            load((st + STAGES - 1) % STAGES, i + st + STAGES - 1);
            compute(st, i + st);
        }
    }
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (i + st < nk)
            compute(st, i + st);

    // ---- epilogue: lane holds columns 4*(lane/16)+q of row 16*m + lane%16 of each tile
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r = 64 * wm + 16 * m + rr;
        int dst = -1;
        if (SRC == moe::ROWS_SORTED) {
            const int route = g.sorted_ids[row0 + r];
            if (route >= 0)
                dst = GATE_UP ? row0 + r : route;
        } else if (r < n_rows) {
            dst = row0 + r;
        }
        if (dst < 0)
            continue;
        uint16_t *orow = g.out + (size_t)dst * g.n_out;
        constexpr int NOUT = GATE_UP ? TN / 2 : TN;
#pragma unroll
        for (int n = 0; n < NOUT; ++n) {
            const int col = GATE_UP ? col_wg + 16 * (TN / 2) * wn + 16 * n
                                    : col_wg + 16 * TN * wn + 16 * n;
            if (col >= g.n_out)
                continue;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (GATE_UP) {
                    const float gate = acc[m][n][q];
                    const float up = acc[m][n + TN / 2][q];
                    v[q] = gate / (1.0f + __expf(-gate)) * up;
                } else {
                    v[q] = acc[m][n][q];
                }
            }
            moe_u32x2 packed;
            packed.x = moe_pack2<DT>(v[0], v[1]);
            packed.y = moe_pack2<DT>(v[2], v[3]);
            *reinterpret_cast<moe_u32x2 *>(orow + col + 4 * rq) = packed;
        }
    }
}

// Persistent grid (gridDim.x a multiple of 8): round r hands XCD x the tiles
// [r*W + x*W/8, r*W + (x+1)*W/8), W = the slots in use.
template <bool GATE_UP, int SRC, int TN, int STAGES, int DT>
__global__ __launch_bounds__(64 * kWaves) void k_block_gemm(GemmProblem g, int n_blocks,
                                                           int m_tiles)
{
    static_assert(!GATE_UP || TN % 2 == 0, "gate-up pairs gate and up tiles");
    __shared__ moe_u32x4 s_x[2][kBM * 8];
    __shared__ moe_u32x4 s_w[2][32 * TN * 8];

    const int total = block_total<SRC>(g, n_blocks, m_tiles);
    // fewer tiles than slots: spread them evenly over the XCDs
    const int W = min((int)gridDim.x, (total + kXcds - 1) / kXcds * kXcds);
    const int per = W / kXcds;
    const int idx = blockIdx.x / kXcds;
    if (idx >= per)
        return;
    for (int t = (blockIdx.x % kXcds) * per + idx; t < total; t += W) {
        int nblk, mtile, expert;
        block_decode<SRC>(g, t, n_blocks, m_tiles, nblk, mtile, expert);
        block_tile<GATE_UP, SRC, TN, STAGES, DT>(g, nblk, mtile, expert, s_x, s_w);
        __syncthreads();  // the next tile's first LDS stores follow every wave's last reads
    }
}

}  // namespace moe_block
