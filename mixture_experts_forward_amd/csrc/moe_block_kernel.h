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
//     lines; weights non-temporal), STAGES-1 k-steps ahead in registers, and written to a
//     double-buffered, XOR-swizzled LDS tile -- one barrier per k-step;
//   - for gate-up, a wave's weight rows are TN/2 gate tiles and the TN/2 up tiles of the same
//     columns, so SiLU(gate)*up is applied in registers;
//   - blocks are dealt round-robin to the 8 XCDs, so consecutive tile numbers on one XCD run
//     together and share its L2; the row tiles of one column block are numbered consecutively
//     and share its weight tile (numbering the column blocks of one row tile consecutively
//     instead, to keep an activation tile in L2, measured slower on MI355X for both prefill
//     experts and the dense shared expert).  Workgroups that share a weight tile start their
//     K loop at the same k-step; different column blocks start at different k-steps, which
//     spreads the concurrent requests over the HBM channels.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe_block {

using moe::GemmProblem;

constexpr int kWaves = 4;
constexpr int kXcds = 8;
constexpr int kBM = 128;

__host__ __device__ inline int block_grid(int n_blocks, int m_tiles)
{
    const int b = n_blocks * m_tiles;
    return (b + kXcds - 1) / kXcds * kXcds;
}

__device__ __forceinline__ moe_u32x4 load_nt(const uint16_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const moe_u32x4 *>(p));
}

__device__ __forceinline__ moe_u32x4 load_cached(const uint16_t *p)
{
    return *reinterpret_cast<const moe_u32x4 *>(p);
}

// slot of 16-byte chunk c of row r in a swizzled 8-slot row
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <bool GATE_UP, int SRC, int TN, int STAGES>
__global__ __launch_bounds__(64 * kWaves) void k_block_gemm(GemmProblem g, int n_blocks,
                                                           int m_tiles)
{
    constexpr int BW = 32 * TN;        // weight rows per workgroup
    constexpr int XL = kBM / 32;       // activation loads per thread per k-step
    constexpr int WL = BW / 32;        // weight loads per thread per k-step
    static_assert(!GATE_UP || TN % 2 == 0, "gate-up pairs gate and up tiles");
    __shared__ moe_u32x4 s_x[2][kBM * 8];
    __shared__ moe_u32x4 s_w[2][BW * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;

    // ---- tile of this workgroup (XCD-aware order)
    const int per_xcd = block_grid(n_blocks, m_tiles) / kXcds;
    const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= n_blocks * m_tiles)
        return;
    const int nblk = logical / m_tiles;
    const int mtile = logical % m_tiles;
    const int row0 = mtile * kBM;
    int expert = 0, n_rows = kBM;
    if (SRC == moe::ROWS_SORTED) {
        expert = g.tile_expert[mtile];
        if (expert < 0)
            return;
    } else {
        n_rows = min(kBM, g.rows - row0);
        if (n_rows <= 0)
            return;
    }
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

    // K-loop start: the same for the row tiles of one column block (they then read each k-slice
    // of the shared weight tile at about the same time), different across column blocks
    const int nk = K / 64;
    const int rot = (int)((nblk * 7u) % (unsigned)nk);

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
            wraw[st][j] = load_nt(wld[j] + k);
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
                acc[m][n] = moe_mfma_16x16x32(a[n][0], b0, acc[m][n]);
#pragma unroll
            for (int n = 0; n < TN; ++n)
                acc[m][n] = moe_mfma_16x16x32(a[n][1], b1, acc[m][n]);
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
            packed.x = moe_pack_bf16x2(v[0], v[1]);
            packed.y = moe_pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<moe_u32x2 *>(orow + col + 4 * rq) = packed;
        }
    }
}

}  // namespace moe_block
