// moe_tiled_kernel.h -- row-tiled grouped GEMM of the MoE experts for experts that hold tens to
// thousands of routed rows (batch and prefill), and for the dense shared expert.
//
// Same math as moe_ws_kernel.h (gate-up with the SiLU(gate)*up epilogue, or down), organised
// around a BM-row tile of one expert:
//   - the workgroup (4 waves) owns one BM-row tile (rows of one expert's padded segment, padded
//     to BM by moe_align_sort with block_m = BM; or BM consecutive tokens for the shared expert)
//     and 4*NTW 16-column tiles of the output; wave w owns NTW of those column tiles;
//   - each wave streams its own weight rows exactly as the weight-streaming kernel does
//     (non-temporal 128-byte-line loads, STAGES-1 k-steps in registers, per-wave LDS transpose
//     into the MFMA A operand layout), since no other wave uses them;
//   - the BM activation rows of a k-step are loaded once per workgroup (each wave loads a
//     quarter, 8 rows x 128 bytes per instruction) into a double-buffered, XOR-swizzled LDS
//     tile that all four waves read as MFMA B operands -- one barrier per k-step;
//   - sorted rows: tiles are numbered row tile by row tile (expert by expert), so the column
//     blocks of one row tile are consecutive and land on the same XCD (blocks are dealt
//     round-robin to the 8 XCDs, each XCD taking a contiguous range) and re-read the tile's
//     activation rows from that XCD's L2 rather than from HBM; only the real row tiles (the
//     padded segments' total over BM) are dealt out, not the empty slots of the upper bound.
//     At tens of rows per expert an expert has one or two row tiles, so there is little weight
//     sharing to keep, and each expert's activation rows are read once instead of once per
//     column block (Qwen3-235B batch 0.871 -> 0.846 ms, Kimi-K2 with its shared expert 3.408 ->
//     3.363 ms).  Dense rows: the row tiles of a column block consecutive;
//   - every workgroup starts its K loop at a different k-step (rotated), spreading concurrent
//     HBM requests over all channels.
// A lane ends with four consecutive output columns of one row; the gate and up tiles of the
// same columns sit in the same lanes of the same wave.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe_tiled {

using moe::GemmProblem;

__device__ __forceinline__ moe_u32x4 load_nt(const uint16_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const moe_u32x4 *>(p));
}

__device__ __forceinline__ moe_u32x4 load_cached(const uint16_t *p)
{
    return *reinterpret_cast<const moe_u32x4 *>(p);
}

constexpr int kWaves = 4;
constexpr int kXcds = 8;

// Blocks of one launch: n_blocks column blocks x m_tiles row tiles, rounded up to a multiple of
// the XCD count (surplus blocks exit).
__host__ __device__ inline int tiled_grid(int n_blocks, int m_tiles)
{
    const int b = n_blocks * m_tiles;
    return (b + kXcds - 1) / kXcds * kXcds;
}

template <bool GATE_UP, int SRC, int BM, int NTW, int STAGES, int DT>
__global__ __launch_bounds__(64 * kWaves) void k_tiled_gemm(GemmProblem g, int n_blocks,
                                                           int m_tiles)
{
    constexpr int NW = GATE_UP ? 2 * NTW : NTW;  // 16-row weight tiles per wave per k-step
    constexpr int TM = BM / 16;                  // 16-row MFMA tiles of the row tile
    constexpr int XI = BM / (8 * kWaves);        // activation load instructions per wave
    static_assert(BM % (8 * kWaves) == 0, "BM must be a multiple of 32");
    __shared__ moe_u32x4 s_x[2][BM * 8];              // activation tile, 16-byte slots
    __shared__ moe_u32x4 s_t[kWaves][NW * 128];       // per-wave weight transpose buffers

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- tile of this workgroup: XCD-aware order (see the header)
    int nblk, mtile;
    if (SRC == moe::ROWS_SORTED) {
        const int real_tiles = g.offsets[g.num_experts] / BM;
        const int total = real_tiles * n_blocks;
        const int per_xcd = (total + kXcds - 1) / kXcds;
        const int idx = blockIdx.x / kXcds;
        if (idx >= per_xcd)
            return;
        const int logical = (blockIdx.x % kXcds) * per_xcd + idx;
        if (logical >= total)
            return;
        mtile = logical / n_blocks;
        nblk = logical % n_blocks;
    } else {
        const int nb_total = tiled_grid(n_blocks, m_tiles);
        const int per_xcd = nb_total / kXcds;
        const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
        if (logical >= n_blocks * m_tiles)
            return;
        nblk = logical / m_tiles;
        mtile = logical % m_tiles;
    }
    const int row0 = mtile * BM;

    int expert = 0;
    int n_rows = BM;
    if (SRC == moe::ROWS_SORTED) {
        expert = g.tile_expert[mtile];
        if (expert < 0)
            return;  // past the last tile of this routing
    } else {
        n_rows = min(BM, g.rows - row0);
        if (n_rows <= 0)
            return;
    }
    const int K = g.K;
    const int col0 = nblk * (16 * NTW * kWaves) + wv * (16 * NTW);

    // ---- weight rows of this wave: lane reads chunk lane%8 of rows lane/8 and 8 + lane/8
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const uint16_t *W = g.weight + (size_t)expert * w_rows * K;
    const int lrow = lane >> 3, lchunk = lane & 7;
    const uint16_t *wld[NW];
    bool tile_ok[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < g.n_out;
        const int row = (tile_ok[nt] ? c : 0) + lrow;
        wld[nt] = W + (size_t)row * K + 8 * lchunk;
        if (GATE_UP)
            wld[NTW + nt] = W + (size_t)(row + g.n_out) * K + 8 * lchunk;
    }
    moe_u32x4 *tbuf = s_t[wv];
    const int wslot0 = lrow * 8 + (lchunk ^ (lrow >> 1));
    const int wslot1 = (lrow + 8) * 8 + (lchunk ^ ((lrow + 8) >> 1));
    const int rrow = lane & 15, rq = lane >> 4;
    const int rslot0 = rrow * 8 + (rq ^ (rrow >> 1));
    const int rslot1 = rrow * 8 + ((rq + 4) ^ (rrow >> 1));

    // ---- activation rows this lane loads: tile rows wv*BM/4 + 8*i + lane/8, chunk lane%8
    const uint16_t *xld[XI];
    int xslot[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = wv * (BM / kWaves) + 8 * i + lrow;
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
        xslot[i] = r * 8 + (lchunk ^ ((r >> 1) & 7));
    }

    // K-loop start: different across column blocks, so that the column blocks of a row tile,
    // running together, spread their weight requests over the HBM channels (the tile's
    // activation rows stay in L2 whichever k-step each starts at); the same for the row tiles
    // of one column block
    const int nk = K / 64;
    const int rot = (int)((nblk * 7u) % (unsigned)nk);

    moe_f32x4 acc[TM][NW];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
        for (int nw = 0; nw < NW; ++nw)
            acc[mt][nw] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

    moe_u32x4 wraw[STAGES][NW][2], xraw[STAGES][XI];
    auto load = [&](int st, int i) {
        const int k = ((i + rot) % nk) * 64;
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
            wraw[st][nw][0] = load_nt(wld[nw] + k);
            wraw[st][nw][1] = load_nt(wld[nw] + (size_t)8 * K + k);
        }
#pragma unroll
        for (int x = 0; x < XI; ++x)
            xraw[st][x] = load_cached(xld[x] + k);
    };
    auto compute = [&](int st, int i) {
        moe_u32x4 *xb = s_x[i & 1];
#pragma unroll
        for (int x = 0; x < XI; ++x)
            xb[xslot[x]] = xraw[st][x];
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
            tbuf[nw * 128 + wslot0] = wraw[st][nw][0];
            tbuf[nw * 128 + wslot1] = wraw[st][nw][1];
        }
        __syncthreads();  // activation tile complete; also orders this wave's transpose buffer
        moe_u32x4 a[NW][2];
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
            a[nw][0] = tbuf[nw * 128 + rslot0];
            a[nw][1] = tbuf[nw * 128 + rslot1];
        }
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
            const int r = mt * 16 + rrow;
            const int sw = (r >> 1) & 7;
            const moe_u32x4 b0 = xb[r * 8 + (rq ^ sw)];
            const moe_u32x4 b1 = xb[r * 8 + ((rq + 4) ^ sw)];
#pragma unroll
            for (int nw = 0; nw < NW; ++nw)
                acc[mt][nw] = moe_mma16<DT>(a[nw][0], b0, acc[mt][nw]);
#pragma unroll
            for (int nw = 0; nw < NW; ++nw)
                acc[mt][nw] = moe_mma16<DT>(a[nw][1], b1, acc[mt][nw]);
        }
        moe_wave_sync();  // this wave's transpose reads finish before its next writes
    };

    // Software pipeline, STAGES-1 k-steps in flight.  The steady state is branch-free so that
    // the compiler's wait counts stay exact: past the end, the prefetch wraps to an early
    // k-step (in bounds, never consumed).  Weight tiles past the last column read row 0 of the
    // expert (wld is clamped); they only feed columns that are never stored.
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        load(st, st);
    int i = 0;
    for (; i + STAGES <= nk; i += STAGES) {
#pragma unroll
        for (int st = 0; st < STAGES; ++st) {
            load((st + STAGES - 1) % STAGES, i + st + STAGES - 1);
            // keep the next k-step's loads ahead of this step's wait: the scheduler would
            // otherwise sink them below this step's LDS writes, leaving nothing in flight
            // while the wave waits for this step's operands
            __builtin_amdgcn_sched_barrier(0);
            compute(st, i + st);
        }
    }
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (i + st < nk)
            compute(st, i + st);

    // ---- epilogue: lane holds columns 4*(lane/16)+r of row mt*16 + lane%16
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
        const int r = mt * 16 + rrow;
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
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            if (!tile_ok[nt])
                continue;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (GATE_UP) {
                    const float gate = acc[mt][nt][q];
                    const float up = acc[mt][NTW + nt][q];
                    v[q] = gate / (1.0f + __expf(-gate)) * up;
                } else {
                    v[q] = acc[mt][nt][q];
                }
            }
            moe_u32x2 packed;
            packed.x = moe_pack2<DT>(v[0], v[1]);
            packed.y = moe_pack2<DT>(v[2], v[3]);
            *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * rq) = packed;
        }
    }
}

}  // namespace moe_tiled
