// moe_mx_kernel.h -- the expert GEMMs with MXFP4 weights and bf16 activations (W4A16).
//
// Weights in the OCP MX format (block size 32 along K): e2m1 elements, two per byte (element 2i
// in the low nibble of byte i), one E8M0 scale byte 2^(s-127) per 32 consecutive elements of a
// row.  Math as moe_ws_kernel.h (gate-up with SiLU(gate)*up, or down) on the dequantised
// weights; the activations and outputs stay bf16, so a decode step reads a quarter of the bf16
// weight bytes (plus 1/32 byte of scale per element).
//
// Built for the decode shapes it is meant for (weight-bound):
//   - lane l of a wave owns weight row l%16 of each 16-row tile and 32-element block l/16 of each
//     128-element k-step: one 16-byte load (32 codes) and one scale byte per tile
//     and k-step, STAGES-1 k-steps ahead in registers;
//   - the gfx950 conversion v_cvt_scalef32_pk_bf16_fp4 turns a byte into two bf16 values times
//     the block's scale (exact: an e2m1 value has at most two significant bits), sixteen of them
//     giving the lane's four 8-element MFMA A operands -- no LDS transpose;
//   - within a k-step the MFMA's k order is permuted the same way in both operands: MFMA j takes
//     elements 32p + 8j .. 32p + 8j + 7 from lane group p, in the A operand (that lane's own block)
//     and in the activation B operand (loaded to match), so each dot product is unchanged;
//   - row sources, K split over KSPLIT waves (fixed-order LDS sum), rotated K start and the
//     epilogue are those of the bf16 weight-streaming kernel.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_mx_dequant.h"
#include "moe_tiled_kernel.h"
#include "moe_ws_kernel.h"

namespace moe_mx {

using moe::GemmProblem;

template <bool GATE_UP, int SRC, int NT, int KSPLIT, int STAGES>
__global__ __launch_bounds__(64 * KSPLIT) void k_mx_gemm(GemmProblem g)
{
    constexpr int NW = GATE_UP ? 2 * NT : NT;  // 16-row weight tiles per k-step
    __shared__ moe_f32x4 s_red[(KSPLIT > 1 ? KSPLIT - 1 : 1) * NW * 64];

    const int lane = threadIdx.x & 63;
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col0 = blockIdx.x * (16 * NT);
    const int grp = blockIdx.y;
    const int K = g.K;

    // ---- which rows this workgroup owns (as the weight-streaming kernel)
    int expert = 0, seg_begin = 0, n_rows = 0;
    uint64_t members = 0;
    uint64_t scan_masks[moe_ws::kScanChunks];
    if (SRC == moe::ROWS_SCAN) {
        expert = grp;
#pragma unroll
        for (int c = 0; c < moe_ws::kScanChunks; ++c) {
            const int r = 64 * c + lane;
            const int id = (r < g.P) ? g.topk_ids[r] : -1;
            scan_masks[c] = __ballot(id == expert);
            n_rows += __popcll(scan_masks[c]);
        }
    } else if (SRC == moe::ROWS_SORTED) {
        expert = grp;
        seg_begin = g.offsets[grp];
        n_rows = g.offsets[grp + 1] - seg_begin;
    } else {  // ROWS_DIRECT
        const int e = g.topk_ids[grp];
        if (e < 0 || e >= g.num_experts)
            return;
        const int mine = (lane < g.P) ? g.topk_ids[lane] : -1;
        members = __ballot(mine == e);
        if (members & ((1ull << grp) - 1))
            return;  // an earlier route of this expert owns it
        expert = e;
        n_rows = __popcll(members);
    }
    if (n_rows <= 0)
        return;

    // ---- weights: lane owns row lane%16 of each tile, block lane/16 of each k-step
    const int r16 = lane & 15, p = lane >> 4;
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const size_t qrow = (size_t)K / 2, srow = (size_t)K / 32;  // bytes per weight row
    const uint8_t *Wq = g.wq + (size_t)expert * w_rows * qrow;
    const uint8_t *Ws = g.wscale + (size_t)expert * w_rows * srow;
    const uint8_t *wq[NW];
    const uint8_t *wsc[NW];
    bool tile_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < g.n_out;
        const int row = (tile_ok[nt] ? c : 0) + r16;
        wq[nt] = Wq + row * qrow + 16 * p;
        wsc[nt] = Ws + row * srow + p;
        if (GATE_UP) {
            wq[NT + nt] = Wq + (row + g.n_out) * qrow + 16 * p;
            wsc[NT + nt] = Ws + (row + g.n_out) * srow + p;
        }
    }

    // ---- K range of this wave (128-element k-steps), visited from a rotated start
    const int nks = K / 128;
    const int per = (nks + KSPLIT - 1) / KSPLIT;
    const int ks0 = kw * per;
    const int nk = max(0, min(nks, ks0 + per) - ks0);
    const int rot = nk > 0 ? (int)((blockIdx.x * 7u + blockIdx.y * 13u) % (unsigned)nk) : 0;

    for (int pass0 = 0; pass0 < n_rows; pass0 += 16) {
        // B operand column lane%16: row pass0 + lane%16 of the expert's rows
        const int s = pass0 + r16;
        int src_row = -1, dst_row = -1;
        if (s < n_rows) {
            if (SRC == moe::ROWS_SORTED) {
                const int row = seg_begin + s;
                const int route = g.sorted_ids[row];
                if (route >= 0) {
                    src_row = GATE_UP ? route / g.top_k : row;
                    dst_row = GATE_UP ? row : route;
                }
            } else {
                const int route = SRC == moe::ROWS_DIRECT ? moe_ws::nth_set_bit(members, s)
                                                          : moe_ws::nth_member(scan_masks, s);
                src_row = GATE_UP ? route / g.top_k : route;
                dst_row = route;
            }
        }
        // an unused column reads row 0: its results are never stored
        const uint16_t *arow = g.act + (size_t)(src_row < 0 ? 0 : src_row) * K + 32 * p;

        moe_f32x4 acc[NW];
#pragma unroll
        for (int nw = 0; nw < NW; ++nw)
            acc[nw] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

        moe_u32x4 wraw[STAGES][NW];
        uint32_t sraw[STAGES][NW];
        moe_u32x4 xv[STAGES][4];
        auto load = [&](int st, int i) {
            const int k = (ks0 + (i + rot) % nk) * 128;
#pragma unroll
            for (int nw = 0; nw < NW; ++nw) {
                if (tile_ok[nw % NT]) {
                    wraw[st][nw] = *(reinterpret_cast<const moe_u32x4 *>(wq[nw] + k / 2));
                    sraw[st][nw] = wsc[nw][k / 32];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xv[st][j] = moe_ws::load_cached(arow + k + 8 * j);
        };
        auto compute = [&](int st) {
#pragma unroll
            for (int nw = 0; nw < NW; ++nw) {
                if (!tile_ok[nw % NT])
                    continue;
                const float sc = e8m0_to_f32(sraw[st][nw]);
                const moe_u32x4 q = wraw[st][nw];
                const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[nw] = moe_mma16<0>(dequant8(words[j], sc), xv[st][j], acc[nw]);
            }
        };

        // software pipeline: STAGES-1 k-steps in flight
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            if (st < nk)
                load(st, st);
        for (int i = 0; i < nk; i += STAGES) {
#pragma unroll
            for (int st = 0; st < STAGES; ++st) {
                const int cur = i + st;
                if (cur < nk) {
                    const int nxt = cur + STAGES - 1;
                    if (nxt < nk)
                        load((st + STAGES - 1) % STAGES, nxt);
                    compute(st);
                }
            }
        }

        // ---- fixed-order sum over the K-split waves
        if (KSPLIT > 1) {
            __syncthreads();
            if (kw > 0) {
#pragma unroll
                for (int nw = 0; nw < NW; ++nw)
                    s_red[((kw - 1) * NW + nw) * 64 + lane] = acc[nw];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
                    for (int nw = 0; nw < NW; ++nw)
                        acc[nw] += s_red[(w * NW + nw) * 64 + lane];
            }
        }

        // ---- epilogue (wave 0): lane holds columns 4*(lane/16)+q of row lane%16
        if (kw == 0 && dst_row >= 0) {
            uint16_t *orow = g.out + (size_t)dst_row * g.n_out;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (!tile_ok[nt])
                    continue;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (GATE_UP) {
                        const float gate = acc[nt][q];
                        const float up = acc[NT + nt][q];
                        v[q] = gate / (1.0f + __expf(-gate)) * up;
                    } else {
                        v[q] = acc[nt][q];
                    }
                }
                moe_u32x2 packed;
                packed.x = moe_pack_bf16x2(v[0], v[1]);
                packed.y = moe_pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * p) = packed;
            }
        }
        if (KSPLIT > 1)
            __syncthreads();  // s_red is reused by the next pass
    }
}

// Row-tiled form, for tens to hundreds of routed rows per expert: the 16-row passes above stream
// an expert's weights once per pass; here a workgroup (4 waves) owns a 64-row tile of one
// expert's segment of the sorted layout (block_m 64) and 4 * NTW 16-column tiles, so each
// weight byte feeds 64 rows.
//   - each wave streams its own NTW (gate-up: NTW gate and NTW up) 16-row weight tiles exactly
//     as k_mx_gemm does: per 128-element k-step and tile one 16-byte load of codes and one scale
//     byte per lane, STAGES-1 k-steps ahead in registers, dequantised straight into the four
//     MFMA A operands (the same permuted k order: MFMA j takes elements 32p + 8j .. + 7 from
//     lane group p);
//   - the tile's 64 activation rows of a k-step (16 KB) are loaded once per workgroup (each wave
//     a quarter: 4 rows x 256 bytes per instruction) into a double-buffered LDS tile whose
//     16-byte chunk c of row r sits at position c ^ (r & 15), so that the B-operand reads (chunk
//     4p + j of 16 different rows) and the row-wise writes are free of bank conflicts; one
//     barrier per k-step;
//   - the 16-row MFMA tiles past the tile's last routed row are skipped;
//   - tile numbering and the rotated K start as the bf16 row-tiled kernel on sorted rows (the
//     column blocks of one row tile consecutive on one XCD, sharing its activation rows through
//     L2; only the real row tiles dealt out): Qwen3-235B batch 0.532 -> 0.519 ms, Qwen3-30B at
//     160 tokens 0.166 -> 0.158 ms.
// The code loads of both kernels are plain loads: a k-step reads 64 of a weight row's 128-byte
// line and the next k-step the other half, so the lines are worth keeping in L2 (non-temporal
// loads measured 15 % slower here at 11 and 32 rows per expert).
template <bool GATE_UP, int NTW, int STAGES>
__global__ __launch_bounds__(256) void k_mx_tiled(GemmProblem g, int n_blocks, int m_tiles)
{
    constexpr int kW = 4;                        // waves
    constexpr int BM = 64, TM = BM / 16;         // rows per tile, 16-row MFMA tiles
    constexpr int NW = GATE_UP ? 2 * NTW : NTW;  // 16-row weight tiles per wave per k-step
    constexpr int XI = BM / kW / 4;              // activation load instructions per wave
    __shared__ moe_u32x4 s_x[2][BM * 16];        // 64 rows x 16 chunks of 16 bytes

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const int real_tiles = g.offsets[g.num_experts] / BM;
    const int total = real_tiles * n_blocks;
    const int per_xcd = (total + moe_tiled::kXcds - 1) / moe_tiled::kXcds;
    const int idx = blockIdx.x / moe_tiled::kXcds;
    if (idx >= per_xcd)
        return;
    const int logical = (blockIdx.x % moe_tiled::kXcds) * per_xcd + idx;
    if (logical >= total)
        return;
    const int mtile = logical / n_blocks;
    const int nblk = logical % n_blocks;
    const int row0 = mtile * BM;
    const int expert = g.tile_expert[mtile];
    if (expert < 0)
        return;  // past the last tile of this routing
    const int K = g.K;
    const int col0 = nblk * (16 * NTW * kW) + wv * (16 * NTW);

    // routed rows of the tile (padding is a suffix of the expert's segment): one id per lane
    const int my_route = g.sorted_ids[row0 + lane];
    const int n_real = __popcll(__ballot(my_route >= 0));
    const int mt_active = (n_real + 15) / 16;

    // ---- weights: lane owns row lane%16 of each tile, block lane/16 of each k-step
    const int r16 = lane & 15, p = lane >> 4;
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const size_t qrow = (size_t)K / 2, srow = (size_t)K / 32;  // bytes per weight row
    const uint8_t *Wq = g.wq + (size_t)expert * w_rows * qrow;
    const uint8_t *Ws = g.wscale + (size_t)expert * w_rows * srow;
    const uint8_t *wq[NW];
    const uint8_t *wsc[NW];
    bool tile_ok[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < g.n_out;
        const int row = (tile_ok[nt] ? c : 0) + r16;  // past the last column: row 0, never stored
        wq[nt] = Wq + row * qrow + 16 * p;
        wsc[nt] = Ws + row * srow + p;
        if (GATE_UP) {
            wq[NTW + nt] = Wq + (row + g.n_out) * qrow + 16 * p;
            wsc[NTW + nt] = Ws + (row + g.n_out) * srow + p;
        }
    }

    // ---- activations: instruction i of this wave loads chunk lane%16 of tile row
    //      16*wv + 4*i + lane/16
    const uint16_t *xld[XI];
    int xslot[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = (BM / kW) * wv + 4 * i + (lane >> 4);
        const int route = g.sorted_ids[row0 + r];
        const int src = route < 0 ? 0 : (GATE_UP ? route / g.top_k : row0 + r);  // 0: unused
        xld[i] = g.act + (size_t)src * K + 8 * (lane & 15);
        xslot[i] = r * 16 + ((lane & 15) ^ (r & 15));
    }

    const int nk = K / 128;
    const int rot = (int)((nblk * 7u) % (unsigned)nk);

    moe_f32x4 acc[TM][NW];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
        for (int nw = 0; nw < NW; ++nw)
            acc[mt][nw] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

    moe_u32x4 wraw[STAGES][NW], xraw[STAGES][XI];
    uint32_t sraw[STAGES][NW];
    auto load = [&](int st, int i) {
        const int k = ((i + rot) % nk) * 128;
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
            wraw[st][nw] = *(reinterpret_cast<const moe_u32x4 *>(wq[nw] + k / 2));
            sraw[st][nw] = wsc[nw][k / 32];
        }
#pragma unroll
        for (int x = 0; x < XI; ++x)
            xraw[st][x] = moe_ws::load_cached(xld[x] + k);
    };
    auto compute = [&](int st, int i) {
        moe_u32x4 *xb = s_x[i & 1];
#pragma unroll
        for (int x = 0; x < XI; ++x)
            xb[xslot[x]] = xraw[st][x];
        __syncthreads();  // the activation tile of this k-step is complete
        moe_u32x4 a[NW][4];
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
            const float sc = e8m0_to_f32(sraw[st][nw]);
            const moe_u32x4 q = wraw[st][nw];
            a[nw][0] = dequant8(q.x, sc);
            a[nw][1] = dequant8(q.y, sc);
            a[nw][2] = dequant8(q.z, sc);
            a[nw][3] = dequant8(q.w, sc);
        }
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
            if (mt >= mt_active)
                break;
            const int r = mt * 16 + r16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const moe_u32x4 b = xb[r * 16 + ((4 * p + j) ^ r16)];
#pragma unroll
                for (int nw = 0; nw < NW; ++nw)
                    acc[mt][nw] = moe_mma16<0>(a[nw][j], b, acc[mt][nw]);
            }
        }
    };

    // Software pipeline, STAGES-1 k-steps in flight; the steady state is branch-free (past the
    // end the prefetch wraps to an early k-step, in bounds and never consumed).  The barrier in
    // compute() of step i also guarantees every wave has finished step i-1's reads of the
    // buffer that step i+1 overwrites.
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

    // ---- epilogue: lane holds columns 4*(lane/16)+q of row mt*16 + lane%16
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
        if (mt >= mt_active)
            break;
        const int r = mt * 16 + r16;
        const int route = g.sorted_ids[row0 + r];
        if (route < 0)
            continue;
        const int dst = GATE_UP ? row0 + r : route;
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
            packed.x = moe_pack_bf16x2(v[0], v[1]);
            packed.y = moe_pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * p) = packed;
        }
    }
}

}  // namespace moe_mx
