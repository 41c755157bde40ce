// moe_ws_kernel.h -- the weight-streaming grouped GEMM kernel of the MoE experts (gfx950).
//
// gate-up (TileOPs "MoE" page, MoEGroupedGemmFwd with activation=silu_and_mul on
// w_gate_up [E, 2F, H]):  h[row, f] = silu(x_row . Wg[e,f,:]) * (x_row . Wu[e,f,:])
//   with Wg = rows [0,F) and Wu = rows [F,2F) of the expert's w_gate_up.
// down (MoEGroupedGemmFwd on w_down [E, H, F]):  y[row, c] = h_row . Wd[e,c,:]
//
// At the routed-rows-per-expert counts of decode and batch MoE these GEMMs are bound by
// reading every touched expert's weights from HBM once, so the kernel is built around that
// stream:
//   - a workgroup owns one expert (or one route on the direct path, or a block of tokens for
//     the shared expert) and NT 16-column tiles of the output; it reads each weight row it
//     needs once per pass over its rows;
//   - weight loads are non-temporal and each load instruction covers whole 128-byte lines, with
//     STAGES-1 segments of SEGK k-steps (64 elements each) in flight per wave in registers.  A
//     load instruction reads 8/SEGK rows x 128*SEGK bytes: with SEGK = 1, 8 rows x one k-step;
//     with SEGK = 2, 4 rows x 256 bytes.  Rows a power-of-two multiple of 4 KB apart read at the
//     same offset map onto few HBM channels, so on such strides the longer row segments stream
//     faster (MI355X, 4 KB rows: 6.8 -> 7.1 TB/s for a pure read of the same bytes);
//   - every workgroup starts its K loop at a different k-step (rotated, wrapping around), so
//     the concurrent requests of the whole grid spread over all HBM channels instead of all
//     hitting the same offset of 4 KB rows at once;
//   - each k-step is transposed through a per-wave LDS buffer (XOR-swizzled 16-byte slots,
//     conflict-free on both sides) into the v_mfma_f32_16x16x32_bf16 operand layout; the
//     weights are the A operand, so a lane ends with four consecutive output columns of one row;
//   - the activation rows (L2-resident) are loaded straight into the B operand layout;
//   - KSPLIT waves split the K loop of the same tile and are summed through LDS in a fixed
//     order: more bytes in flight per tile, no second kernel, deterministic results.
// The gate and up tiles of the same columns sit in the same lanes, so SiLU(gate)*up is applied
// in registers and h is rounded to bf16 once; stores are 8 bytes (4 bf16) per lane.
//
// Row sources: ROWS_SORTED walks one expert's padded segment of the sorted route list (pad
// rows hold route -1 and are neither read nor written).  Without a sort: ROWS_DIRECT (T*k <= 64)
// runs one workgroup per route, the first route of an expert gathers all routes of that expert
// and later ones exit; ROWS_SCAN (T*k <= 512) runs one workgroup per expert, which finds its
// routes by scanning topk_ids with wave ballots.  Either way an expert's weights are streamed
// once however many tokens chose it, and rows are taken in route order.  (The dense shared
// expert runs on the 256 x 256 tile kernel; no dense form of this kernel is instantiated.)
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe_ws {

using moe::GemmProblem;

// index of the n-th (0-based) set bit of m, or -1
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n)
{
    for (int i = 0; i < n && m; ++i)
        m &= m - 1;
    return m ? (int)__builtin_ctzll(m) : -1;
}

constexpr int kScanChunks = moe::kScanMaxRoutes / 64;

// index of the n-th member of the route set given as kScanChunks 64-bit masks, or -1
__device__ __forceinline__ int nth_member(const uint64_t (&masks)[kScanChunks], int n)
{
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
        const int pc = __popcll(masks[c]);
        if (n < pc)
            return 64 * c + nth_set_bit(masks[c], n);
        n -= pc;
    }
    return -1;
}

__device__ __forceinline__ moe_u32x4 load_nt(const uint16_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const moe_u32x4 *>(p));
}

__device__ __forceinline__ moe_u32x4 load_cached(const uint16_t *p)
{
    return *reinterpret_cast<const moe_u32x4 *>(p);
}

// LDS bytes of one workgroup: per-wave transpose buffers, reused for the K-split sum.
template <int NW, int MT, int KSPLIT, int SEGK>
struct WsSmem {
    static constexpr int kTranspose = KSPLIT * NW * 16 * 8 * SEGK;     // 16-byte slots
    static constexpr int kReduce = (KSPLIT > 1 ? KSPLIT - 1 : 0) * MT * NW * 64;  // f32x4
    static constexpr int kSlots = kTranspose > kReduce ? kTranspose : kReduce;
};

// One workgroup's tile: column block bx, row group by.
// SEGK: k-steps per weight load segment (1 or 2); the K range of every wave must hold a whole
// number of segments (the launcher checks K).
template <bool GATE_UP, int SRC, int NT, int MT, int KSPLIT, int STAGES, int DT, int SEGK>
__device__ __forceinline__ void ws_body(const GemmProblem &g, int bx, int by, moe_u32x4 *s_mem)
{
    constexpr int NW = GATE_UP ? 2 * NT : NT;  // 16-row weight tiles per k-step
    constexpr int ROWS = 16 * MT;              // rows per pass
    constexpr int RPI = 8 / SEGK;              // weight rows per load instruction
    constexpr int LPR = 8 * SEGK;              // lanes per row of an instruction = row slots
    constexpr int NLD = 2 * SEGK;              // load instructions per 16-row tile and segment
    constexpr int TS = 16 * LPR;               // transpose slots per 16-row tile
    static_assert(SEGK == 1 || SEGK == 2, "segments of one or two k-steps");

    const int lane = threadIdx.x & 63;
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int col0 = bx * (16 * NT);
    const int grp = by;
    const int K = g.K;

    // ---- which rows this workgroup owns
    int expert = 0, seg_begin = 0, n_rows = 0;
    uint64_t members = 0;
    uint64_t scan_masks[kScanChunks];
    if (SRC == moe::ROWS_SCAN) {
        expert = grp;
#pragma unroll
        for (int c = 0; c < kScanChunks; ++c) {
            const int r = 64 * c + lane;
            const int id = (r < g.P) ? g.topk_ids[r] : -1;
            scan_masks[c] = __ballot(id == expert);
            n_rows += __popcll(scan_masks[c]);
        }
    } else if (SRC == moe::ROWS_SORTED) {
        expert = grp;
        seg_begin = g.offsets[grp];
        n_rows = g.offsets[grp + 1] - seg_begin;
    } else if (SRC == moe::ROWS_DIRECT) {
        const int e = g.topk_ids[grp];
        if (e < 0 || e >= g.num_experts)
            return;
        const int mine = (lane < g.P) ? g.topk_ids[lane] : -1;
        members = __ballot(mine == e);
        if (members & ((1ull << grp) - 1))
            return;  // an earlier route of this expert owns it
        expert = e;
        n_rows = __popcll(members);
    } else {
        seg_begin = grp * ROWS;
        n_rows = min(ROWS, g.rows - seg_begin);
    }
    if (n_rows <= 0)
        return;

    // ---- weight loads: instruction j of a segment reads 16 bytes (chunk lane % LPR) of row
    //      RPI*j + lane / LPR of each 16-row tile
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const uint16_t *W = g.weight + (size_t)expert * w_rows * K;
    const int lrow = lane / LPR, lchunk = lane % LPR;
    const uint16_t *wld[NW];
    bool tile_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < g.n_out;
        const int row = (tile_ok[nt] ? c : 0) + lrow;
        wld[nt] = W + (size_t)row * K + 8 * lchunk;
        if (GATE_UP)
            wld[NT + nt] = W + (size_t)(row + g.n_out) * K + 8 * lchunk;
    }
    // LDS transpose buffer of this wave: NW tiles x 16 rows x LPR slots; row r keeps chunk c
    // (elements 8c .. 8c+7 of the segment) in slot c ^ swz(r): the 16 rows read at one chunk
    // position, and the LPR chunks of a row written by one instruction, hit distinct banks
    auto swz = [](int r) { return SEGK == 1 ? (r >> 1) : (r & 15); };
    moe_u32x4 *tbuf = s_mem + kw * NW * TS;
    int wslot[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
        const int r = RPI * j + lrow;
        wslot[j] = r * LPR + (lchunk ^ swz(r));
    }
    const int rrow = lane & 15, rq = lane >> 4;
    int rslot0[SEGK], rslot1[SEGK];
#pragma unroll
    for (int h = 0; h < SEGK; ++h) {
        rslot0[h] = rrow * LPR + ((8 * h + rq) ^ swz(rrow));      // k-step h, k 0..31
        rslot1[h] = rrow * LPR + ((8 * h + rq + 4) ^ swz(rrow));  // k-step h, k 32..63
    }
    const int xoff = 8 * rq;  // B operand: k = 8*(lane/16) (+32)

    // ---- K range of this wave (nk k-steps, nseg segments), visited from a rotated start
    const int nks = K / 64;
    const int per = (nks + KSPLIT - 1) / KSPLIT;
    const int ks0 = kw * per;
    const int nk = max(0, min(nks, ks0 + per) - ks0);
    const int nseg = nk / SEGK;
    const int rot =
        nseg > 0 ? (int)((bx * 7u + by * 13u) % (unsigned)nseg) : 0;

    // Every load below is issued on every path, the same number per segment: segments past
    // the wave's K range (and the prefetch past its end) read one 16-byte line at the start of
    // the activations, all lanes alike (a cache hit), instead of being skipped.  With loads
    // under branches the compiler cannot count the outstanding ones and waits for all of them
    // before each segment's compute, which drains the prefetch.  Weight tiles past the last
    // column and row slots past the rows read clamped, in-bounds rows (wld, arow).
    const uint16_t *const dummy = g.act;
    const int nseg1 = max(nseg, 1);
    moe_u32x4 wraw[STAGES][NW][NLD];
    auto load_w = [&](int st, int i) {
        const bool on = i < nseg;
        const int k = (ks0 + ((i + rot) % nseg1) * SEGK) * 64;
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
#pragma unroll
            for (int j = 0; j < NLD; ++j)
                wraw[st][nw][j] = load_nt(on ? wld[nw] + (size_t)(RPI * j) * K + k : dummy);
        }
    };

    for (int pass0 = 0; pass0 < n_rows; pass0 += ROWS) {
        // The pass's weight prefetch is issued before its row plan: the plan's dependent loads
        // (sorted ids or scan -> route -> token row) then overlap the weight latency.
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            load_w(st, st);
        // ---- row plan: activation row and output row of slot lane%16 of each m-tile
        const uint16_t *arow[MT];
        int dst[MT];
        const int mt_active = min(MT, (n_rows - pass0 + 15) / 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int s = pass0 + 16 * mt + (lane & 15);
            int src_row = -1, dst_row = -1;
            if (s < n_rows) {
                if (SRC == moe::ROWS_SORTED) {
                    const int row = seg_begin + s;
                    const int route = g.sorted_ids[row];
                    if (route >= 0) {
                        src_row = GATE_UP ? route / g.top_k : row;
                        dst_row = GATE_UP ? row : route;
                    }
                } else if (SRC == moe::ROWS_DIRECT || SRC == moe::ROWS_SCAN) {
                    const int route = SRC == moe::ROWS_DIRECT ? nth_set_bit(members, s)
                                                              : nth_member(scan_masks, s);
                    src_row = GATE_UP ? route / g.top_k : route;
                    dst_row = route;
                } else {
                    src_row = dst_row = seg_begin + s;
                }
            }
            // an unused slot reads row 0: its column of the result is never stored
            arow[mt] = g.act + (size_t)(src_row < 0 ? 0 : src_row) * K + xoff;
            dst[mt] = dst_row;
        }

        moe_f32x4 acc[MT][NW];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nw = 0; nw < NW; ++nw)
                acc[mt][nw] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

        moe_u32x4 xv[STAGES][SEGK][MT][2];
        auto load_x = [&](int st, int i) {
            const bool on = i < nseg;
            const int k0 = (ks0 + ((i + rot) % nseg1) * SEGK) * 64;
#pragma unroll
            for (int h = 0; h < SEGK; ++h) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xv[st][h][mt][0] = load_cached(on ? arow[mt] + k0 + 64 * h : dummy);
                    xv[st][h][mt][1] = load_cached(on ? arow[mt] + k0 + 64 * h + 32 : dummy);
                }
            }
        };
        auto compute = [&](int st) {
#pragma unroll
            for (int nw = 0; nw < NW; ++nw) {
                if (tile_ok[nw % NT]) {
#pragma unroll
                    for (int j = 0; j < NLD; ++j)
                        tbuf[nw * TS + wslot[j]] = wraw[st][nw][j];
                }
            }
            moe_wave_sync();
#pragma unroll
            for (int h = 0; h < SEGK; ++h) {
#pragma unroll
                for (int nw = 0; nw < NW; ++nw) {
                    if (!tile_ok[nw % NT])
                        continue;
                    const moe_u32x4 a0 = tbuf[nw * TS + rslot0[h]];
                    const moe_u32x4 a1 = tbuf[nw * TS + rslot1[h]];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        if (mt < mt_active) {
                            acc[mt][nw] = moe_mma16<DT>(a0, xv[st][h][mt][0], acc[mt][nw]);
                            acc[mt][nw] = moe_mma16<DT>(a1, xv[st][h][mt][1], acc[mt][nw]);
                        }
                    }
                }
            }
            moe_wave_sync();
        };

        // software pipeline: STAGES-1 segments in flight (their weights already requested);
        // the loads are issued ahead of the segment's compute on every path (see above)
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            load_x(st, st);
        for (int i = 0; i < nseg; i += STAGES) {
#pragma unroll
            for (int st = 0; st < STAGES; ++st) {
                const int cur = i + st;
                load_w((st + STAGES - 1) % STAGES, cur + STAGES - 1);
                load_x((st + STAGES - 1) % STAGES, cur + STAGES - 1);
                __builtin_amdgcn_sched_barrier(0);
                if (cur < nseg)
                    compute(st);
            }
        }

        // ---- fixed-order sum over the K-split waves (LDS reused once every wave is done)
        if (KSPLIT > 1) {
            moe_f32x4 *red = reinterpret_cast<moe_f32x4 *>(s_mem);
            __syncthreads();
            if (kw > 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nw = 0; nw < NW; ++nw)
                        red[(((kw - 1) * MT + mt) * NW + nw) * 64 + lane] = acc[mt][nw];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nw = 0; nw < NW; ++nw)
                            acc[mt][nw] += red[((w * MT + mt) * NW + nw) * 64 + lane];
            }
            __syncthreads();
        }

        // ---- epilogue (wave 0): lane holds columns 4*(lane/16)+r of row lane%16
        if (kw == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt >= mt_active || dst[mt] < 0)
                    continue;
                uint16_t *orow = g.out + (size_t)dst[mt] * g.n_out;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if (!tile_ok[nt])
                        continue;
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (GATE_UP) {
                            const float gate = acc[mt][nt][r];
                            const float up = acc[mt][NT + nt][r];
                            v[r] = gate / (1.0f + __expf(-gate)) * up;
                        } else {
                            v[r] = acc[mt][nt][r];
                        }
                    }
                    moe_u32x2 packed;
                    packed.x = moe_pack2<DT>(v[0], v[1]);
                    packed.y = moe_pack2<DT>(v[2], v[3]);
                    *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * rq) = packed;
                }
            }
        }
    }
}

template <bool GATE_UP, int SRC, int NT, int MT, int KSPLIT, int STAGES, int DT, int SEGK = 1>
__global__ __launch_bounds__(64 * KSPLIT)
__attribute__((amdgpu_waves_per_eu(SEGK == 2 ? 3 : 1))) void k_ws_gemm(GemmProblem g)
{
    constexpr int NW = GATE_UP ? 2 * NT : NT;
    __shared__ moe_u32x4 s_mem[WsSmem<NW, MT, KSPLIT, SEGK>::kSlots];
    ws_body<GATE_UP, SRC, NT, MT, KSPLIT, STAGES, DT, SEGK>(g, blockIdx.x, blockIdx.y, s_mem);
}

}  // namespace moe_ws
