// moe_gemm_ws.hip -- weight-streaming grouped GEMMs of the MoE experts (gfx950, bf16 MFMA).
//
// gate-up (TileOPs "MoE" page, MoEGroupedGemmFwd with activation=silu_and_mul on
// w_gate_up [E, 2F, H]):  h[row, f] = silu(x_row . Wg[e,f,:]) * (x_row . Wu[e,f,:])
//   with Wg = rows [0,F) and Wu = rows [F,2F) of the expert's w_gate_up.
// down (MoEGroupedGemmFwd on w_down [E, H, F]):  y[row, c] = h_row . Wd[e,c,:]
//
// At the routed-rows-per-expert counts of decode and batch MoE (1 to ~150 rows per expert)
// these GEMMs are bound by reading each expert's weights from HBM once, so the kernel is built
// around streaming weights:
//   - a workgroup owns one expert (or one route, on the direct path) and NT 16-column tiles of
//     the output; every weight row it needs is read exactly once per pass over the rows;
//   - each lane reads 32 contiguous bytes of one weight row per 64-element k-step, straight
//     from global memory into registers in the MFMA operand layout (no LDS staging: nothing is
//     reused across waves), double-buffered so one k-step is always in flight;
//   - the activation rows (a few KB, L2-resident) ride along in the same layout;
//   - KSPLIT waves split the K loop of the same tile and are summed through LDS in a fixed
//     order, which multiplies the in-flight weight bytes without a second kernel and keeps the
//     result deterministic;
//   - the output tile is D[n][m] = W[n,:] . X[m,:] (weights as the MFMA A operand), so a lane
//     ends with four consecutive output columns of one row and stores them as 8 bytes.
// The gate and up tiles of the same columns sit in the same lanes, so SiLU(gate)*up is applied
// in registers; h is rounded to bf16 once.
//
// Row sources: ROWS_SORTED walks one expert's padded segment of the sorted route list (pad
// rows hold route -1 and are neither read nor written); ROWS_DIRECT scans topk_ids (T*k <= 64):
// the first route of an expert gathers all routes of that expert, later ones exit (the weights
// are then streamed once per expert, not once per route); ROWS_DENSE takes every token
// (shared expert).
#include "moe_device.h"
#include "moe_internal.h"

namespace {

using moe::GemmProblem;

// index of the n-th (0-based) set bit of m, or -1
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n)
{
    for (int i = 0; i < n && m; ++i)
        m &= m - 1;
    return m ? (int)__builtin_ctzll(m) : -1;
}

template <bool GATE_UP, int SRC, int NT, int MT, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void k_ws_gemm(GemmProblem g)
{
    constexpr int NW = GATE_UP ? 2 * NT : NT;  // 16-row weight tiles per k-step
    constexpr int ROWS = 16 * MT;              // rows per pass
    __shared__ moe_f32x4 s_red[KSPLIT > 1 ? KSPLIT - 1 : 1][MT][NW][64];

    const int lane = threadIdx.x & 63;
    const int kw = threadIdx.x >> 6;
    const int col0 = blockIdx.x * (16 * NT);
    const int grp = blockIdx.y;
    const int K = g.K;

    // ---- which rows this workgroup owns
    int expert = 0, seg_begin = 0, n_rows = 0;
    uint64_t members = 0;
    if (SRC == moe::ROWS_SORTED) {
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

    // ---- weight rows of this lane (row lane%16 of each 16-row tile)
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const uint16_t *W = g.weight + (size_t)expert * w_rows * K;
    const uint16_t *wrow[NW];
    bool tile_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < g.n_out;
        const int row = tile_ok[nt] ? c + (lane & 15) : 0;
        wrow[nt] = W + (size_t)row * K;
        if (GATE_UP)
            wrow[NT + nt] = W + (size_t)(row + g.n_out) * K;
    }

    const int nks = K / 64;
    const int per = (nks + KSPLIT - 1) / KSPLIT;
    const int ks0 = kw * per;
    const int ks1 = min(nks, ks0 + per);
    const int koff = 16 * (lane >> 4);

    for (int pass0 = 0; pass0 < n_rows; pass0 += ROWS) {
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
                } else if (SRC == moe::ROWS_DIRECT) {
                    const int route = nth_set_bit(members, s);
                    src_row = GATE_UP ? route / g.top_k : route;
                    dst_row = route;
                } else {
                    src_row = dst_row = seg_begin + s;
                }
            }
            // an unused slot reads row 0: its column of the result is never stored
            arow[mt] = g.act + (size_t)(src_row < 0 ? 0 : src_row) * K;
            dst[mt] = dst_row;
        }

        moe_f32x4 acc[MT][NW];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nw = 0; nw < NW; ++nw)
                acc[mt][nw] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

        moe_u32x4 wf0[NW][2], af0[MT][2], wf1[NW][2], af1[MT][2];
        auto load = [&](moe_u32x4(&wf)[NW][2], moe_u32x4(&af)[MT][2], int ks) {
            const int k = ks * 64 + koff;
#pragma unroll
            for (int nw = 0; nw < NW; ++nw) {
                if (tile_ok[nw % NT]) {
                    const moe_u32x4 *p = reinterpret_cast<const moe_u32x4 *>(wrow[nw] + k);
                    wf[nw][0] = p[0];
                    wf[nw][1] = p[1];
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < mt_active) {
                    const moe_u32x4 *p = reinterpret_cast<const moe_u32x4 *>(arow[mt] + k);
                    af[mt][0] = p[0];
                    af[mt][1] = p[1];
                }
            }
        };
        auto compute = [&](moe_u32x4(&wf)[NW][2], moe_u32x4(&af)[MT][2]) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < mt_active) {
#pragma unroll
                    for (int nw = 0; nw < NW; ++nw) {
                        if (tile_ok[nw % NT]) {
                            acc[mt][nw] = moe_mfma_16x16x32(wf[nw][0], af[mt][0], acc[mt][nw]);
                            acc[mt][nw] = moe_mfma_16x16x32(wf[nw][1], af[mt][1], acc[mt][nw]);
                        }
                    }
                }
            }
        };

        int ks = ks0;
        if (ks < ks1)
            load(wf0, af0, ks);
        while (ks < ks1) {
            if (ks + 1 < ks1)
                load(wf1, af1, ks + 1);
            compute(wf0, af0);
            if (ks + 2 < ks1)
                load(wf0, af0, ks + 2);
            if (ks + 1 < ks1)
                compute(wf1, af1);
            ks += 2;
        }

        // ---- fixed-order sum over the K-split waves
        if (KSPLIT > 1) {
            if (kw > 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nw = 0; nw < NW; ++nw)
                        s_red[kw - 1][mt][nw][lane] = acc[mt][nw];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nw = 0; nw < NW; ++nw)
                            acc[mt][nw] += s_red[w][mt][nw][lane];
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
                    packed.x = moe_pack_bf16x2(v[0], v[1]);
                    packed.y = moe_pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * (lane >> 4)) =
                        packed;
                }
            }
        }
    }
}

template <bool GATE_UP, int SRC, int NT, int MT, int KSPLIT>
void launch_one(const GemmProblem &g, hipStream_t stream)
{
    const dim3 grid((g.n_out + 16 * NT - 1) / (16 * NT), g.num_groups);
    hipLaunchKernelGGL((k_ws_gemm<GATE_UP, SRC, NT, MT, KSPLIT>), grid, dim3(64 * KSPLIT), 0,
                       stream, g);
}

// Instantiated tile shapes.  Every shape the host dispatch may pick must be listed here.
template <bool GATE_UP, int SRC>
bool dispatch(const GemmProblem &g, moe::WsTile t, hipStream_t s)
{
#define MOE_WS_CASE(NT_, MT_, KS_)                                                               \
    if (t.nt == NT_ && t.mt == MT_ && t.ksplit == KS_) {                                         \
        launch_one<GATE_UP, SRC, NT_, MT_, KS_>(g, s);                                           \
        return true;                                                                             \
    }
    MOE_WS_CASE(1, 1, 4)
    MOE_WS_CASE(2, 1, 2)
    MOE_WS_CASE(2, 1, 4)
    MOE_WS_CASE(2, 2, 2)
    MOE_WS_CASE(2, 4, 1)
    MOE_WS_CASE(2, 4, 2)
    MOE_WS_CASE(4, 1, 2)
    MOE_WS_CASE(4, 1, 4)
    MOE_WS_CASE(4, 2, 2)
    MOE_WS_CASE(4, 4, 1)
    MOE_WS_CASE(4, 4, 2)
#undef MOE_WS_CASE
    return false;
}

}  // namespace

namespace moe {

static bool launch_any(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
                       hipStream_t stream)
{
    if (gate_up) {
        if (src == ROWS_SORTED)
            return dispatch<true, ROWS_SORTED>(g, tile, stream);
        if (src == ROWS_DIRECT)
            return dispatch<true, ROWS_DIRECT>(g, tile, stream);
        return dispatch<true, ROWS_DENSE>(g, tile, stream);
    }
    if (src == ROWS_SORTED)
        return dispatch<false, ROWS_SORTED>(g, tile, stream);
    if (src == ROWS_DIRECT)
        return dispatch<false, ROWS_DIRECT>(g, tile, stream);
    return dispatch<false, ROWS_DENSE>(g, tile, stream);
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
