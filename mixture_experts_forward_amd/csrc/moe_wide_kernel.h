// moe_wide_kernel.h -- 256 x 256 tile GEMM of the MoE experts for prefill (hundreds of routed
// rows per expert) and the dense shared expert.
//
// Same math as moe_ws_kernel.h (gate-up with the SiLU(gate)*up epilogue, or down).  Built so
// that each weight byte and each activation byte fetched from beyond L2 feeds as many MFMAs as
// one CU can hold:
//   - a workgroup of 8 waves owns a 256-row tile and 256 weight rows (gate-up: 128 gate rows and
//     the 128 up rows of the same columns); waves form a 4 x 2 grid, wave (wm, wn) computing the
//     32-row tiles wm and wm+4 of the row tile against weight rows [128*wn, 128*wn + 128) --
//     2 x 4 accumulators of v_mfma_f32_32x32x16_bf16, which does twice the work of the
//     16x16x32 form per issue slot on gfx950 (measured 2.25 vs 1.29 PFLOP/s);
//   - each operand's 64-element k-step (256 rows x 128 B, 32 KB) goes from global memory
//     straight into LDS with global_load_lds_dwordx4 -- each wave instruction covers 8 whole
//     128-byte rows and no register holds them -- into the slot order
//     slot(r, c) = 8r + (c ^ ((r >> 1) & 7)) that the MFMA operand reads take without bank
//     conflicts: lane l of an instruction writes slot 8*(l/8) + l%8 of its 8 rows, so it
//     fetches chunk (l%8) ^ swizzle(row) of its row;
//   - the operands run separate pipelines: the weight rows (from HBM) WS - 1 k-steps ahead in
//     WS stages, the activation rows (mostly L2 hits: every column block of an expert reads
//     them) one k-step ahead in two; WS = 3 fills the 160 KB of LDS and keeps two k-steps of
//     weights in flight per CU.  One barrier per k-step;
//   - padding rows of an expert's segment form a suffix, so the 32-row tiles that hold only
//     padding are known from their first row: their loads and MFMAs are skipped, and the
//     interleaved row-tile assignment spreads the real rows over the four SIMDs.  MFMA work
//     thus follows the routed rows, not the 256-row padding;
//   - the bf16 output tile is staged in LDS (XOR-swizzled 16-byte chunks) and stored as whole
//     rows;
//   - tiles are numbered expert by expert (sorted rows) or row tiles of a column block
//     consecutively (dense rows) and blocks are dealt round-robin to the 8 XCDs, each XCD
//     taking a contiguous range of tile numbers; tiles sharing a weight or activation tile
//     start their K loop at the same k-step (they stay in step and share the lines in L2),
//     others at different ones (HBM channels).
// The shared pieces (Stage, dma16, wait_loads, the tile numbering) also serve moe_fp8_kernel.h.
#pragma once

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_mx_dequant.h"

namespace moe_wide {

using moe::GemmProblem;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr int kBM = 256;                       // rows per tile
constexpr int kBW = 256;                       // weight rows per tile
constexpr int kWM = 4, kWN = 2;                // wave grid
constexpr int kMT = kBM / 16 / kWM;            // 16-row tiles per wave (4)
constexpr int kNT = kBW / 16 / kWN;            // 16-row weight tiles per wave (8)

// LDS shape of one pipeline stage holding a KSTEP-element k-step of both operands: rows of
// KSTEP/8 16-byte slots, activation rows first.
template <int KSTEP>
struct Stage {
    static constexpr int kSlots = KSTEP / 8;                    // 16-byte slots per row
    static constexpr int kRowsPerLoad = 64 / kSlots;            // rows per wave DMA instruction
    static constexpr int kXLoads = kBM / kWaves / kRowsPerLoad; // per wave
    static constexpr int kWLoads = kBW / kWaves / kRowsPerLoad;
    static constexpr int kBytes = (kBM + kBW) * KSTEP * 2;
    // slot of chunk c of row r: XOR-swizzled so that the MFMA operand reads (16 rows x one
    // chunk per 16 lanes) hit distinct banks
    static __device__ __forceinline__ int slot(int r, int c)
    {
        return r * kSlots + (c ^ ((r >> 1) & (kSlots - 1)));
    }
};

// Grid of a launch: resident slots (a multiple of 8), or fewer when there are fewer tiles
// (total_cap: an upper bound of the tile count).
inline int wide_grid(int total_cap, int slots)
{
    const int cap = (total_cap + kXcds - 1) / kXcds * kXcds;
    const int s = slots / kXcds * kXcds;
    return cap < kXcds ? kXcds : (s < kXcds ? kXcds : (cap < s ? cap : s));
}

// 16 bytes from global address g into LDS byte address lds_base + 16 * lane (the whole wave
// writes 1 KB).  Issued as inline assembly so that the compiler's wait-count pass does not
// drain it before every LDS read; the kernel waits for it explicitly (vmcnt) before the
// barrier that publishes the stage.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_base)
                 : "memory", "m0");
}

// The same for 4 bytes a lane (lane l writes LDS bytes lds_base + 4l .. + 3).
__device__ __forceinline__ void dma4(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(g), "s"(lds_base)
                 : "memory", "m0");
}

// Wait until at most n of this wave's vector-memory loads are outstanding (0 <= n <= 63).
__device__ __forceinline__ void wait_loads(int n)
{
#define MOE_WAIT_CASE(N)                                                                         \
    case N:                                                                                      \
        asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory");                                  \
        break;
    switch (n) {
        MOE_WAIT_CASE(1) MOE_WAIT_CASE(2) MOE_WAIT_CASE(3) MOE_WAIT_CASE(4) MOE_WAIT_CASE(5)
        MOE_WAIT_CASE(6) MOE_WAIT_CASE(7) MOE_WAIT_CASE(8) MOE_WAIT_CASE(9) MOE_WAIT_CASE(10)
        MOE_WAIT_CASE(11) MOE_WAIT_CASE(12) MOE_WAIT_CASE(13) MOE_WAIT_CASE(14) MOE_WAIT_CASE(15)
        MOE_WAIT_CASE(16) MOE_WAIT_CASE(17) MOE_WAIT_CASE(18) MOE_WAIT_CASE(19) MOE_WAIT_CASE(20)
        MOE_WAIT_CASE(21) MOE_WAIT_CASE(22) MOE_WAIT_CASE(23) MOE_WAIT_CASE(24) MOE_WAIT_CASE(25)
        MOE_WAIT_CASE(26) MOE_WAIT_CASE(27) MOE_WAIT_CASE(28) MOE_WAIT_CASE(29) MOE_WAIT_CASE(30)
        MOE_WAIT_CASE(31) MOE_WAIT_CASE(32) MOE_WAIT_CASE(33) MOE_WAIT_CASE(34) MOE_WAIT_CASE(35)
        MOE_WAIT_CASE(36) MOE_WAIT_CASE(37) MOE_WAIT_CASE(38) MOE_WAIT_CASE(39) MOE_WAIT_CASE(40)
        MOE_WAIT_CASE(41) MOE_WAIT_CASE(42) MOE_WAIT_CASE(43) MOE_WAIT_CASE(44) MOE_WAIT_CASE(45)
        MOE_WAIT_CASE(46) MOE_WAIT_CASE(47) MOE_WAIT_CASE(48) MOE_WAIT_CASE(49) MOE_WAIT_CASE(50)
        MOE_WAIT_CASE(51) MOE_WAIT_CASE(52) MOE_WAIT_CASE(53) MOE_WAIT_CASE(54) MOE_WAIT_CASE(55)
        MOE_WAIT_CASE(56) MOE_WAIT_CASE(57) MOE_WAIT_CASE(58) MOE_WAIT_CASE(59) MOE_WAIT_CASE(60)
        MOE_WAIT_CASE(61) MOE_WAIT_CASE(62) MOE_WAIT_CASE(63)
    default:
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        break;
    }
#undef MOE_WAIT_CASE
}

// Workgroup barrier of a k-loop whose stages are filled by dma16: waits until at most n
// (0 <= n <= 63) of this wave's vector-memory loads are outstanding and its LDS reads are
// done, then s_barrier.  After it every wave's DMA of the awaited k-steps has landed in LDS and
// every wave has finished reading the previous stage.  The DMAs' LDS writes are counted by
// vmcnt, which __syncthreads() (lgkmcnt(0) and s_barrier here) does not wait on, and the
// compiler cannot see them; so the wait is explicit, counted to leave the later k-steps' loads
// in flight.  The "memory" clobber keeps LDS accesses on their side.
__device__ __forceinline__ void step_barrier(int n)
{
#define MOE_BAR_CASE(N)                                                                          \
    case N:                                                                                      \
        asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory");          \
        break;
    switch (n) {
        MOE_BAR_CASE(1) MOE_BAR_CASE(2) MOE_BAR_CASE(3) MOE_BAR_CASE(4) MOE_BAR_CASE(5)
        MOE_BAR_CASE(6) MOE_BAR_CASE(7) MOE_BAR_CASE(8) MOE_BAR_CASE(9) MOE_BAR_CASE(10)
        MOE_BAR_CASE(11) MOE_BAR_CASE(12) MOE_BAR_CASE(13) MOE_BAR_CASE(14) MOE_BAR_CASE(15)
        MOE_BAR_CASE(16)
    default:
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        break;
    }
#undef MOE_BAR_CASE
}

template <int SRC>
__device__ __forceinline__ int wide_total(const GemmProblem &g, int n_blocks, int m_tiles)
{
    if (SRC == moe::ROWS_SORTED)
        return g.offsets[g.num_experts] / kBM * n_blocks;
    return m_tiles * n_blocks;
}

// Tile number t -> (column block, row tile, expert).  Sorted rows: tiles are numbered expert by
// expert; within an expert, column block by column block with the expert's row tiles
// innermost.  Dense rows: column block by column block, row tiles innermost.
template <int SRC>
__device__ __forceinline__ void wide_decode(const GemmProblem &g, int t, int n_blocks,
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

// Number of leading real rows of the tile: sorted rows -> padding is a suffix of the expert's
// segment (found by a binary search of the first -1); dense rows -> min(256, rows - row0).
// Every lane of the wave calls it: lane l reads the ids of rows 4l .. 4l+3 (one 16-byte load;
// row0 is a multiple of 256 and the padded layout holds whole 256-row tiles), and four ballots
// count the rows that hold a route -- one load latency instead of a dependent search.
template <int SRC>
__device__ __forceinline__ int wide_real_rows(const GemmProblem &g, int row0)
{
    if (SRC != moe::ROWS_SORTED)
        return min(kBM, g.rows - row0);
    const int lane = threadIdx.x & 63;
    const moe_u32x4 v = *reinterpret_cast<const moe_u32x4 *>(g.sorted_ids + row0 + 4 * lane);
    return __popcll(__ballot((int)v.x >= 0)) + __popcll(__ballot((int)v.y >= 0)) +
           __popcll(__ballot((int)v.z >= 0)) + __popcll(__ballot((int)v.w >= 0));
}

// The bf16 tile: 32 x 32 x 16 MFMAs (twice the work per issue of 16 x 16 x 32 on gfx950), a wave
// computing 2 row tiles x 4 weight tiles of 32.
constexpr int kMT32 = kBM / 32 / kWM;     // 32-row tiles per wave (2)
constexpr int kNT32 = kBW / 32 / kWN;     // 32-row weight tiles per wave (4)
constexpr int kStep = 64;                 // elements per k-step (128-byte rows)
constexpr int kHalf = kBM * kStep * 2;    // LDS bytes of one operand's k-step (32 KB)
// The weight rows come from HBM and the activation rows mostly from L2, so the two operands
// run separate pipelines: activations one k-step ahead (two stages), weights WS - 1 k-steps
// ahead (WS stages; WS = 3 takes all 160 KB of LDS).
constexpr int kXStages = 2;
template <int WS>
constexpr int wide_lds_bytes() { return (kXStages + WS) * kHalf; }
static_assert(kBM == kBW, "both operands' k-steps take kHalf bytes");
// Tiles of at most kSmallRows real rows run a deeper pipeline: kSmallStages stages of a
// 64-row activation k-step (kSmallX bytes) and a 256-row weight k-step.
#ifndef MOE_WIDE_SMALL_ROWS
#define MOE_WIDE_SMALL_ROWS 64
#endif
constexpr int kSmallRows = MOE_WIDE_SMALL_ROWS;
constexpr int kSmallStages = 4;
constexpr int kSmallX = 64 * kStep * 2;
static_assert(kSmallRows <= 64, "the small pipeline's activation stage holds 64 rows");
static_assert(kSmallStages * (kSmallX + kHalf) <= wide_lds_bytes<3>(),
              "the small pipeline fits the LDS of the three-stage kernel");

// One 256 x 256 tile over k-steps [kbeg, kbeg + kcnt) of the K loop (visited from a rotated
// start).  part == NULL: the whole K range, written as bf16 (gate-up: SiLU(gate)*up).  Else the
// f32 accumulators of this K range go to part as [256 activation rows][256 weight rows] (rows
// past the tile's real rows are not written), for k_wide_reduce to sum.
struct NoHook {
    __device__ void operator()() const {}
};

// MX: the weights are MXFP4 (g.wq, g.wscale) and are dequantised into the bf16 weight stages
// (k_loop_mx below); sorted rows, the whole K range, K a multiple of 256.
// settle (optional): a value the hook loads (the next tile's number); the tile takes it after
// its K loop, before its output stores, so that waiting for that load cannot include them.
template <bool GATE_UP, int SRC, int WS, int DT, bool MX = false, typename Hook = NoHook>
__device__ __forceinline__ void wide_tile(const GemmProblem &g, int nblk, int mtile, int expert,
                                          moe_u32x4 *smem, int kbeg = 0, int kcnt = -1,
                                          float *part = nullptr, Hook hook = Hook(),
                                          const int *settle = nullptr)
{
    using St = Stage<kStep>;
    constexpr int kSlots = St::kSlots, kRows = St::kRowsPerLoad;
    constexpr int kXLoads = St::kXLoads, kWLoads = St::kWLoads;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / kWN, wn = wv % kWN;
    const int row0 = mtile * kBM;
    const int K = g.K;
    const int n_real = __builtin_amdgcn_readfirstlane(wide_real_rows<SRC>(g, row0));

    // output columns of this workgroup: gate-up kBW/2 (gate and up rows), down kBW
    const int cols_per_wg = GATE_UP ? kBW / 2 : kBW;
    const int col_wg = nblk * cols_per_wg;

    // ---- DMA sources.  Instruction j of this wave covers kRows consecutive tile rows; lane l
    // fetches chunk (l % kSlots) ^ swizzle(row) of row first + l / kSlots, which is the slot
    // that lane writes (a wave instruction fills 1 KB of LDS, lane l at 16 * l).
    const int lrow = lane / kSlots, lpos = lane % kSlots;
    const int w_rows = GATE_UP ? 2 * g.n_out : g.n_out;
    const uint16_t *W = MX ? nullptr : g.weight + (size_t)expert * w_rows * K;
    const uint16_t *wsrc[kWLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
        const int r = wv * (kBW / kWaves) + kRows * j + lrow;  // weight row within the tile
        // gate-up: rows [0, kBW/2) are gate rows of the workgroup's columns, [kBW/2, kBW) the
        // up rows of the same columns; rows past the last column read row 0 (never stored)
        const int c = col_wg + (GATE_UP ? r % (kBW / 2) : r);
        const bool ok = c < g.n_out;
        const int src = (GATE_UP && r >= kBW / 2) ? c + g.n_out : c;
        const int chunk = lpos ^ ((r >> 1) & (kSlots - 1));
        wsrc[j] = W + (size_t)(ok ? src : 0) * K + 8 * chunk;
    }
    const uint16_t *xsrc[kXLoads];
    bool xload[kXLoads];  // wave-uniform: the instruction's rows hold a real row
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
        const int rfirst = wv * (kBM / kWaves) + kRows * j;
        const int r = rfirst + lrow;
        xload[j] = rfirst < n_real;
        int src = 0;  // padding rows of a loaded group read row 0 (never stored)
        if (r < n_real)
            src = SRC == moe::ROWS_SORTED
                      ? (GATE_UP ? g.sorted_ids[row0 + r] / g.top_k : row0 + r)
                      : row0 + r;
        const int chunk = lpos ^ ((r >> 1) & (kSlots - 1));
        xsrc[j] = g.act + (size_t)src * K + 8 * chunk;
    }
    // LDS byte addresses: the activation stages, then the weight stages
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t x_dst = lds0 + wv * (kBM / kWaves) * (kStep * 2);
    const uint32_t w_dst = lds0 + kXStages * kHalf + wv * (kBW / kWaves) * (kStep * 2);

    // ---- operand rows of this wave
    // weight tile n of wave wn: gate-up: n < kNT32/2 -> gate rows 32*(kNT32/2)*wn + 32*n of the
    // gate half; n >= kNT32/2 -> the matching up rows.  down: rows 32*kNT32*wn + 32*n.
    int wrow0[kNT32];
#pragma unroll
    for (int n = 0; n < kNT32; ++n) {
        if (GATE_UP) {
            const int hn = n % (kNT32 / 2);
            const int base = 32 * (kNT32 / 2) * wn + 32 * hn;
            wrow0[n] = (n < kNT32 / 2) ? base : kBW / 2 + base;
        } else {
            wrow0[n] = 32 * kNT32 * wn + 32 * n;
        }
    }
    const int rr = lane & 31, rq = lane >> 5;
    // real 32-row tiles of this wave: tiles wm + 4i for i < mt_real (wave-uniform)
    int mt_real = 0;
#pragma unroll
    for (int i = 0; i < kMT32; ++i)
        mt_real += (32 * (wm + kWM * i) < n_real) ? 1 : 0;

    const int nk = kcnt < 0 ? K / kStep : kcnt;
    // every wave calls hook() once, after issuing the loads of k-step hook_at (three k-steps
    // before the tile's last)
    const int hook_at = nk > 3 ? nk - 3 : 0;
    const unsigned rkey = SRC == moe::ROWS_SORTED ? expert : nblk;
    // (MX: a multiple of 4, so every run of 4 visits from a multiple of 4 is one scale group)
    const int rot = MX ? (int)((rkey * 7u) % (unsigned)(nk / 4)) * 4
                       : (int)((rkey * 7u) % (unsigned)nk);

    moe_f32x16 acc[kMT32][kNT32];
#pragma unroll
    for (int m = 0; m < kMT32; ++m)
#pragma unroll
        for (int n = 0; n < kNT32; ++n)
            acc[m][n] = moe_f32x16{};

    auto issue_x = [&](int i) {
        const int kb = (kbeg + (i + rot) % nk) * kStep;  // element offset of k-step i
        const uint32_t so = (i % kXStages) * kHalf;
#pragma unroll
        for (int j = 0; j < kXLoads; ++j)
            if (xload[j])
                dma16(xsrc[j] + kb, x_dst + so + j * 1024);
    };
    auto issue_w = [&](int i) {
        const int kb = (kbeg + (i + rot) % nk) * kStep;
        const uint32_t so = (i % WS) * kHalf;
#pragma unroll
        for (int j = 0; j < kWLoads; ++j)
            dma16(wsrc[j] + kb, w_dst + so + j * 1024);
    };

    // Pipeline, A = WS - 1 weight k-steps ahead.  Issue order: x(0) w(0) .. w(A-1), then in step
    // i x(i+1) w(i+A).  Loads complete in issue order, so at the top of step i it is enough that
    // only the loads issued after x(i) and w(i) are left: w(i+A-1), which step i-1 issued after
    // x(i) (at step 0: w(1) .. w(A-1)).  That leaves this wave's parts of x(i) and w(i) in LDS,
    // and the barrier publishes every wave's parts.  It also guarantees that every wave has
    // finished step i-1, whose stages x(i+1) and w(i+A) then overwrite.  The loop is
    // instantiated per count MTR of real 32-row tiles of this wave, so the MFMA block has no
    // branches (a wave with none still loads its share and meets every barrier).
    auto k_loop = [&](auto mtr) {
        constexpr int MTR = decltype(mtr)::value;
        constexpr int A = WS - 1;
        issue_x(0);
#pragma unroll
        for (int s = 0; s < A; ++s)
            if (s < nk)
                issue_w(s);
        for (int i = 0; i < nk; ++i) {
            step_barrier((i == 0 ? min(A - 1, nk - 1) : (i + A - 1 < nk ? 1 : 0)) * kWLoads);
            if (i + 1 < nk)
                issue_x(i + 1);
            if (i + A < nk)
                issue_w(i + A);
            if (i == hook_at)
                hook();
            if (MTR == 0)
                continue;
            const moe_u32x4 *xb = smem + (i % kXStages) * (kHalf / 16);
            const moe_u32x4 *wb = smem + (kXStages + i % WS) * (kHalf / 16);
            // operands of 16-element sub-step h; those of h + 1 are read while the MFMAs of h
            // run, so the LDS latency hides behind 8 MFMAs instead of stalling them
            moe_u32x4 a[2][kNT32], b[2][MTR > 0 ? MTR : 1];
            auto read = [&](int buf, int h) {
#pragma unroll
                for (int m = 0; m < MTR; ++m)
                    b[buf][m] = xb[St::slot(32 * (wm + kWM * m) + rr, 2 * h + rq)];
#pragma unroll
                for (int n = 0; n < kNT32; ++n)
                    a[buf][n] = wb[St::slot(wrow0[n] + rr, 2 * h + rq)];
            };
            read(0, 0);
#pragma unroll
            for (int h = 0; h < kStep / 16; ++h) {
                if (h + 1 < kStep / 16)
                    read((h + 1) & 1, h + 1);
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of these MFMAs
#pragma unroll
                for (int n = 0; n < kNT32; ++n)
#pragma unroll
                    for (int m = 0; m < MTR; ++m)
                        acc[m][n] = moe_mma32<DT>(a[h & 1][n], b[h & 1][m], acc[m][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // ---- MXFP4 weights.  A k-step of the tile's 256 weight rows is 32 code bytes a row (two
    // e2m1 codes per byte, low nibble first) and, per group of 4 k-steps, 8 E8M0 scale bytes a
    // row (one per 32 elements); both come by DMA into LDS beside the activation rows, two
    // k-steps ahead (three stages each; the scales with a group's first k-step, two buffers).
    // No bf16 weight stage: each wave reads the codes of its own weight rows (one 16-byte read
    // per 32-row tile and k-step, conflict-free) and turns them into its MFMA A operands in
    // registers with v_cvt_scalef32_pk_bf16_fp4.  Within a k-step both operands take the k
    // order permuted alike: sub-step h, lane group rq takes elements 32rq + 8h .. + 7 (a lane's
    // 16 code bytes then serve all four sub-steps; each dot product is unchanged).  LDS:
    // activation stages [0, 96 KB), code slots [96, 120 KB), scale buffers [120, 124 KB).
    // DMA lanes: lane l of wave w covers weight row r = 32w + l/2 (codes: the row's 16-byte
    // half (l%2) ^ ((r >> 3) & 1) of the k-step, so that the halves of rows 8..15 of every 16
    // sit swapped and the 16-byte reads of 16 consecutive rows at one half hit distinct banks;
    // scales: the group's bytes 4(l%2) .. +3), writing LDS at 16l / 4l.
    constexpr int kMxStages = 3;
    constexpr uint32_t kMxCodeSlot = kBW * kStep / 2;
    constexpr uint32_t kMxCodes = kMxStages * kHalf;
    constexpr uint32_t kMxScaleBuf = kBW * 8;
    constexpr uint32_t kMxScales = kMxCodes + kMxStages * kMxCodeSlot;
    static_assert(kMxScales + 2 * kMxScaleBuf <= wide_lds_bytes<3>(), "MX stages fit the LDS");
    const uint8_t *mx_code = nullptr, *mx_scale = nullptr;
    if (MX) {
        const int r = wv * (kBW / kWaves) + (lane >> 1);  // weight row within the tile
        const int c = col_wg + (GATE_UP ? r % (kBW / 2) : r);
        const int src = (GATE_UP && r >= kBW / 2) ? c + g.n_out : c;
        const size_t row = (size_t)expert * w_rows + (c < g.n_out ? src : 0);
        mx_code = g.wq + row * (size_t)(K / 2) + 16 * ((lane & 1) ^ ((r >> 3) & 1));
        mx_scale = g.wscale + row * (size_t)(K / 32) + 4 * (lane & 1);
    }
    int mx_nx = 0;  // this wave's activation DMAs per k-step
#pragma unroll
    for (int j = 0; j < kXLoads; ++j)
        mx_nx += xload[j] ? 1 : 0;
    // k-step i's activation rows, codes and (at a group's first k-step) scales
    auto issue_mx = [&](int i) {
        const int ks = (i + rot) % nk;
        const int st = i % kMxStages;
#pragma unroll
        for (int j = 0; j < kXLoads; ++j)
            if (xload[j])
                dma16(xsrc[j] + ks * kStep, x_dst + st * kHalf + j * 1024);
        dma16(mx_code + ks * 32,
              __builtin_amdgcn_readfirstlane(lds0 + kMxCodes + st * kMxCodeSlot + wv * 1024));
        if (i % 4 == 0)
            dma4(mx_scale + ks * 2, __builtin_amdgcn_readfirstlane(
                                        lds0 + kMxScales + ((i / 4) % 2) * kMxScaleBuf + wv * 256));
    };
    auto mx_loads = [&](int i) {  // this wave's DMAs of k-step i (0 past the K loop)
        return i < nk ? mx_nx + 1 + (i % 4 == 0 ? 1 : 0) : 0;
    };
    // Step i: wait until only k-step i+1's loads are outstanding, barrier (every wave's parts
    // of k-step i landed, every wave done with step i-1); issue k-step i+2 into the stage and
    // slot step i-1 read (its scales into the buffer of group (i+2)/4 - 2, last read at step
    // i-3 or before); MFMAs of step i.
    auto k_loop_mx = [&](auto mtr) {
        constexpr int MTR = decltype(mtr)::value;
        issue_mx(0);
        if (1 < nk)
            issue_mx(1);
        for (int i = 0; i < nk; ++i) {
            step_barrier(mx_loads(i + 1));
            if (i + 2 < nk)
                issue_mx(i + 2);
            if (i == hook_at)
                hook();
            if (MTR == 0)
                continue;
            const int ks = (i + rot) % nk;
            const moe_u32x4 *xb = smem + (i % kMxStages) * (kHalf / 16);
            const uint8_t *sm8 = reinterpret_cast<const uint8_t *>(smem);
            const uint8_t *cs = sm8 + kMxCodes + (i % kMxStages) * kMxCodeSlot;
            const uint8_t *ss = sm8 + kMxScales + ((i / 4) % 2) * kMxScaleBuf;
            moe_u32x4 q[kNT32];
            float sc[kNT32];
#pragma unroll
            for (int n = 0; n < kNT32; ++n) {
                const int r = wrow0[n] + rr;
                q[n] = *reinterpret_cast<const moe_u32x4 *>(cs + r * 32 + 16 * (rq ^ ((r >> 3) & 1)));
                sc[n] = moe_mx::e8m0_to_f32(ss[r * 8 + (ks % 4) * 2 + rq]);
            }
            moe_u32x4 b[2][MTR > 0 ? MTR : 1];
            auto read_b = [&](int buf, int h) {
#pragma unroll
                for (int m = 0; m < MTR; ++m)
                    b[buf][m] = xb[St::slot(32 * (wm + kWM * m) + rr, 4 * rq + h)];
            };
            read_b(0, 0);
#pragma unroll
            for (int h = 0; h < kStep / 16; ++h) {
                if (h + 1 < kStep / 16)
                    read_b((h + 1) & 1, h + 1);
                moe_u32x4 a[kNT32];
#pragma unroll
                for (int n = 0; n < kNT32; ++n) {
                    const uint32_t w = h == 0 ? q[n].x : h == 1 ? q[n].y : h == 2 ? q[n].z : q[n].w;
                    a[n] = moe_mx::dequant8(w, sc[n]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n = 0; n < kNT32; ++n)
#pragma unroll
                    for (int m = 0; m < MTR; ++m)
                        acc[m][n] = moe_mma32<DT>(a[n], b[h & 1][m], acc[m][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Tiles of at most kSmallRows real rows (the few-row experts of prefill, an expert's ragged
    // last tile) are bound by their weight stream, not by MFMAs.  Their activation rows fit
    // 8 KB stages, so the LDS holds four stages of both operands and the weights run three
    // k-steps ahead instead of two: 96 KB of weights in flight per CU, which lets these tiles
    // draw more than an even share of HBM while tiles of fuller experts on other CUs are busy
    // with MFMAs.  Each wave fetches 8 of the 64 activation rows and its 32 weight rows per
    // k-step; both operands of a k-step are issued together, so one wait covers them.
    auto k_loop_small = [&](auto mtr) {
        constexpr int MTR = decltype(mtr)::value;   // 0 or 1 (rows < 64: tile m = 0 only)
        constexpr int SA = kSmallStages - 1;        // k-steps ahead
        static_assert(kSmallStages * (kSmallX + kHalf) <= wide_lds_bytes<WS>(),
                      "the small pipeline fits this kernel's LDS");
        const int srow = 8 * wv + lrow;             // this lane's activation row of the tile
        const bool sxl = 8 * wv < n_real;           // wave-uniform: its 8 rows hold a real row
        int ssrc = 0;
        if (srow < n_real)
            ssrc = SRC == moe::ROWS_SORTED
                       ? (GATE_UP ? g.sorted_ids[row0 + srow] / g.top_k : row0 + srow)
                       : row0 + srow;
        const uint16_t *sx = g.act + (size_t)ssrc * K + 8 * (lpos ^ ((srow >> 1) & (kSlots - 1)));
        const uint32_t sx_dst = lds0 + wv * 1024;
        const uint32_t sw_dst = lds0 + kSmallStages * kSmallX + wv * (kBW / kWaves) * (kStep * 2);
        const int per_step = kWLoads + (sxl ? 1 : 0);
        auto issue = [&](int i) {
            const int kb = (kbeg + (i + rot) % nk) * kStep;
            const int st = i % kSmallStages;
            if (sxl)
                dma16(sx + kb, sx_dst + st * kSmallX);
#pragma unroll
            for (int j = 0; j < kWLoads; ++j)
                dma16(wsrc[j] + kb, sw_dst + st * kHalf + j * 1024);
        };
#pragma unroll
        for (int s = 0; s < SA; ++s)
            if (s < nk)
                issue(s);
        for (int i = 0; i < nk; ++i) {
            // at most the loads of steps i+1 .. i+SA-1 may still be in flight: this wave's part
            // of step i has landed; the barrier publishes every wave's part and guarantees that
            // every wave is done with step i-1, whose stage step i+SA overwrites
            step_barrier(min(SA - 1, nk - 1 - i) * per_step);
            if (i + SA < nk)
                issue(i + SA);
            if (i == hook_at)
                hook();
            if (MTR == 0)
                continue;
            const int st = i % kSmallStages;
            const moe_u32x4 *xb = smem + st * (kSmallX / 16);
            const moe_u32x4 *wb = smem + (kSmallStages * kSmallX + st * kHalf) / 16;
            moe_u32x4 a[2][kNT32], b[2];
            auto read = [&](int buf, int h) {
                b[buf] = xb[St::slot(32 * wm + rr, 2 * h + rq)];
#pragma unroll
                for (int n = 0; n < kNT32; ++n)
                    a[buf][n] = wb[St::slot(wrow0[n] + rr, 2 * h + rq)];
            };
            read(0, 0);
#pragma unroll
            for (int h = 0; h < kStep / 16; ++h) {
                if (h + 1 < kStep / 16)
                    read((h + 1) & 1, h + 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n = 0; n < kNT32; ++n)
                    acc[0][n] = moe_mma32<DT>(a[h & 1][n], b[h & 1], acc[0][n]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (MX) {
        switch (mt_real) {
        case 0: k_loop_mx(std::integral_constant<int, 0>()); break;
        case 1: k_loop_mx(std::integral_constant<int, 1>()); break;
        default: k_loop_mx(std::integral_constant<int, 2>()); break;
        }
    } else if (n_real <= kSmallRows) {
        if (mt_real == 0)
            k_loop_small(std::integral_constant<int, 0>());
        else
            k_loop_small(std::integral_constant<int, 1>());
    } else {
        switch (mt_real) {
        case 0: k_loop(std::integral_constant<int, 0>()); break;
        case 1: k_loop(std::integral_constant<int, 1>()); break;
        default: k_loop(std::integral_constant<int, 2>()); break;
        }
    }

    if (settle != nullptr)
        asm volatile("" ::"v"(*settle));

    // ---- epilogue.  For weight tile n, register 4q' + q holds column 8q' + 4*(lane/32) + q of
    // the tile, row 32*(wm + 4m) + lane%32.  The bf16 tile (kBM rows x TC columns) goes through
    // LDS so that global stores write whole rows: 16-byte chunk c of row r sits at chunk
    // position c ^ (r % CPR) of the row (the 8-byte writes of 32 rows at one column then
    // spread over the banks; the 16-byte reads of one row stay conflict-free).
    if (part != nullptr) {
        // register 4q' + q of weight tile n: weight row wrow0[n] + 8q' + 4*(lane/32) + q of the
        // tile, activation row 32*(wm + 4m) + lane%32; four consecutive f32 per store
#pragma unroll
        for (int m = 0; m < kMT32; ++m) {
            if (m >= mt_real)
                continue;
            const int r = 32 * (wm + kWM * m) + rr;
            if (r >= n_real)
                continue;
#pragma unroll
            for (int n = 0; n < kNT32; ++n)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    moe_f32x4 v;
                    v.x = acc[m][n][4 * q4 + 0];
                    v.y = acc[m][n][4 * q4 + 1];
                    v.z = acc[m][n][4 * q4 + 2];
                    v.w = acc[m][n][4 * q4 + 3];
                    *reinterpret_cast<moe_f32x4 *>(
                        part + (size_t)r * kBW + wrow0[n] + 8 * q4 + 4 * rq) = v;
                }
        }
        return;
    }
    constexpr int TC = GATE_UP ? kBW / 2 : kBW;  // output columns of the tile
    constexpr int CPR = TC / 8;                  // 16-byte chunks per row
    constexpr int RSTEP = kThreads / CPR;        // rows stored per pass of the workgroup
    static_assert(kBM * TC * 2 <= wide_lds_bytes<2>(), "output tile fits in LDS");
    // The down GEMM on sorted rows writes each row to its route's row.  Those 256 lookups are
    // issued together (one per thread) before the staging and kept in LDS past the output tile,
    // so the store loop does not wait on a lookup before each store.
    constexpr bool kRouteDst = SRC == moe::ROWS_SORTED && !GATE_UP;
    static_assert(kBM * TC * 2 + kBM * 4 <= wide_lds_bytes<WS>(), "lookups fit beside the tile");
    int my_dst = -1;
    if (kRouteDst && tid < kBM && tid < n_real)
        my_dst = g.sorted_ids[row0 + tid];
    __syncthreads();  // every wave is done with the last k-step's operands
    uint16_t *otile = reinterpret_cast<uint16_t *>(smem);
    int *s_dst = reinterpret_cast<int *>(smem) + kBM * TC * 2 / 4;
    auto opos = [](int r, int c) { return r * CPR + (c ^ (r & (CPR - 1))); };
#pragma unroll
    for (int m = 0; m < kMT32; ++m) {
        if (m >= mt_real)
            continue;
        const int r = 32 * (wm + kWM * m) + rr;
        constexpr int NOUT = GATE_UP ? kNT32 / 2 : kNT32;
#pragma unroll
        for (int n = 0; n < NOUT; ++n) {
            const int lc0 = (GATE_UP ? 32 * (kNT32 / 2) * wn : 32 * kNT32 * wn) + 32 * n;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (GATE_UP) {
                        const float gate = acc[m][n][4 * q4 + q];
                        const float up = acc[m][n + kNT32 / 2][4 * q4 + q];
                        v[q] = gate / (1.0f + __expf(-gate)) * up;
                    } else {
                        v[q] = acc[m][n][4 * q4 + q];
                    }
                }
                moe_u32x2 packed;
                packed.x = moe_pack2<DT>(v[0], v[1]);
                packed.y = moe_pack2<DT>(v[2], v[3]);
                const int lc = lc0 + 8 * q4;  // first column of the 16-byte chunk
                *reinterpret_cast<moe_u32x2 *>(otile + 8 * opos(r, lc / 8) + 4 * rq) = packed;
            }
        }
    }
    if (kRouteDst && tid < kBM)
        s_dst[tid] = my_dst;
    __syncthreads();
    // thread t stores chunk t % CPR of rows t / CPR, t / CPR + RSTEP, ...
    const int oc = tid % CPR;
    const int col = col_wg + 8 * oc;
    if (col < g.n_out) {
        for (int r = tid / CPR; r < n_real; r += RSTEP) {
            const int dst = kRouteDst ? s_dst[r] : row0 + r;
            // output rows are read once, by a later launch: non-temporal, so they do not evict
            // the operands this launch's other tiles still share through L2
            __builtin_nontemporal_store(
                *reinterpret_cast<const moe_u32x4 *>(otile + 8 * opos(r, oc)),
                reinterpret_cast<moe_u32x4 *>(g.out + (size_t)dst * g.n_out + col));
        }
    }
}

// Barrier between tiles: only LDS accesses need ordering there (the epilogue's reads of its
// staged output, the tile number passed through LDS), so it waits on lgkmcnt alone and the
// tile's output stores stay in flight.  The next tile's counted DMA waits stay correct with
// older stores outstanding: a load's data only returns after the loads issued before it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile t of the schedule's range p (p = 0..8: the range starts, in tiles of a GEMM with
// n_blocks column blocks; range 8's start is the tile count).
__device__ __forceinline__ int sched_bound(const moe::TileSchedule *sched, int p, int n_blocks,
                                           int total)
{
    if (p <= 0)
        return 0;
    if (p >= moe::kSchedParts)
        return total;
    const int b = __float2int_rn(sched->bounds[p] * (float)n_blocks);
    return min(max(b, 0), total);
}

// Sorted rows with a schedule: a persistent workgroup on XCD x (= blockIdx % 8) takes the next
// tile of range x from its counter (one atomic per tile; tiles of one expert stay on one XCD
// and share its L2), and once range x is used up, the next tiles of ranges x+1, x+2, ...  The
// workgroup leaves when every range is used up; the last one to leave zeroes the counters for
// the next launch.  No workgroup ever waits for another.
template <bool GATE_UP, int SRC, int WS, int DT, bool MX = false>
__device__ __forceinline__ void wide_queue_loop(const GemmProblem &g, int n_blocks, int total,
                                                moe_u32x4 *smem)
{
    constexpr int P = moe::kSchedParts;
    // thread 0 passes the tile number through the first word of the (idle) stage memory.  An
    // LDS-typed pointer: through a generic one these were flat accesses, which the compiler
    // waits for with vmcnt(0) -- and so for every output store of the tile just finished.
    volatile __attribute__((address_space(3))) int *s_next =
        (volatile __attribute__((address_space(3))) int *)(smem);

    moe::TileSchedule *sched = g.sched;
    const int home = blockIdx.x % kXcds;
    // thread 0's state: ranges found used up, the bounds [lo, hi) of the range it takes from,
    // and the counter value of a take issued during the current tile (-1: none)
    int tried = 0, lo = 0, hi = 0, pend = -1;
    auto range = [&]() {
        const int p = (home + tried) % P;
        lo = sched_bound(sched, p, n_blocks, total);
        hi = sched_bound(sched, p + 1, n_blocks, total);
    };
    auto next_tile = [&]() -> int {
        while (tried < P) {
            if (lo < hi) {
                const int n = pend >= 0 ? pend : atomicAdd(&sched->queue[(home + tried) % P], 1);
                pend = -1;
                if (n < hi - lo)
                    return lo + n;
            }
            pend = -1;
            if (++tried < P)
                range();
        }
        return -1;
    };
    if (threadIdx.x == 0) {
        range();
        *s_next = next_tile();
    }
    lds_barrier();
    int t = *s_next;
    lds_barrier();  // every wave has read it before the tile's loads overwrite the stage
    while (t >= 0) {
        int nblk, mtile, expert;
        wide_decode<SRC>(g, t, n_blocks, 0, nblk, mtile, expert);
        // Three k-steps before the tile ends, thread 0 takes the next tile number from its
        // range's counter; the round trip overlaps the tile's last k-steps and the result is
        // first read after the tile (the take needs no load: the bounds are in registers).
        wide_tile<GATE_UP, SRC, WS, DT, MX>(
            g, nblk, mtile, expert, smem, 0, -1, nullptr,
            [&]() {
                if (threadIdx.x == 0 && tried < P && lo < hi)
                    pend = atomicAdd(&sched->queue[(home + tried) % P], 1);
            },
            &pend);
        lds_barrier();  // every wave is done with the tile's LDS
        if (threadIdx.x == 0)
            *s_next = next_tile();
        lds_barrier();
        t = *s_next;
        lds_barrier();  // every wave has read it before the next tile's loads overwrite it
    }
    if (threadIdx.x == 0) {
        // thread 0's counter updates are complete (their results were used); the last
        // workgroup out sees every other one's and zeroes the counters
        __threadfence();
        if (atomicAdd(&sched->queue[P], 1) == (int)gridDim.x - 1) {
            for (int p = 0; p <= P; ++p)
                atomicExch(&sched->queue[p], 0);
        }
    }
}

// K split of the dense tiles (the shared expert at a few hundred tokens has too few 256 x 256
// tiles for a whole number of rounds over the CUs): the launch's units are its first
// total - n_split tiles whole, then each of the last n_split tiles as q_split parts of its K
// loop, part j covering k-steps [j*nk/q_split, (j+1)*nk/q_split).  Units are dealt like tiles
// (XCD-contiguous ranges per round); part j of split tile s writes f32 partial (s*q_split + j).
__host__ __device__ inline int wide_split_units(int total, int n_split, int q_split)
{
    return total - n_split + n_split * q_split;
}

template <bool GATE_UP, int SRC, int WS, int DT>
__device__ __forceinline__ void wide_split_loop(const GemmProblem &g, int n_blocks, int m_tiles,
                                                int total, moe_u32x4 *smem)
{
    const int n_split = g.split_tiles, q_split = g.split_parts;
    const int whole = total - n_split;
    const int units = wide_split_units(total, n_split, q_split);
    const int W = min((int)gridDim.x, (units + kXcds - 1) / kXcds * kXcds);
    const int per = W / kXcds;
    const int idx = blockIdx.x / kXcds;
    if (idx >= per)
        return;
    const int nk = g.K / kStep;
    for (int u = (blockIdx.x % kXcds) * per + idx; u < units; u += W) {
        int t = u, kbeg = 0, kcnt = -1;
        float *part = nullptr;
        if (u >= whole) {
            const int s = (u - whole) / q_split, j = (u - whole) % q_split;
            t = whole + s;
            kbeg = j * nk / q_split;
            kcnt = (j + 1) * nk / q_split - kbeg;
            part = g.partial + (size_t)(s * q_split + j) * (kBM * kBW);
        }
        int nblk, mtile, expert;
        wide_decode<SRC>(g, t, n_blocks, m_tiles, nblk, mtile, expert);
        wide_tile<GATE_UP, SRC, WS, DT>(g, nblk, mtile, expert, smem, kbeg, kcnt, part);
        __syncthreads();  // the next unit's first loads follow every wave's last reads
    }
}

// Sum of the K parts of the split tiles, in part order, and the tile epilogue: gate-up ->
// SiLU(gate)*up, down -> the sum; rounded once to the element type.  One thread per 8 output
// columns of one activation row of one split tile.
template <bool GATE_UP, int DT>
__global__ __launch_bounds__(256) void k_wide_reduce(GemmProblem g, int n_blocks, int m_tiles,
                                                     int total)
{
    constexpr int TC = GATE_UP ? kBW / 2 : kBW;  // output columns of a tile
    constexpr int C8 = TC / 8;
    const int n_split = g.split_tiles, q_split = g.split_parts;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_split * kBM * C8)
        return;
    const int s = i / (kBM * C8), r = (i / C8) % kBM, c8 = i % C8;
    const int t = total - n_split + s;
    const int nblk = t / m_tiles, mtile = t % m_tiles;
    const int row = mtile * kBM + r;
    const int col = nblk * TC + 8 * c8;
    if (row >= g.rows || col >= g.n_out)
        return;
    float a[8] = {}, b[8] = {};
    for (int j = 0; j < q_split; ++j) {
        const float *p = g.partial + (size_t)(s * q_split + j) * (kBM * kBW) + (size_t)r * kBW;
        const moe_f32x4 a0 = *reinterpret_cast<const moe_f32x4 *>(p + 8 * c8);
        const moe_f32x4 a1 = *reinterpret_cast<const moe_f32x4 *>(p + 8 * c8 + 4);
        a[0] += a0.x; a[1] += a0.y; a[2] += a0.z; a[3] += a0.w;
        a[4] += a1.x; a[5] += a1.y; a[6] += a1.z; a[7] += a1.w;
        if (GATE_UP) {  // the up rows of the same columns: weight rows 128 + c
            const moe_f32x4 b0 = *reinterpret_cast<const moe_f32x4 *>(p + TC + 8 * c8);
            const moe_f32x4 b1 = *reinterpret_cast<const moe_f32x4 *>(p + TC + 8 * c8 + 4);
            b[0] += b0.x; b[1] += b0.y; b[2] += b0.z; b[3] += b0.w;
            b[4] += b1.x; b[5] += b1.y; b[6] += b1.z; b[7] += b1.w;
        }
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = GATE_UP ? a[e] / (1.0f + __expf(-a[e])) * b[e] : a[e];
    moe_u32x4 o;
    o.x = moe_pack2<DT>(v[0], v[1]);
    o.y = moe_pack2<DT>(v[2], v[3]);
    o.z = moe_pack2<DT>(v[4], v[5]);
    o.w = moe_pack2<DT>(v[6], v[7]);
    *reinterpret_cast<moe_u32x4 *>(g.out + (size_t)row * g.n_out + col) = o;
}

// Round r hands XCD x the tiles [r*W + x*W/8, r*W + (x+1)*W/8), W = the slots in use.
template <bool GATE_UP, int SRC, int WS, int DT>
__global__ __launch_bounds__(kThreads) void k_wide_gemm(GemmProblem g, int n_blocks, int m_tiles)
{
    __shared__ moe_u32x4 smem[wide_lds_bytes<WS>() / 16];

    const int total = wide_total<SRC>(g, n_blocks, m_tiles);
    if (SRC == moe::ROWS_SORTED && g.sched != nullptr) {
        wide_queue_loop<GATE_UP, SRC, WS, DT>(g, n_blocks, total, smem);
        return;
    }
    if (SRC != moe::ROWS_SORTED && g.partial != nullptr) {
        wide_split_loop<GATE_UP, SRC, WS, DT>(g, n_blocks, m_tiles, total, smem);
        return;
    }
    const int W = min((int)gridDim.x, (total + kXcds - 1) / kXcds * kXcds);
    const int per = W / kXcds;
    const int idx = blockIdx.x / kXcds;
    if (idx >= per)
        return;
    for (int t = (blockIdx.x % kXcds) * per + idx; t < total; t += W) {
        int nblk, mtile, expert;
        wide_decode<SRC>(g, t, n_blocks, m_tiles, nblk, mtile, expert);
        wide_tile<GATE_UP, SRC, WS, DT>(g, nblk, mtile, expert, smem);
        __syncthreads();  // the next tile's first loads follow every wave's last reads
    }
}

// MXFP4 weights on sorted rows with a schedule (the queue loop above, k_loop_mx per tile).
template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) void k_wide_mx(GemmProblem g, int n_blocks, int m_tiles)
{
    __shared__ moe_u32x4 smem[wide_lds_bytes<3>() / 16];
    const int total = wide_total<moe::ROWS_SORTED>(g, n_blocks, m_tiles);
    wide_queue_loop<GATE_UP, moe::ROWS_SORTED, 3, 0, true>(g, n_blocks, total, smem);
}

}  // namespace moe_wide
