// moe_fp8_kernel.h -- block-scaled FP8 grouped GEMM of the masked layout (TileOPs "MoE" page,
// MoEGroupedGemmFP8Fwd: a [E, layout.max_m, K] e4m3 with a_scale [E, layout.max_m, K/128] f32,
// b [E, N, K] e4m3 with b_scale [E, N/128, K/128] f32, layout_metadata [E] = rows in use):
//
//   out[e, m, n] = bf16( sum_kb a_scale[e, m, kb] * b_scale[e, n/128, kb]
//                        * sum_{k in block kb} a[e, m, k] * b[e, n, k] ),  m < masked_m[e]
//
// and of the contiguous layout of the page's grouped GEMMs (a [P, K], expert e owning rows
// [offsets[e], offsets[e+1])), the same sum per row.
//
// Built like the row-tiled bf16 kernel, for the decode and small-batch shapes the page lists
// (64 to 256 rows per expert; weight-bandwidth bound):
//   - a workgroup (4 waves) owns a BM-row tile of one expert's block and 4 * NTW 16-column
//     tiles of the output; wave w owns NTW of them and streams its own weight rows with
//     non-temporal 16-byte loads covering whole 128-byte lines (8 lanes per row), STAGES-1
//     k-steps ahead, through a per-wave swizzled LDS transpose into the MFMA A operand;
//   - a k-step is 128 elements: one 128-byte line per row, one scale block, and one
//     v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 x e4m3, hardware block scales left at 1.0) per
//     pair of 16-row tiles.  A lane's four results share one output row and one 128-column
//     weight block, so the block's partial sum is scaled by a_scale * b_scale (f32) and added to
//     the f32 accumulator;
//   - the tile's activation rows of a k-step are loaded once per workgroup into a
//     double-buffered swizzled LDS tile read by all four waves (one barrier per k-step);
//   - tiles are numbered expert by expert, column block by column block, the row tiles of a
//     column block innermost; blocks are dealt round-robin to the 8 XCDs, each XCD taking a
//     contiguous range, so an expert's activation tile and each weight tile are shared through
//     one L2, and every tile of an expert starts its K loop at the same k-step.
// A lane ends with four consecutive output columns of one row.
//
// k_fp8_wide is the same computation on the 256 x 256 tile of moe_wide_kernel.h, for blocks of
// ~128 rows and more: 8 waves, both operands loaded straight into LDS (a 128-element FP8 k-step
// is the 128-byte row segment that kernel's load path and swizzle are built for), 16-row tiles
// without rows in use skipped, so each weight byte is requested once per 256 rows.  It needs
// K % 512 == 0, K <= 16384 and a 16-byte aligned a_scale (activation scales are staged 4
// blocks at a time; a wave holds its column block's weight scales in two registers).  The block sums of one weight tile are scaled while the next tile's MFMAs run.
#pragma once

#include <type_traits>

#include "moe_device.h"
#include "moe_fp8_quant.h"
#include "moe_wide_kernel.h"
#include "moe_ws_kernel.h"

namespace moe_fp8 {

// Masked layout (offsets == nullptr): expert e's rows are a[e, 0 .. masked_m[e]) of
// a [E, max_m, K].  Contiguous layout: a [P, K], expert e's rows are [offsets[e], offsets[e+1])
// (the TileOPs page's layout=contiguous with physical prefix-sum metadata); a_scale and out
// follow a's rows.
struct Fp8Problem {
    const uint8_t *a;         // [E, max_m, K] or [P, K] e4m3
    const float *a_scale;     // [E, max_m, KB] or [P, KB]
    const uint8_t *b;         // [E, N, K] e4m3
    const float *b_scale;     // [E, NB, KB]
    const int32_t *masked_m;  // [E] (masked layout)
    const int32_t *offsets;   // [E + 1] (contiguous layout), else nullptr
    uint16_t *out;            // [E, max_m, N] or [P, N] bf16
    int E, max_m, P, N, K, KB, NB;
    // contiguous layout, optional: row q of a and a_scale is row a_route[q] / a_div of them
    // (the FP8 pass quantises each token once and its gate-up GEMM reads a route's row as its
    // token's); nullptr: row q is row q
    const int32_t *a_route;
    int a_div;
};

// Row of a / a_scale that contiguous row q reads.
__device__ __forceinline__ size_t fp8_arow(const Fp8Problem &p, int q)
{
    return p.a_route ? (size_t)(p.a_route[q] / p.a_div) : (size_t)q;
}

constexpr int kWaves = 4;
constexpr int kXcds = 8;

typedef int moe_i32x8 __attribute__((ext_vector_type(8)));

__host__ __device__ inline int fp8_grid(int tiles)
{
    return (tiles + kXcds - 1) / kXcds * kXcds;
}

// One tile of a launch: its expert, column block, the a/out row of its first row, its rows.
struct Fp8Tile {
    int expert, nblk, rbase, n_rows;
};

// Rows of expert e in the contiguous layout: [r0, r1) of offsets, clamped to [0, P].
__device__ __forceinline__ void contig_rows(const Fp8Problem &p, int e, int &r0, int &r1)
{
    r0 = min(max(p.offsets[e], 0), p.P);
    r1 = min(max(p.offsets[e + 1], r0), p.P);
}

// Row tile j of an expert with r rows: its first row and its row count (<= 0: no rows).
template <int BM, bool EVEN>
__device__ __forceinline__ void fp8_tile_rows(int r, int j, int &row0, int &n)
{
    const int te = (r + BM - 1) / BM;
    if (!EVEN || j >= te) {
        row0 = j * BM;
        n = min(BM, r - row0);
        return;
    }
    const int q = r / te, rm = r % te;
    row0 = j * q + min(j, rm);
    n = q + (j < rm ? 1 : 0);
}

// Tile of this workgroup.  Tiles are numbered expert by expert, column blocks, then the BM-row
// tiles of the expert innermost, and blocks are dealt to the 8 XCDs (blockIdx % 8) as
// contiguous ranges of tile numbers.  Masked layout: m_tiles row tiles per expert (tiles past
// its rows in use are empty).  Contiguous layout: ceil(rows / BM) per expert; every wave sums
// them over the experts itself (lane l a run of ceil(E/64) experts, then a wave prefix sum),
// which gives the tile count and, by a ballot, the expert of tile t.  EVEN: an expert's r rows
// are spread over its ceil(r / BM) row tiles as evenly as they go (the first r mod te tiles one
// row more) instead of filling them in order, so its tiles move through the same weight slices
// at one pace.  Wave-uniform; false: no tile for this workgroup.
template <int BM, bool EVEN = false>
__device__ __forceinline__ bool fp8_locate(const Fp8Problem &p, int n_blocks, int m_tiles,
                                           Fp8Tile &o)
{
    const int idx = blockIdx.x / kXcds;
    if (p.offsets == nullptr) {
        const int per_expert = n_blocks * m_tiles;
        const int total = p.E * per_expert;
        const int per = fp8_grid(total) / kXcds;
        const int t = (blockIdx.x % kXcds) * per + idx;
        if (idx >= per || t >= total)
            return false;
        o.expert = t / per_expert;
        const int rem = t - o.expert * per_expert;
        o.nblk = rem / m_tiles;
        const int j = rem - o.nblk * m_tiles;
        const int rows_used = min(max(p.masked_m[o.expert], 0), p.max_m);
        int row0;
        fp8_tile_rows<BM, EVEN>(rows_used, j, row0, o.n_rows);
        o.rbase = o.expert * p.max_m + row0;
        return o.n_rows > 0;
    }
    // Lane l owns the run of experts [e0, e1), run = ceil(E / 64) <= 16 (E <= 1024): its
    // run + 1 offsets are loaded together (indices clamped to E, so every load is in bounds and
    // issued on every path; one wait), the run's tile counts summed and prefix-summed over the
    // wave.  The lane whose range holds tile t finds the expert in its registers, and every
    // lane reads that lane's result.
    constexpr int kMaxRun = 16;
    const int lane = threadIdx.x & 63;
    const int run = (p.E + 63) / 64;
    const int e0 = min(p.E, lane * run);
    int off[kMaxRun + 1];
#pragma unroll
    for (int j = 0; j <= kMaxRun; ++j)
        off[j] = p.offsets[min(e0 + j, p.E)];
    // rows of expert e0 + j as contig_rows gives them: [lo_j, hi_j), lo_j = clamp(off_j, 0, P),
    // hi_j = clamp(off_{j+1}, lo_j, P); experts past the run or past E count none
    int cnt[kMaxRun], lo[kMaxRun];
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kMaxRun; ++j) {
        lo[j] = min(max(off[j], 0), p.P);
        const int hi = min(max(off[j + 1], lo[j]), p.P);
        cnt[j] = (j < run && e0 + j < p.E) ? hi - lo[j] : 0;
        mine += (cnt[j] + BM - 1) / BM * n_blocks;
    }
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d)
            incl += v;
    }
    const int total = __shfl(incl, 63);
    const int per = fp8_grid(total) / kXcds;
    const int t = (blockIdx.x % kXcds) * per + idx;
    if (idx >= per || t >= total)
        return false;
    const unsigned long long hit = __ballot(t >= incl - mine && t < incl);
    const int owner = __ffsll((long long)hit) - 1;
    // every lane walks its own run for t (only the owner's walk is used)
    int cum = incl - mine, je = 0, r0 = 0, c = 0;
#pragma unroll
    for (int j = 0; j < kMaxRun; ++j) {
        const int te = (cnt[j] + BM - 1) / BM * n_blocks;
        if (t >= cum && t < cum + te && c == 0) {
            je = j;
            r0 = lo[j];
            c = cnt[j];
        }
        if (c == 0)
            cum += te;
    }
    const int e = __builtin_amdgcn_readlane(e0 + je, owner);
    cum = __builtin_amdgcn_readlane(cum, owner);
    r0 = __builtin_amdgcn_readlane(r0, owner);
    const int r1 = r0 + __builtin_amdgcn_readlane(c, owner);
    const int mt_e = (r1 - r0 + BM - 1) / BM;
    const int rem = t - cum;
    o.expert = e;
    o.nblk = rem / mt_e;
    int row0;
    fp8_tile_rows<BM, EVEN>(r1 - r0, rem - o.nblk * mt_e, row0, o.n_rows);
    o.rbase = r0 + row0;
    return o.n_rows > 0;
}

__device__ __forceinline__ moe_u32x4 load_nt16(const uint8_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const moe_u32x4 *>(p));
}

__device__ __forceinline__ moe_u32x4 load16(const uint8_t *p)
{
    return *reinterpret_cast<const moe_u32x4 *>(p);
}

// 32 bytes of one operand row for the 16x16x128 MFMA: chunks c and c + 4 of the 128-byte row
// segment (the same pair for both operands, so each lane group covers the same 32 k-values).
__device__ __forceinline__ moe_i32x8 join(moe_u32x4 lo, moe_u32x4 hi)
{
    return moe_i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ moe_f32x4 mfma_fp8_block(moe_i32x8 a, moe_i32x8 b)
{
    // format selectors 0/0: both operands OCP e4m3; block scales 127 (E8M0) = 1.0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, moe_f32x4{0.f, 0.f, 0.f, 0.f},
                                                            0, 0, 0, 127, 0, 127);
}

template <int BM, int NTW, int STAGES>
__global__ __launch_bounds__(64 * kWaves) void k_fp8_gemm(Fp8Problem p, int n_blocks, int m_tiles)
{
    constexpr int TM = BM / 16;                  // 16-row MFMA tiles of the row tile
    constexpr int XI = BM / (8 * kWaves);        // activation load instructions per wave
    static_assert(BM % (8 * kWaves) == 0, "BM must be a multiple of 32");
    __shared__ moe_u32x4 s_x[2][BM * 8];          // activation tile, 16-byte slots
    __shared__ moe_u32x4 s_t[kWaves][NTW * 128];  // per-wave weight transpose buffers

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- tile: expert-major, column blocks, row tiles innermost; XCD-contiguous ranges
    Fp8Tile tile;
    if (!fp8_locate<BM>(p, n_blocks, m_tiles, tile))
        return;
    const int expert = tile.expert, nblk = tile.nblk, rbase = tile.rbase;
    const int n_rows = tile.n_rows;
    const int K = p.K, KB = p.KB;
    const int col0 = nblk * (16 * NTW * kWaves) + wv * (16 * NTW);

    // ---- weight rows of this wave: lane reads chunk lane%8 of rows lane/8 and 8 + lane/8
    const uint8_t *B = p.b + (size_t)expert * p.N * K;
    const int lrow = lane >> 3, lchunk = lane & 7;
    const uint8_t *wld[NTW];
    bool tile_ok[NTW];
    int sb_base[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < p.N;
        const int cc = tile_ok[nt] ? c : 0;
        wld[nt] = B + (size_t)(cc + lrow) * K + 16 * lchunk;
        sb_base[nt] = (expert * p.NB + cc / 128) * KB;
    }
    moe_u32x4 *tbuf = s_t[wv];
    const int wslot0 = lrow * 8 + (lchunk ^ (lrow >> 1));
    const int wslot1 = (lrow + 8) * 8 + (lchunk ^ ((lrow + 8) >> 1));
    const int rr = lane & 15, rq = lane >> 4;
    const int rslot0 = rr * 8 + (rq ^ (rr >> 1));
    const int rslot1 = rr * 8 + ((rq + 4) ^ (rr >> 1));

    // ---- activation rows this lane loads: tile rows wv*BM/4 + 8*i + lane/8, chunk lane%8;
    // rows past the rows in use read the tile's first row (their results are never stored)
    const uint8_t *xld[XI];
    int xslot[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = wv * (BM / kWaves) + 8 * i + lrow;
        const int src = r < n_rows ? r : 0;
        xld[i] = p.a + fp8_arow(p, rbase + src) * K + 16 * lchunk;
        xslot[i] = r * 8 + (lchunk ^ ((r >> 1) & 7));
    }
    // a_scale rows of this lane's results: row 16*mt + lane%16 of the tile
    size_t sa_base[TM];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
        const int r = 16 * mt + rr;
        sa_base[mt] = fp8_arow(p, rbase + (r < n_rows ? r : 0)) * KB;
    }

    const int rot = (int)((expert * 7u) % (unsigned)KB);

    moe_f32x4 acc[TM][NTW];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
            acc[mt][nt] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

    moe_u32x4 wraw[STAGES][NTW][2], xraw[STAGES][XI];
    float sa[STAGES][TM], sb[STAGES][NTW];
    auto load = [&](int st, int i) {
        const int kb = (i + rot) % KB;
        const int k = kb * 128;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            wraw[st][nt][0] = load_nt16(wld[nt] + k);
            wraw[st][nt][1] = load_nt16(wld[nt] + (size_t)8 * K + k);
            sb[st][nt] = p.b_scale[sb_base[nt] + kb];
        }
#pragma unroll
        for (int x = 0; x < XI; ++x)
            xraw[st][x] = load16(xld[x] + k);
#pragma unroll
        for (int mt = 0; mt < TM; ++mt)
            sa[st][mt] = p.a_scale[sa_base[mt] + kb];
    };
    auto compute = [&](int st, int i) {
        moe_u32x4 *xb = s_x[i & 1];
#pragma unroll
        for (int x = 0; x < XI; ++x)
            xb[xslot[x]] = xraw[st][x];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            tbuf[nt * 128 + wslot0] = wraw[st][nt][0];
            tbuf[nt * 128 + wslot1] = wraw[st][nt][1];
        }
        __syncthreads();  // activation tile complete; also orders this wave's transpose buffer
        moe_i32x8 a[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
            a[nt] = join(tbuf[nt * 128 + rslot0], tbuf[nt * 128 + rslot1]);
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
            const int r = mt * 16 + rr;
            const int sw = (r >> 1) & 7;
            const moe_i32x8 bx = join(xb[r * 8 + (rq ^ sw)], xb[r * 8 + ((rq + 4) ^ sw)]);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const moe_f32x4 part = mfma_fp8_block(a[nt], bx);
                const float s = sa[st][mt] * sb[st][nt];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[mt][nt][q] = fmaf(part[q], s, acc[mt][nt][q]);
            }
        }
        moe_wave_sync();  // this wave's transpose reads finish before its next writes
    };

    // Software pipeline, STAGES-1 k-steps in flight; branch-free steady state (the prefetch past
    // the end wraps to an early k-step: in bounds, never consumed).
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        load(st, st);
    int i = 0;
    for (; i + STAGES <= KB; i += STAGES) {
#pragma unroll
        for (int st = 0; st < STAGES; ++st) {
            load((st + STAGES - 1) % STAGES, i + st + STAGES - 1);
            compute(st, i + st);
        }
    }
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (i + st < KB)
            compute(st, i + st);

    // ---- epilogue: lane holds columns 4*(lane/16)+q of row 16*mt + lane%16
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
        const int r = mt * 16 + rr;
        if (r >= n_rows)
            continue;
        uint16_t *orow = p.out + ((size_t)rbase + r) * p.N;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            if (!tile_ok[nt])
                continue;
            moe_u32x2 packed;
            packed.x = moe_pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
            packed.y = moe_pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
            *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * rq) = packed;
        }
    }
}

// ---------------------------------------------------------------- weight-streaming form
// A few rows per expert (decode): a workgroup owns one expert and NT 16-column tiles of the
// output; its KSPLIT waves split the K loop and are summed through LDS in a fixed order, and the
// expert's rows go through in 16-row passes (one pass at decode).  An e4m3 k-step of a weight
// row is one 128-byte line; lane l loads bytes [16q, 16q + 16) and [64 + 16q, 80 + 16q) of row
// l%16 (q = l/16), the two chunks join() pairs, straight into the MFMA A operand -- no LDS
// transpose -- with non-temporal loads STAGES-1 k-steps ahead, and its activation row likewise
// into B; a wave's two load instructions cover the tile's 16 whole lines.  Scales and
// accumulation as k_fp8_gemm.
// SEG = 2 (weight rows a multiple of 2 KB apart): a load instruction reads 4 rows x 256 bytes
// (two k-steps) instead, the layout that streams fastest on such strides, and a per-wave
// XOR-swizzled LDS transpose (16 rows x 16 chunks) hands the same A operand to the MFMA;
// STAGES then counts two-k-step segments.  Every wave's K range must hold whole segments.
template <int NT, int KSPLIT, int STAGES, int SEG = 1>
__global__ __launch_bounds__(64 * KSPLIT)
void k_fp8_ws(Fp8Problem p)
{
    static_assert(SEG == 1 || SEG == 2, "one- or two-k-step segments");
    __shared__ moe_f32x4 s_red[(KSPLIT > 1 ? KSPLIT - 1 : 1) * NT * 64];
    __shared__ moe_u32x4 s_t[SEG > 1 ? KSPLIT * NT * 256 : 1];
    const int lane = threadIdx.x & 63;
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int expert = blockIdx.y;
    const int col0 = blockIdx.x * (16 * NT);
    int r0, r1;
    if (p.offsets != nullptr) {
        contig_rows(p, expert, r0, r1);
    } else {
        r0 = expert * p.max_m;
        r1 = r0 + min(max(p.masked_m[expert], 0), p.max_m);
    }
    const int n_rows = r1 - r0;
    if (n_rows <= 0)
        return;
    const int K = p.K, KB = p.KB;
    const int rr = lane & 15, rq = lane >> 4;

    const uint8_t *B = p.b + (size_t)expert * p.N * K;
    const uint8_t *wrow[NT];
    bool tile_ok[NT];
    int sb_base[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < p.N;
        const int cc = tile_ok[nt] ? c : 0;
        wrow[nt] = SEG == 1 ? B + (size_t)(cc + rr) * K + 16 * rq
                            : B + (size_t)(cc + (lane >> 4)) * K + 16 * (lane & 15);
        sb_base[nt] = (expert * p.NB + cc / 128) * KB;
    }
    // K blocks of this wave (nseg segments of SEG blocks), visited from a rotated start
    const int per = (KB + KSPLIT - 1) / KSPLIT;
    const int kb0 = kw * per;
    const int nk = max(0, min(KB, kb0 + per) - kb0);
    const int nseg = nk / SEG;
    const int rot =
        nseg > 0 ? (int)((blockIdx.x * 7u + blockIdx.y * 13u) % (unsigned)nseg) : 0;
    // SEG = 2 transpose buffer of this wave: row r keeps 16-byte chunk c in slot c ^ r; a lane
    // of instruction j writes chunk lane%16 of row 4j + lane/16, and reads chunks 8h + rq and
    // 8h + 4 + rq (bytes 16rq and 64 + 16rq of k-step h) of row rr
    moe_u32x4 *tb = s_t + (SEG > 1 ? kw * NT * 256 : 0);
    int wslot[2 * SEG], rslot[SEG][2];
#pragma unroll
    for (int j = 0; j < 2 * SEG; ++j) {
        const int r = 4 * j + (lane >> 4);
        wslot[j] = r * 16 + ((lane & 15) ^ r);
    }
#pragma unroll
    for (int h = 0; h < SEG; ++h) {
        rslot[h][0] = rr * 16 + ((8 * h + rq) ^ rr);
        rslot[h][1] = rr * 16 + ((8 * h + 4 + rq) ^ rr);
    }

    for (int pass0 = 0; pass0 < n_rows; pass0 += 16) {
        // B operand column lane%16: row pass0 + lane%16 of the expert's rows (past its rows:
        // its first row, whose results are never stored)
        const int r = pass0 + rr;
        const bool rok = r < n_rows;
        const size_t arow_i = fp8_arow(p, r0 + (rok ? r : 0));
        const uint8_t *arow = p.a + arow_i * K + 16 * rq;
        const float *asc = p.a_scale + arow_i * KB;

        moe_f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc[nt] = moe_f32x4{0.f, 0.f, 0.f, 0.f};
        // Every load is issued on every path, the same number per segment: past the wave's K
        // range they read one cached line at the start of the weights' scales (all lanes
        // alike), past the last column the clamped row 0.  With loads under branches the
        // compiler cannot count the outstanding ones and waits for all of them before each
        // segment's compute, which drains the prefetch.
        const uint8_t *const dummy = reinterpret_cast<const uint8_t *>(p.b_scale);
        const int nseg1 = max(nseg, 1);
        moe_u32x4 w[STAGES][NT][2 * SEG], x[STAGES][SEG][2];
        float sa[STAGES][SEG], sb[STAGES][SEG][NT];
        auto load = [&](int st, int i) {
            const bool on = i < nseg;
            const int kb = kb0 + ((i + rot) % nseg1) * SEG;  // first K block of segment i
            const int k = kb * 128;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (SEG == 1) {
                    w[st][nt][0] = load_nt16(on ? wrow[nt] + k : dummy);
                    w[st][nt][1] = load_nt16(on ? wrow[nt] + k + 64 : dummy);
                } else {
#pragma unroll
                    for (int j = 0; j < 2 * SEG; ++j)
                        w[st][nt][j] = load_nt16(on ? wrow[nt] + (size_t)(4 * j) * K + k : dummy);
                }
#pragma unroll
                for (int h = 0; h < SEG; ++h)
                    sb[st][h][nt] = on ? p.b_scale[sb_base[nt] + kb + h]
                                       : *reinterpret_cast<const float *>(dummy);
            }
#pragma unroll
            for (int h = 0; h < SEG; ++h) {
                x[st][h][0] = load16(on ? arow + k + 128 * h : dummy);
                x[st][h][1] = load16(on ? arow + k + 128 * h + 64 : dummy);
                sa[st][h] = on ? asc[kb + h] : *reinterpret_cast<const float *>(dummy);
            }
        };
        auto compute = [&](int st) {
            if (SEG > 1) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    if (tile_ok[nt])
#pragma unroll
                        for (int j = 0; j < 2 * SEG; ++j)
                            tb[nt * 256 + wslot[j]] = w[st][nt][j];
                moe_wave_sync();
            }
#pragma unroll
            for (int h = 0; h < SEG; ++h) {
                const moe_i32x8 bx = join(x[st][h][0], x[st][h][1]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if (!tile_ok[nt])
                        continue;
                    const moe_i32x8 a = SEG == 1 ? join(w[st][nt][0], w[st][nt][1])
                                                 : join(tb[nt * 256 + rslot[h][0]],
                                                        tb[nt * 256 + rslot[h][1]]);
                    const moe_f32x4 part = mfma_fp8_block(a, bx);
                    const float s = sa[st][h] * sb[st][h][nt];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[nt][q] = fmaf(part[q], s, acc[nt][q]);
                }
            }
            if (SEG > 1)
                moe_wave_sync();  // this wave's transpose reads finish before its next writes
        };
        // software pipeline: STAGES-1 segments in flight
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            load(st, st);
        for (int i = 0; i < nseg; i += STAGES) {
#pragma unroll
            for (int st = 0; st < STAGES; ++st) {
                const int cur = i + st;
                load((st + STAGES - 1) % STAGES, cur + STAGES - 1);
                __builtin_amdgcn_sched_barrier(0);
                if (cur < nseg)
                    compute(st);
            }
        }

        // ---- fixed-order sum over the K-split waves
        if (KSPLIT > 1) {
            __syncthreads();
            if (kw > 0) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    s_red[((kw - 1) * NT + nt) * 64 + lane] = acc[nt];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int v = 0; v < KSPLIT - 1; ++v)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[nt] += s_red[(v * NT + nt) * 64 + lane];
            }
        }

        // ---- epilogue (wave 0): lane holds columns 4*(lane/16)+q of row pass0 + lane%16
        if (kw == 0 && rok) {
            uint16_t *orow = p.out + ((size_t)r0 + r) * p.N;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (!tile_ok[nt])
                    continue;
                moe_u32x2 packed;
                packed.x = moe_pack_bf16x2(acc[nt][0], acc[nt][1]);
                packed.y = moe_pack_bf16x2(acc[nt][2], acc[nt][3]);
                *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * rq) = packed;
            }
        }
        if (KSPLIT > 1)
            __syncthreads();  // the next pass reuses s_red
    }
}

// ---------------------------------------------------------------- 256 x 256 tile form

// Grid of a launch: tiles rounded up to a multiple of 8.
__host__ __device__ inline int fp8_wide_grid(int tiles)
{
    return (tiles + kXcds - 1) / kXcds * kXcds;
}

// NT: 16-row weight tiles per wave (8: 256 output columns per workgroup, 4: 128 -- twice the
// workgroups, for launches that would not fill the GPU).
template <int NT>
__global__ __launch_bounds__(moe_wide::kThreads) void k_fp8_wide(Fp8Problem p, int n_blocks,
                                                                  int m_tiles)
{
    // moe_wide's tile constants (this namespace's kWaves is the 4-wave kernel's)
    using moe_wide::kBM;
    using moe_wide::kMT;
    using moe_wide::kWM;
    using moe_wide::kWN;
    using moe_wide::kXcds;
    using moe_wide::kThreads;
    using moe_wide::Stage;
    using moe_wide::dma16;
    using moe_wide::step_barrier;
    using St = Stage<64>;                 // 128-byte rows: 128 e4m3 codes (slot order)
    constexpr int BW = 32 * NT;           // output columns (weight rows) per workgroup
    constexpr int WLoads = BW / 64;       // weight DMA instructions per wave
    constexpr int kG = 4;               // k-steps per group of staged activation scales
    // A stage holds one k-step: the tile's activation rows, then its BW weight rows.  Tiles of
    // more than kSmallRows rows take two stages of 256 activation rows (the next k-step loads
    // while this one computes); smaller ones take three stages of kSmallRows activation rows in
    // the same memory, so their weight stream runs two k-steps ahead -- such tiles have few
    // MFMAs to hide a k-step's load latency behind.
    constexpr int kSmallRows = 128;
    constexpr int kW = BW * 128;
    constexpr int kFullStage = kBM * 128 + kW;
    constexpr int kSmallStage = kSmallRows * 128 + kW;
    constexpr int kSmem = 2 * kFullStage > 3 * kSmallStage ? 2 * kFullStage : 3 * kSmallStage;
    __shared__ moe_u32x4 smem[kSmem / 16];
    __shared__ float s_scale[2][kBM * kG];  // a_scale of the tile rows, two groups

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / kWN, wn = wv % kWN;

    // ---- tile: expert-major, column blocks, row tiles innermost; XCD-contiguous ranges
    Fp8Tile tile;
    if (!fp8_locate<kBM, true>(p, n_blocks, m_tiles, tile))
        return;
    const int expert = tile.expert, nblk = tile.nblk, rbase = tile.rbase;
    const int n_real = __builtin_amdgcn_readfirstlane(tile.n_rows);
    const int K = p.K, KB = p.KB;
    const int col_wg = nblk * BW;

    // ---- DMA sources (see moe_wide_kernel.h): instruction j of this wave covers tile rows
    // wv*32 + 8j .. +7, lane l fetching chunk (l%8) ^ swizzle(row) of row wv*32 + 8j + l/8
    const int lrow = lane >> 3, lpos = lane & 7;
    const uint8_t *B = p.b + (size_t)expert * p.N * K;
    const uint8_t *wsrc[WLoads];
#pragma unroll
    for (int j = 0; j < WLoads; ++j) {
        const int r = wv * (BW / moe_wide::kWaves) + 8 * j + lrow;
        const int c = col_wg + r;
        wsrc[j] = B + (size_t)(c < p.N ? c : 0) * K + 16 * (lpos ^ ((r >> 1) & 7));
    }
    const uint8_t *xsrc[St::kXLoads];
    bool xload[St::kXLoads];
#pragma unroll
    for (int j = 0; j < St::kXLoads; ++j) {
        const int rfirst = wv * (kBM / moe_wide::kWaves) + 8 * j;
        const int r = rfirst + lrow;
        xload[j] = rfirst < n_real;
        xsrc[j] = p.a + fp8_arow(p, rbase + (r < n_real ? r : 0)) * K +
                  16 * (lpos ^ ((r >> 1) & 7));
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    // (rows past kSmallRows have no loads in the three-stage form, so the offsets hold for both)
    const uint32_t x_dst = lds0 + wv * (kBM / moe_wide::kWaves) * 128;
    int nx = 0;  // this wave's activation DMAs per k-step
#pragma unroll
    for (int j = 0; j < St::kXLoads; ++j)
        nx += xload[j] ? 1 : 0;

    const int rr = lane & 15, rq = lane >> 4;
    int mt_real = 0;
#pragma unroll
    for (int i = 0; i < kMT; ++i)
        mt_real += (16 * (wm + kWM * i) < n_real) ? 1 : 0;
    // scales: a_scale of the tile's rows is staged in LDS kG k-steps at a time -- waves 0..3
    // each copy 64 rows x kG consecutive blocks (16 bytes a row, one load instruction; rows past
    // the rows in use copy row 0) -- instead of one strided load per row per k-step.  b_scale:
    // the block of this wave's 128 columns, one uniform load per k-step.
    const float *sa_src =
        p.a_scale +
        fp8_arow(p, rbase + (64 * (wv & 3) + lane < n_real ? 64 * (wv & 3) + lane : 0)) * KB;
    const uint32_t sa_dst = (uint32_t)(uintptr_t)&s_scale[0][0] + (wv & 3) * 64 * 16;
    const int wcol = col_wg + 16 * NT * wn;  // this wave's columns: one 128-column block
    const int sb_base = (expert * p.NB + (wcol < p.N ? wcol : 0) / 128) * KB;
    // b_scale of that block, lane l holding k-blocks l and l + 64 (KB <= 128), loaded once per
    // tile and picked per k-step by a lane read: the K loop then holds no vector-memory load
    // the compiler knows of, since it cannot see the DMAs and would wait for every outstanding
    // load, the next k-step's DMAs included, before such a load's first use.  The empty asm
    // takes the values before the first DMA, so their wait comes before it.
    const float sb_lo = lane < KB ? p.b_scale[sb_base + lane] : 0.f;
    const float sb_hi = lane + 64 < KB ? p.b_scale[sb_base + lane + 64] : 0.f;
    asm volatile("" ::"v"(sb_lo), "v"(sb_hi));
    // the K loop starts at a multiple of kG blocks (KB % kG == 0), so groups stay aligned
    const int rot = (int)((expert * 7u) % (unsigned)(KB / kG)) * kG;

    moe_f32x4 acc[kMT][NT];
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n)
            acc[m][n] = moe_f32x4{0.f, 0.f, 0.f, 0.f};

    // k-step i's DMAs into the stage at byte offset so (weights at wd + so); a new group of kG
    // k-steps also brings a_scale[rows][kb .. kb + kG) into its half of s_scale
    auto issue = [&](uint32_t so, uint32_t wd, int i) {
        const int kb = (i + rot) % KB;
        const int k = kb * 128;
#pragma unroll
        for (int j = 0; j < St::kXLoads; ++j)
            if (xload[j])
                dma16(xsrc[j] + k, x_dst + so + j * 1024);
#pragma unroll
        for (int j = 0; j < WLoads; ++j)
            dma16(wsrc[j] + k, wd + so + j * 1024);
        if (i % kG == 0 && wv < 4)
            dma16(sa_src + kb, sa_dst + ((i / kG) & 1) * (kBM * kG * 4));
    };
    // this wave's DMAs of k-step i (0 past the K loop)
    auto n_loads = [&](int i) {
        return i < KB ? nx + WLoads + ((i % kG == 0 && wv < 4) ? 1 : 0) : 0;
    };

    // S stages, the loads S - 1 k-steps ahead.  At the top of step i this wave's outstanding
    // loads are those of k-steps i .. i+S-2 (oldest first); waiting until only the later ones
    // are left puts its part of k-step i in LDS, and the barrier publishes every wave's part
    // and shows that every wave has finished step i-1, whose stage k-step i+S-1 then reuses.
    // a_scale group g is loaded with k-step g*kG, S - 1 <= 2 steps before its first use, into
    // the half that group g-2 used, whose last step (g-1)*kG - 1 is then finished.
    // Instantiated per count of real 16-row tiles (MTR) and stage form.
    auto k_loop = [&](auto mtr, auto small) {
        constexpr int MTR = decltype(mtr)::value;
        constexpr bool SMALL = decltype(small)::value;
        constexpr int S = SMALL ? 3 : 2;
        constexpr int kSt = SMALL ? kSmallStage : kFullStage;
        constexpr int kX = kSt - kW;
        const uint32_t wd = lds0 + kX + wv * (BW / moe_wide::kWaves) * 128;
#pragma unroll
        for (int i = 0; i < S - 1; ++i)
            if (i < KB)
                issue(i * kSt, wd, i);
        for (int i = 0; i < KB; ++i) {
            int later = 0;
#pragma unroll
            for (int j = 1; j < S - 1; ++j)
                later += n_loads(i + j);
            step_barrier(later);
            if (i + S - 1 < KB)
                issue(((i + S - 1) % S) * kSt, wd, i + S - 1);
            if (MTR == 0)
                continue;
            const moe_u32x4 *xb = smem + (i % S) * (kSt / 16);
            const moe_u32x4 *wb = xb + kX / 16;
            moe_i32x8 bx[MTR > 0 ? MTR : 1];
            float s[MTR > 0 ? MTR : 1];
            const float *sa = s_scale[(i / kG) & 1];
            const int kb = (i + rot) % KB;
            const float sbv = __int_as_float(
                kb < 64 ? __builtin_amdgcn_readlane(__float_as_int(sb_lo), kb)
                        : __builtin_amdgcn_readlane(__float_as_int(sb_hi), kb - 64));
#pragma unroll
            for (int m = 0; m < MTR; ++m) {
                const int r = 16 * (wm + kWM * m) + rr;
                bx[m] = join(xb[St::slot(r, rq)], xb[St::slot(r, rq + 4)]);
                s[m] = sa[r * kG + i % kG] * sbv;
            }
            // The block sums of weight tile n are scaled into the accumulators while the MFMAs
            // of tile n+1 run (two sets of partials), so no FMA waits on the MFMA just issued.
            moe_f32x4 part[2][MTR > 0 ? MTR : 1];
#pragma unroll
            for (int n = 0; n <= NT; ++n) {
                if (n < NT) {
                    const int r = 16 * NT * wn + 16 * n + rr;
                    const moe_i32x8 aw = join(wb[St::slot(r, rq)], wb[St::slot(r, rq + 4)]);
#pragma unroll
                    for (int m = 0; m < MTR; ++m)
                        part[n & 1][m] = mfma_fp8_block(aw, bx[m]);
                }
                if (n > 0) {
#pragma unroll
                    for (int m = 0; m < MTR; ++m)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[m][n - 1][q] =
                                fmaf(part[(n - 1) & 1][m][q], s[m], acc[m][n - 1][q]);
                }
            }
        }
    };
    // more than kSmallRows rows give every wave 2 to 4 real 16-row tiles, fewer 0 to 2
    using Full = std::false_type;
    using Small = std::true_type;
    if (n_real <= kSmallRows) {
        switch (mt_real) {
        case 0: k_loop(std::integral_constant<int, 0>(), Small()); break;
        case 1: k_loop(std::integral_constant<int, 1>(), Small()); break;
        default: k_loop(std::integral_constant<int, 2>(), Small()); break;
        }
    } else {
        switch (mt_real) {
        case 2: k_loop(std::integral_constant<int, 2>(), Full()); break;
        case 3: k_loop(std::integral_constant<int, 3>(), Full()); break;
        default: k_loop(std::integral_constant<int, 4>(), Full()); break;
        }
    }

    // ---- epilogue: lane holds columns 4*(lane/16)+q of row 16*(wm + 4m) + lane%16
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
        const int r = 16 * (wm + kWM * m) + rr;
        if (m >= mt_real || r >= n_real)
            continue;
        uint16_t *orow = p.out + ((size_t)rbase + r) * p.N;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int col = wcol + 16 * n + 4 * rq;
            if (col >= p.N)
                continue;
            moe_u32x2 packed;
            packed.x = moe_pack_bf16x2(acc[m][n][0], acc[m][n][1]);
            packed.y = moe_pack_bf16x2(acc[m][n][2], acc[m][n][3]);
            *reinterpret_cast<moe_u32x2 *>(orow + col) = packed;
        }
    }
}

// ---------------------------------------------------------------- direct form (a few tokens)
// The FP8 pass for T * k <= 64 routes without the align and quantiser launches (aiter MI308
// decoding PR, "Changes": direct decoding from topk_ids): one workgroup per (column block,
// route); the first route of an expert gathers every route of that expert (the others leave),
// so an expert's weights are streamed once.  The workgroup quantises its rows itself, per
// 1 x 128 group exactly as k_quant_fp8 does (16 lanes per group, s = amax / 448, the same
// encoder), into an LDS copy of the rows (RL per pass, row r's 16-byte chunk c at position
// c ^ r, so the B-operand reads of several rows at one chunk hit distinct banks) with their
// scales.  RL (1..16) is the most rows an expert can hold in one pass: min(16, T) when every
// token's experts are distinct, so at decode sizes the LDS copy is a few rows and several
// workgroups share a CU; an expert with more rows takes more passes.  The MFMA's B columns
// past RL read row 0, and their results are never stored.
// Weights, block scaling and the K split are k_fp8_ws's.
//   gate-up: rows are x[route / k]; the workgroup's NT gate tiles and the NT up tiles of the
//     same columns; out h[route] = bf16(SiLU(g) * u) with g and u first rounded to bf16 (the
//     values the two-kernel form stores and its quantiser reads);
//   down: rows are h[route]; out y[route] = bf16(sum).
struct Fp8Direct {
    const uint16_t *act;      // gate-up: x [T, K]; down: h [P, K] bf16
    const int32_t *topk_ids;  // [P]
    const uint8_t *b;         // [E, rows_b, K] e4m3
    const float *b_scale;     // [E, rows_b / 128, KB]
    uint16_t *out;            // [P, n_out] bf16
    int P, top_k, E, n_out, K, KB, NB;  // NB = rows_b / 128 (rows_b = 2 n_out for gate-up)
    int RL;                             // rows per pass, 1..16
};

// LDS bytes of the direct form: RL rows of K codes, their scales, the K-split partial sums
// and (SEG 2) the per-wave transpose buffers.
__host__ __device__ inline size_t fp8_direct_lds(int K, int NW, int KSPLIT, int SEG, int RL)
{
    return (size_t)RL * K + (size_t)RL * (K / 128) * 4 +
           (size_t)(KSPLIT > 1 ? KSPLIT - 1 : 1) * NW * 64 * 16 +
           (SEG > 1 ? (size_t)KSPLIT * NW * 256 * 16 : 0);
}

template <bool GATE_UP, int NT, int KSPLIT, int STAGES, int SEG>
__global__ __launch_bounds__(64 * KSPLIT) void k_fp8_direct(Fp8Direct d)
{
    static_assert(SEG == 1 || SEG == 2, "one- or two-k-step segments");
    constexpr int NW = GATE_UP ? 2 * NT : NT;  // 16-row weight tiles per k-step
    extern __shared__ moe_u32x4 s_dyn[];
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    const int kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col0 = blockIdx.x * (16 * NT);
    const int route0 = blockIdx.y;
    const int K = d.K, KB = d.KB;

    // ---- the expert of this route, and all routes of it (P <= 64: one id per lane)
    const int e = d.topk_ids[route0];
    if (e < 0 || e >= d.E)
        return;
    const int mine = lane < d.P ? d.topk_ids[lane] : -1;
    const uint64_t members = __ballot(mine == e);
    if (members & ((1ull << route0) - 1))
        return;  // an earlier route of this expert owns it
    const int n_rows = __popcll(members);

    // ---- LDS: codes [RL][K], scales [RL][KB], K-split sums, transpose buffers
    const int RL = d.RL;
    uint8_t *s_codes = reinterpret_cast<uint8_t *>(s_dyn);
    float *s_scale = reinterpret_cast<float *>(s_codes + (size_t)RL * K);
    moe_f32x4 *s_red = reinterpret_cast<moe_f32x4 *>(s_scale + RL * KB);
    moe_u32x4 *s_t = reinterpret_cast<moe_u32x4 *>(s_red + (KSPLIT > 1 ? KSPLIT - 1 : 1) * NW * 64);

    const int rr = lane & 15, rq = lane >> 4;
    const uint8_t *B = d.b + (size_t)e * (GATE_UP ? 2 * d.n_out : d.n_out) * K;
    const uint8_t *wrow[NW];
    int sb_base[NW];
    bool tile_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + 16 * nt;
        tile_ok[nt] = c < d.n_out;
        const int cc = tile_ok[nt] ? c : 0;
#pragma unroll
        for (int half = 0; half < (GATE_UP ? 2 : 1); ++half) {
            const int row = cc + half * d.n_out;  // gate rows, then the up rows of the same columns
            const int w = nt + half * NT;
            wrow[w] = SEG == 1 ? B + (size_t)(row + rr) * K + 16 * rq
                               : B + (size_t)(row + (lane >> 4)) * K + 16 * (lane & 15);
            sb_base[w] = (e * d.NB + row / 128) * KB;
        }
    }
    // K blocks of this wave (nseg segments of SEG blocks), visited from a rotated start
    const int per = (KB + KSPLIT - 1) / KSPLIT;
    const int kb0 = kw * per;
    const int nk = max(0, min(KB, kb0 + per) - kb0);
    const int nseg = nk / SEG;
    const int rot =
        nseg > 0 ? (int)((blockIdx.x * 7u + blockIdx.y * 13u) % (unsigned)nseg) : 0;
    moe_u32x4 *tb = s_t + (SEG > 1 ? kw * NW * 256 : 0);
    int wslot[2 * SEG], rslot[SEG][2];
#pragma unroll
    for (int j = 0; j < 2 * SEG; ++j) {
        const int r = 4 * j + (lane >> 4);
        wslot[j] = r * 16 + ((lane & 15) ^ r);
    }
#pragma unroll
    for (int h = 0; h < SEG; ++h) {
        rslot[h][0] = rr * 16 + ((8 * h + rq) ^ rr);
        rslot[h][1] = rr * 16 + ((8 * h + 4 + rq) ^ rr);
    }
    const int rl = rr < RL ? rr : 0;  // this lane's B column reads LDS row rl
    const moe_u32x4 *xrow = reinterpret_cast<const moe_u32x4 *>(s_codes + (size_t)rl * K);

    moe_f32x4 acc[NW];
    moe_u32x4 wv[STAGES][NW][2 * SEG];
    float sb[STAGES][SEG][NW];
    // Every load is issued on every path, the same number per segment (past the wave's K range:
    // one cached line at the start of the weight scales; past the last column: the clamped row
    // 0), so the compiler counts the outstanding loads exactly instead of waiting for all of
    // them before each segment's compute.
    const uint8_t *const dummy = reinterpret_cast<const uint8_t *>(d.b_scale);
    const int nseg1 = max(nseg, 1);
    auto load = [&](int st, int i) {
        const bool on = i < nseg;
        const int kb = kb0 + ((i + rot) % nseg1) * SEG;  // first K block of segment i
        const int k = kb * 128;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if (SEG == 1) {
                wv[st][w][0] = load_nt16(on ? wrow[w] + k : dummy);
                wv[st][w][1] = load_nt16(on ? wrow[w] + k + 64 : dummy);
            } else {
#pragma unroll
                for (int j = 0; j < 2 * SEG; ++j)
                    wv[st][w][j] = load_nt16(on ? wrow[w] + (size_t)(4 * j) * K + k : dummy);
            }
#pragma unroll
            for (int h = 0; h < SEG; ++h)
                sb[st][h][w] = on ? d.b_scale[sb_base[w] + kb + h]
                                  : *reinterpret_cast<const float *>(dummy);
        }
    };
    auto compute = [&](int st, int i) {
        const int kb = kb0 + ((i + rot) % nseg1) * SEG;
        if (SEG > 1) {
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if (tile_ok[w % NT])
#pragma unroll
                    for (int j = 0; j < 2 * SEG; ++j)
                        tb[w * 256 + wslot[j]] = wv[st][w][j];
            moe_wave_sync();
        }
#pragma unroll
        for (int h = 0; h < SEG; ++h) {
            // bytes 16rq and 64 + 16rq of k-step kb + h of row rr: chunks 8(kb+h) + rq, + 4
            const int c0 = 8 * (kb + h) + rq;
            const moe_i32x8 bx = join(xrow[c0 ^ rl], xrow[(c0 + 4) ^ rl]);
            const float sa = s_scale[rl * KB + kb + h];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                if (!tile_ok[w % NT])
                    continue;
                const moe_i32x8 a = SEG == 1 ? join(wv[st][w][0], wv[st][w][1])
                                             : join(tb[w * 256 + rslot[h][0]],
                                                    tb[w * 256 + rslot[h][1]]);
                const moe_f32x4 part = mfma_fp8_block(a, bx);
                const float sscale = sa * sb[st][h][w];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[w][q] = fmaf(part[q], sscale, acc[w][q]);
            }
        }
        if (SEG > 1)
            moe_wave_sync();  // this wave's transpose reads finish before its next writes
    };
    // the first segments of the weight stream go out before the rows are quantised: they do
    // not depend on them
    auto prologue = [&] {
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            load(st, st);
    };
    prologue();

    for (int pass0 = 0; pass0 < n_rows; pass0 += RL) {
        // ---- quantise the pass's real rows: 16 lanes per (row, 1 x 128 group).  Rows past
        // n_rows keep whatever LDS holds: an output element reads only its own row's codes and
        // scale, and those rows are never written out.
        const int nr = min(RL, n_rows - pass0);
        for (int gi = tid / 16; gi < nr * KB; gi += 4 * KSPLIT) {
            const int r = gi / KB, g = gi % KB, sub = tid & 15;
            const int route = moe_ws::nth_set_bit(members, pass0 + r);
            const int src = GATE_UP ? route / d.top_k : route;
            float v[8];
            const moe_u32x4 raw = *reinterpret_cast<const moe_u32x4 *>(
                d.act + (size_t)src * K + 128 * g + 8 * sub);
            const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w4[i] << 16);
                v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
            for (int dd = 1; dd < 16; dd <<= 1)
                amax = fmaxf(amax, __shfl_xor(amax, dd, 16));
            const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
            if (sub == 0)
                s_scale[r * KB + g] = sc;
            const uint32_t lo = moe::e4m3_pack4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
            const uint32_t hi = moe::e4m3_pack4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
            const int chunk = 8 * g + (sub >> 1);  // this lane's 8 codes: half (sub & 1) of it
            moe_u32x2 packed;
            packed.x = lo;
            packed.y = hi;
            *reinterpret_cast<moe_u32x2 *>(s_codes + (size_t)r * K + 16 * (chunk ^ r) +
                                           8 * (sub & 1)) = packed;
        }
        __syncthreads();  // the pass's codes and scales are in LDS

#pragma unroll
        for (int w = 0; w < NW; ++w)
            acc[w] = moe_f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < nseg; i += STAGES) {
#pragma unroll
            for (int st = 0; st < STAGES; ++st) {
                const int cur = i + st;
                load((st + STAGES - 1) % STAGES, cur + STAGES - 1);
                __builtin_amdgcn_sched_barrier(0);
                if (cur < nseg)
                    compute(st, cur);
            }
        }

        // ---- fixed-order sum over the K-split waves
        if (KSPLIT > 1) {
            __syncthreads();
            if (kw > 0) {
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    s_red[((kw - 1) * NW + w) * 64 + lane] = acc[w];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int v = 0; v < KSPLIT - 1; ++v)
#pragma unroll
                    for (int w = 0; w < NW; ++w)
                        acc[w] += s_red[(v * NW + w) * 64 + lane];
            }
        }

        // ---- epilogue (wave 0): lane holds columns 4*(lane/16)+q of row pass0 + lane%16
        const int s = pass0 + rr;
        if (kw == 0 && rr < RL && s < n_rows) {
            const int route = moe_ws::nth_set_bit(members, s);
            uint16_t *orow = d.out + (size_t)route * d.n_out;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (!tile_ok[nt])
                    continue;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (GATE_UP) {
                        const float g = moe_bf16_to_f32(moe_f32_to_bf16(acc[nt][q]));
                        const float u = moe_bf16_to_f32(moe_f32_to_bf16(acc[NT + nt][q]));
                        v[q] = g / (1.0f + __expf(-g)) * u;
                    } else {
                        v[q] = acc[nt][q];
                    }
                }
                moe_u32x2 packed;
                packed.x = moe_pack_bf16x2(v[0], v[1]);
                packed.y = moe_pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<moe_u32x2 *>(orow + col0 + 16 * nt + 4 * rq) = packed;
            }
        }
        if (pass0 + RL < n_rows)
            prologue();   // the next pass's weight stream
        __syncthreads();  // the next pass overwrites the codes, scales and sums
    }
}

}  // namespace moe_fp8
