// moe_gemm_fp8.hip -- launches of the block-scaled FP8 grouped GEMM (moe_fp8_kernel.h): the
// weight-streaming form for a few rows per expert (decode), the 64-row form for blocks of up to
// 64 rows, else the 256-row tile form (256 or, when that gives
// fewer than two workgroups per CU, 128 columns per workgroup); the 64-row form also when K is
// not a multiple of 512 or a_scale is not 16-byte aligned.  Tile shapes measured on MI355X on
// the page's decode shapes.
#include <algorithm>

#include "moe_fp8_kernel.h"
#include "moe_internal.h"

namespace {

// Tiles of a launch: masked layout, E * m_tiles per column block; contiguous layout, at most
// ceil(P / BM) + E per column block (the kernel counts the real ones itself).
int tile_bound(const moe_fp8::Fp8Problem &p, int BM, int n_blocks, int m_tiles)
{
    if (p.offsets == nullptr)
        return p.E * n_blocks * m_tiles;
    return ((p.P + BM - 1) / BM + p.E) * n_blocks;
}

template <int BM, int NTW, int STAGES>
void launch_one(const moe_fp8::Fp8Problem &p, hipStream_t stream)
{
    const int n_blocks = (p.N + 64 * NTW - 1) / (64 * NTW);
    const int m_tiles = (p.max_m + BM - 1) / BM;
    const int tiles = tile_bound(p, BM, n_blocks, m_tiles);
    hipLaunchKernelGGL((moe_fp8::k_fp8_gemm<BM, NTW, STAGES>), dim3(moe_fp8::fp8_grid(tiles)),
                       dim3(64 * moe_fp8::kWaves), 0, stream, p, n_blocks, m_tiles);
}

template <int NT>
void launch_fp8_wide(const moe_fp8::Fp8Problem &p, int m_tiles, hipStream_t stream)
{
    const int n_blocks = (p.N + 32 * NT - 1) / (32 * NT);
    hipLaunchKernelGGL(moe_fp8::k_fp8_wide<NT>,
                       dim3(moe_fp8::fp8_wide_grid(tile_bound(p, moe_wide::kBM, n_blocks, m_tiles))),
                       dim3(moe_wide::kThreads), 0, stream, p, n_blocks, m_tiles);
}

// The weight-streaming form: one workgroup per (32 output columns, expert); K split over four
// waves (two when K has fewer than 16 blocks).
void launch_fp8_ws(const moe_fp8::Fp8Problem &p, hipStream_t stream)
{
    const dim3 grid((p.N + 31) / 32, p.E);
    // weight rows a multiple of 2 KB apart: 4 rows x 256 bytes per load (whole segments per wave)
    const bool seg2 = p.K % 2048 == 0 && p.KB % 8 == 0;
    if (p.KB >= 16 && seg2)
        hipLaunchKernelGGL((moe_fp8::k_fp8_ws<2, 4, 2, 2>), grid, dim3(64 * 4), 0, stream, p);
    else if (p.KB >= 16)
        hipLaunchKernelGGL((moe_fp8::k_fp8_ws<2, 4, 3>), grid, dim3(64 * 4), 0, stream, p);
    else
        hipLaunchKernelGGL((moe_fp8::k_fp8_ws<2, 2, 3>), grid, dim3(64 * 2), 0, stream, p);
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

template <bool GATE_UP, int NT, int KSPLIT, int STAGES, int SEG>
void launch_direct_one(const moe_fp8::Fp8Direct &d, hipStream_t stream)
{
    constexpr int NW = GATE_UP ? 2 * NT : NT;
    const size_t lds = moe_fp8::fp8_direct_lds(d.K, NW, KSPLIT, SEG, d.RL);
    const auto kernel = moe_fp8::k_fp8_direct<GATE_UP, NT, KSPLIT, STAGES, SEG>;
    static const bool attr = [&] {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)moe::kFp8DirectMaxLds) == hipSuccess;
    }();
    (void)attr;
    const dim3 grid((d.n_out + 16 * NT - 1) / (16 * NT), d.P);
    hipLaunchKernelGGL(kernel, grid, dim3(64 * KSPLIT), lds, stream, d);
}

}  // namespace

namespace moe {

// The shapes of the direct form: gate-up one gate and one up tile per workgroup, K split over
// four waves; down two tiles, K split over four waves from 16 K blocks up, else two.  Rows of
// a 1 KB multiple give each of four waves an even count of K blocks: two-k-step weight
// segments (256 contiguous bytes per row and load), where their transpose buffers fit in LDS.
static bool direct_seg2(int K)
{
    return K % 1024 == 0 && moe_fp8::fp8_direct_lds(K, 2, 4, 2, 16) <= kFp8DirectMaxLds;
}

bool fp8_direct_shape_ok(int K)
{
    return K > 0 && K % 256 == 0 && fp8_direct_lds_bytes(K) <= kFp8DirectMaxLds;
}

size_t fp8_direct_lds_bytes(int K)
{
    return moe_fp8::fp8_direct_lds(K, 2, 4, direct_seg2(K) ? 2 : 1, 16);
}

void launch_fp8_direct(bool gate_up, const uint16_t *act, const int32_t *topk_ids, int P,
                       int top_k, int E, const uint8_t *b, const float *b_scale, int n_out, int K,
                       uint16_t *out, hipStream_t stream)
{
    moe_fp8::Fp8Direct d;
    d.act = act;
    d.topk_ids = topk_ids;
    d.b = b;
    d.b_scale = b_scale;
    d.out = out;
    d.P = P;
    d.top_k = top_k;
    d.E = E;
    d.n_out = n_out;
    d.K = K;
    d.KB = K / 128;
    d.NB = (gate_up ? 2 * n_out : n_out) / 128;
    d.RL = std::min(16, std::max(1, P / top_k));  // an expert's rows, when a token's are distinct
    const bool seg2 = direct_seg2(K);
    if (gate_up) {
        if (seg2)
            launch_direct_one<true, 1, 4, 2, 2>(d, stream);
        else
            launch_direct_one<true, 1, 4, 3, 1>(d, stream);
    } else {
        if (seg2)
            launch_direct_one<false, 2, 4, 2, 2>(d, stream);
        else if (d.KB >= 16)
            launch_direct_one<false, 2, 4, 3, 1>(d, stream);
        else
            launch_direct_one<false, 2, 2, 3, 1>(d, stream);
    }
}

void launch_fp8_gemm(const uint8_t *a, const float *a_scale, const uint8_t *b,
                     const float *b_scale, const int32_t *masked_m, int E, int max_m, int N,
                     int K, uint16_t *out, hipStream_t stream)
{
    moe_fp8::Fp8Problem p;
    p.a_route = nullptr;
    p.a_div = 1;
    p.a = a;
    p.a_scale = a_scale;
    p.b = b;
    p.b_scale = b_scale;
    p.masked_m = masked_m;
    p.offsets = nullptr;
    p.out = out;
    p.E = E;
    p.max_m = max_m;
    p.P = 0;
    p.N = N;
    p.K = K;
    p.KB = K / 128;
    p.NB = (N + 127) / 128;
    // Blocks of up to 16 rows (decode): the weight-streaming form.  Up to 64 rows: the 64-row
    // form (one row tile).  Taller blocks: the 256-row form, which needs 4-block scale groups
    // and 16-byte aligned activation scales.
    if (max_m <= 16) {
        launch_fp8_ws(p, stream);
        return;
    }
    if (max_m <= 64 || p.KB % 4 != 0 || p.KB > 128 || ((uintptr_t)a_scale & 15u) != 0) {
        launch_one<64, 4, 2>(p, stream);
        return;
    }
    const int m_tiles = (max_m + moe_wide::kBM - 1) / moe_wide::kBM;
    const int wide_tiles = E * m_tiles * ((N + 255) / 256);
    if (wide_tiles >= 2 * device_cus())
        launch_fp8_wide<8>(p, m_tiles, stream);
    else
        launch_fp8_wide<4>(p, m_tiles, stream);
}

void launch_fp8_gemm_contig(const uint8_t *a, const float *a_scale, const uint8_t *b,
                            const float *b_scale, const int32_t *offsets, int E, int P, int N,
                            int K, uint16_t *out, hipStream_t stream, const int32_t *a_route,
                            int a_div)
{
    moe_fp8::Fp8Problem p;
    p.a_route = a_route;
    p.a_div = a_div;
    p.a = a;
    p.a_scale = a_scale;
    p.b = b;
    p.b_scale = b_scale;
    p.masked_m = nullptr;
    p.offsets = offsets;
    p.out = out;
    p.E = E;
    p.max_m = 0;
    p.P = P;
    p.N = N;
    p.K = K;
    p.KB = K / 128;
    p.NB = (N + 127) / 128;
    // the mean rows per expert picks the tile form, as max_m does for the masked layout
    const int mean_rows = (P + E - 1) / E;
    if (mean_rows <= 8) {
        launch_fp8_ws(p, stream);
        return;
    }
    if (mean_rows <= 64 || p.KB % 4 != 0 || p.KB > 128 || ((uintptr_t)a_scale & 15u) != 0) {
        launch_one<64, 4, 2>(p, stream);
        return;
    }
    const int wide_tiles = ((P + moe_wide::kBM - 1) / moe_wide::kBM) * ((N + 255) / 256);
    if (wide_tiles >= 2 * device_cus())
        launch_fp8_wide<8>(p, 0, stream);
    else
        launch_fp8_wide<4>(p, 0, stream);
}

}  // namespace moe
