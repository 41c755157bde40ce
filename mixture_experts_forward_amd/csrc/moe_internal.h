// moe_internal.h -- host-side interfaces between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- routing
void launch_route(const float *gating, const float *bias, int T, int E, int k, int sigmoid,
                  int renormalize, int n_group, int topk_group, float rsf, int32_t *ids,
                  float *weights, hipStream_t stream);

// ---------------------------------------------------------------- align / sort
// Work schedule of a grouped GEMM over the sorted layout, written by the align step.  The
// layout's tiles (expert by expert, each expert's block_m-row tiles x the GEMM's column blocks)
// are split into kSchedParts contiguous ranges of about equal estimated cost (a row tile of r
// routed rows costs 5*block_m/4 + r: a fixed weight stream plus MFMA work per row), one range
// per XCD.  bounds[p] is the start of range p in row-tile units (a GEMM with n column blocks
// starts range p at tile round(bounds[p] * n)); bounds[0] = 0, bounds[kSchedParts] = the row
// tile count.  queue[p] counts the tiles handed out of range p and queue[kSchedParts] the
// workgroups that have finished; all of queue is zero between launches (the align step zeroes
// it, and the last workgroup of a launch that uses it zeroes it again).
constexpr int kSchedParts = 8;
struct TileSchedule {
    float bounds[kSchedParts + 1];
    int32_t queue[kSchedParts + 1];
};

// scratch: NULL (one workgroup does everything) or align_scratch_ints(P, E) ints of device
// memory (moe_plan.h) for the chunked three-launch form (used when P > 1024).  sched: NULL or
// the TileSchedule to write.  balanced: an expert's routes spread evenly over its block_m-row
// tiles (each tile's rows a prefix of it) instead of filling them in order; the chunked form
// then needs E more ints of scratch (align_scratch_ints(P, E, true)).
void launch_align_sort(const int32_t *ids, int P, int E, int block_m, int32_t *sorted_ids,
                       int32_t *offsets, int32_t *tile_expert, int32_t *inverse, int32_t *n_tiles,
                       int32_t *scratch, hipStream_t stream, TileSchedule *sched = nullptr,
                       bool balanced = false);

// ---------------------------------------------------------------- expert GEMMs
// Where a GEMM takes its rows from.
enum RowSource {
    ROWS_SORTED = 0,  // rows of one expert's padded segment of the sorted route list
    ROWS_DIRECT = 1,  // route-major, no sort: the first route of an expert gathers its routes
    ROWS_DENSE = 2,   // every token, one weight matrix (shared expert)
    ROWS_SCAN = 3,    // expert-major, no sort: the expert's routes found by scanning topk_ids
};
constexpr int kScanMaxRoutes = 512;  // ROWS_SCAN: routes scanned by one workgroup

struct GemmProblem {
    const uint16_t *act;        // activation rows [*, K] bf16
    const uint16_t *weight;     // [experts][n_weight_rows][K] bf16
    uint16_t *out;              // output rows [*, n_out] bf16
    const int32_t *sorted_ids;  // ROWS_SORTED
    const int32_t *offsets;     // ROWS_SORTED: [E+1]
    const int32_t *topk_ids;    // ROWS_DIRECT: [P]
    const int32_t *tile_expert; // row-tiled kernel, ROWS_SORTED: expert of each row tile
    int K;                      // reduction length
    int n_out;                  // output columns (F for gate-up, H for down)
    int top_k;                  // routes per token
    int num_groups;             // weight-streaming: experts (SORTED), routes (DIRECT), row
                                // blocks (DENSE); row-tiled: row tiles
    int P;                      // routes (DIRECT)
    int rows;                   // tokens (DENSE)
    int num_experts;            // E (valid expert ids are [0, E))
    int dtype;                  // element type of act, weight, out: 0 bf16, 1 f16
    const uint8_t *wq;          // MXFP4 weights: [experts][n_weight_rows][K/2] e2m1 pairs
    const uint8_t *wscale;      // MXFP4 weights: [experts][n_weight_rows][K/32] E8M0
    TileSchedule *sched;        // 256 x 256 tile kernel, ROWS_SORTED: per-XCD tile ranges and
                                // their counters (NULL: tiles dealt statically)
    float *partial;             // 256 x 256 tile kernel, ROWS_DENSE: f32 partial tiles of the
                                // K-split tiles (NULL: no split)
    size_t partial_bytes;       // bytes at partial
    int split_tiles;            // set by the launcher: tiles split along K ...
    int split_parts;            // ... into this many parts each
    int slot_eighths;           // 256 x 256 tile kernel, dense rows: the eighths of the
                                // resident workgroup slots it takes (0: all of them)
};

// f32 partial tile of the K-split 256 x 256 kernel: 256 activation rows x 256 weight rows.
constexpr size_t kWidePartialBytes = 256u * 256u * 4u;

// Tile shape of one launch.
//   weight-streaming kernel: NT 16-column tiles per workgroup (per half for gate-up), MT 16-row
//     tiles per pass, KSPLIT waves splitting the K loop;
//   row-tiled kernel: NT 16-column tiles per wave (4 waves), 16*MT rows per tile (ksplit unused);
//   both: STAGES register buffers (STAGES-1 k-steps of 64 in flight per wave).
struct WsTile {
    int nt, mt, ksplit, stages;
};

// false: no kernel is instantiated for this tile shape (nothing launched)
bool launch_gate_up(const GemmProblem &g, RowSource src, WsTile tile, hipStream_t stream);
bool launch_down(const GemmProblem &g, RowSource src, WsTile tile, hipStream_t stream);
// Row-tiled kernel (ROWS_SORTED with block_m = 16*tile.mt).
bool launch_tiled(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
                  hipStream_t stream);
// 256 x 256 tile kernel (ROWS_SORTED with block_m = 256, or ROWS_DENSE with 256-row tiles).
bool launch_wide(bool gate_up, const GemmProblem &g, RowSource src, hipStream_t stream);

// ---------------------------------------------------------------- masked layout
// ids[e * max_m + i] = e for i < clamp(masked_m[e], 0, max_m), else -1.
void launch_masked_ids(const int32_t *masked_m, int E, int max_m, int32_t *ids,
                       hipStream_t stream);

// ---------------------------------------------------------------- MXFP4-weight GEMM
// The weight-streaming GEMM with MXFP4 weights (g.wq, g.wscale) and bf16 activations
// (moe_mx_kernel.h); SORTED, DIRECT or SCAN rows; K % 128 == 0.
bool launch_mx(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
               hipStream_t stream);
// The row-tiled MXFP4-weight GEMM (ROWS_SORTED with block_m = 64; tile.mt = 4, tile.nt
// 16-column tiles per wave, tile.stages).
bool launch_mx_tiled(bool gate_up, const GemmProblem &g, RowSource src, WsTile tile,
                     hipStream_t stream);
// The 256 x 256 tile GEMM with MXFP4 weights dequantised into its bf16 weight stages
// (moe_wide_kernel.h, k_wide_mx): ROWS_SORTED with block_m = 256, a schedule (g.sched) and
// K % 256 == 0; false (nothing launched) otherwise.
bool launch_wide_mx(bool gate_up, const GemmProblem &g, RowSource src, hipStream_t stream);

// ---------------------------------------------------------------- fp8 grouped GEMM
// out[e, m, n] for m < masked_m[e] (moe_fp8_kernel.h); K % 128 == 0, N % 64 == 0.
void launch_fp8_gemm(const uint8_t *a, const float *a_scale, const uint8_t *b,
                     const float *b_scale, const int32_t *masked_m, int E, int max_m, int N,
                     int K, uint16_t *out, hipStream_t stream);
// the same GEMM on the contiguous layout: a [P, K], expert e owning rows [offsets[e], offsets[e+1])
// a_route (optional): row q of a / a_scale is row a_route[q] / a_div of them
void launch_fp8_gemm_contig(const uint8_t *a, const float *a_scale, const uint8_t *b,
                            const float *b_scale, const int32_t *offsets, int E, int P, int N,
                            int K, uint16_t *out, hipStream_t stream,
                            const int32_t *a_route = nullptr, int a_div = 1);

// The direct FP8 pass for T*k <= 64 routes (moe_fp8_kernel.h, k_fp8_direct): one launch per
// GEMM reading the routes from topk_ids and quantising its own activation rows (gate-up: rows
// x[route / top_k], out h[route] = bf16(SiLU(g) * u), n_out = F; down: rows h[route], out
// y[route], n_out = H).  K % 256 == 0 and its LDS within kFp8DirectMaxLds (fp8_direct_shape_ok).
constexpr size_t kFp8DirectMaxLds = 160 * 1024;
size_t fp8_direct_lds_bytes(int K);
bool fp8_direct_shape_ok(int K);
void launch_fp8_direct(bool gate_up, const uint16_t *act, const int32_t *topk_ids, int P,
                       int top_k, int E, const uint8_t *b, const float *b_scale, int n_out, int K,
                       uint16_t *out, hipStream_t stream);

// ---------------------------------------------------------------- fp8 activation quantiser
// x [M, K] bf16 -> q [M, K] e4m3 codes, scale [M, ceil(K/128)] f32 (moe_quant.hip); K % 8 == 0.
void launch_quant_fp8(const uint16_t *x, int M, int K, uint8_t *q, float *scale,
                      hipStream_t stream);
// the same of h = bf16(SiLU(gu[r, k]) * gu[r, K + k]) for gate-up rows gu [M, 2K]
void launch_quant_fp8_swiglu(const uint16_t *gu, int M, int K, uint8_t *q, float *scale,
                             hipStream_t stream);

// ---------------------------------------------------------------- combine
// out[t] = bf16( sum_j w[t,j] * y[t*k+j] (+ ys[t]) ), routes with ids outside [0,E) skipped.
void launch_combine(const uint16_t *y, const int32_t *ids, const float *weights,
                    const uint16_t *ys, uint16_t *out, int T, int H, int k, int E, int dtype,
                    hipStream_t stream, const int32_t *row_of_route = nullptr);

// ---------------------------------------------------------------- measurement
// Workgroups of the streaming-read kernel (one per CU of the current device).
int stream_read_grid();
// Reads bytes (a multiple of 16) of buf once; writes one word per workgroup to sink[grid].
void launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid,
                        hipStream_t stream);

}  // namespace moe
