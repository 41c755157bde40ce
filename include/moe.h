/*
 * moe.h -- C ABI of the MI355X (gfx950) fused mixture-of-experts forward pass.
 *
 * The pass (TileOPs "MoE" benchmark page, FusedMoEFwd / FusedMoESharedExpertFwd):
 *   route    gating_output [T,E] f32 (+ correction_bias [E] f32) -> top-k ids and f32 weights
 *   align    stable sort of the T*k routes by expert, segments padded to a row tile
 *   gate-up  per expert: h = silu(X W_gate^T) * (X W_up^T), bf16 MFMA, f32 accumulate
 *   down     per expert: y = h W_down^T
 *   combine  out[t] = bf16( sum_j w[t,j] * y[t,j] (+ shared expert) ), fixed j order
 *
 * Conventions for every entry point:
 *   - Tensors are dense, row-major and contiguous in GPU device memory.  bf16 tensors are
 *     passed as uint16_t bit patterns.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *     enqueues work on that stream; nothing synchronises with the host and nothing is copied
 *     back to the host.
 *   - The caller owns every buffer (inputs, outputs, workspace).  The library never allocates,
 *     frees, caches or keeps a pointer after the call returns, so fixed buffers stay valid for
 *     graph capture (FlashInfer BF16-activation MoE PR: preallocated sort/workspace buffers
 *     keep graph addresses stable; invocation-local scratch, no module-global arena).
 *   - All arguments are validated on the host before anything is enqueued: a call that returns
 *     an error has launched nothing.  The library never falls back silently to another path.
 *   - Results are bitwise deterministic for identical inputs: no floating-point atomics.  The
 *     only atomics are integer counters: the align step's histograms, whose results do not
 *     depend on their order, and the tile counters of the 256 x 256 tile GEMM on the sorted
 *     layout (workspace), which decide only which workgroup computes a tile, never how.  Calls
 *     that share one workspace must therefore not overlap (as for any workspace contents).
 *   - Inputs are assumed finite.  T = 0 returns MOE_OK and enqueues nothing (pointers may then
 *     be NULL); moe_align_sort is the exception: with T = 0 it still writes its (empty) layout.
 *   - Route ids outside [0, E) (the -1 padding routes of the aiter MI308 decoding PR,
 *     "Changes": routes with expert id -1 are skipped) are skipped wherever ids are inputs.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

/* status codes */
enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* a size is non-positive (T may be 0) or top_k > num_experts */
    MOE_ERR_UNSUPPORTED = -3, /* a combination the kernels do not implement (see moe_params) */
    MOE_ERR_WORKSPACE = -4,   /* workspace smaller than the *_workspace_bytes query */
    MOE_ERR_LAUNCH = -5       /* the HIP runtime reported an error when enqueueing */
};

enum { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1 };

/* Element type of hidden_states, the expert weights, the shared expert's weights and out (and of
 * the intermediate h and expert-output rows): bf16 or IEEE f16 (TileOPs "MoE" page, FusedMoEFwd
 * qwen3-235b-decode: dtype=bf16, f16).  Passed as 16-bit patterns in uint16_t either way; the
 * MFMA products accumulate in f32 and every rounding to the type is to nearest even. */
enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F16 = 1 };

/* Path selection for fused_moe_fwd / fused_moe_shared_fwd / fused_moe_experts_fwd.
 * AUTO: DIRECT when T*k <= MOE_DIRECT_MAX_ROUTES and T*k <= 8*E (a few routed rows per expert),
 *   SORTED otherwise.
 * DIRECT: no sort; the expert GEMMs read topk_ids straight away (aiter MI308 decoding PR,
 *   "Changes": direct decoding from topk_ids).  For T*k <= 64 one workgroup per (route, column
 *   block), the first route of each expert gathering every route of that expert; above that one
 *   workgroup per (expert, column block) scanning all routes for its expert.  Requires
 *   T*k <= MOE_DIRECT_MAX_ROUTES, else MOE_ERR_UNSUPPORTED.
 * SORTED: align/sort first, then expert-contiguous grouped GEMMs. */
enum { MOE_PATH_AUTO = 0, MOE_PATH_DIRECT = 1, MOE_PATH_SORTED = 2 };
#define MOE_DIRECT_MAX_ROUTES 512

/* Attributes of the pass (TileOPs "MoE" page, FusedMoEFwd and FusedTopKFwd attributes).
 *   num_tokens T >= 0; hidden H; num_experts E; inter F (expert intermediate size); top_k k.
 *   scoring: MOE_SCORING_SOFTMAX (the page's default when no scoring_func is given) or
 *     MOE_SCORING_SIGMOID.
 *   renormalize: 0/1 -- divide the chosen weights by their sum.
 *   num_expert_group, topk_group: DeepSeek-style grouped top-k; (1, 1) = ungrouped.
 *   routed_scaling_factor: multiplies every routed weight (after renormalisation); 1 = none.
 *   path: MOE_PATH_*.
 *   dtype: MOE_DTYPE_* (0, the zero-initialised default, is bf16).
 * Supported: 1 <= k <= 32, k <= E <= 1024, E % num_expert_group == 0,
 *   1 <= topk_group <= num_expert_group <= 64, k <= topk_group * E / num_expert_group,
 *   H % 64 == 0 and F % 64 == 0; softmax only with no correction_bias and no grouping.
 *   Anything else returns MOE_ERR_UNSUPPORTED (MOE_ERR_SHAPE for non-positive sizes). */
typedef struct moe_params {
    int32_t num_tokens;
    int32_t hidden;
    int32_t num_experts;
    int32_t inter;
    int32_t top_k;
    int32_t scoring;
    int32_t renormalize;
    int32_t num_expert_group;
    int32_t topk_group;
    float routed_scaling_factor;
    int32_t path;
    int32_t dtype;
} moe_params_t;

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Static, NUL-terminated description of a status code.  Never NULL. */
const char *moe_status_string(int status);

/* Checks *p against the support rules above without touching the GPU.  correction_bias_given
 * and shared_inter (S, 0 = no shared expert) take part in the check.  Returns a status. */
int moe_check_params(const moe_params_t *p, int correction_bias_given, int32_t shared_inter);

/* ---------------------------------------------------------------------------------------
 * moe_route -- top-k routing (TileOPs "MoE" page, FusedTopKFwd: gating_output [T,E] with
 * top_k, renormalize, scoring_func, correction_bias [E] f32, num_expert_group, topk_group,
 * routed_scaling_factor).
 *   gating_output   [T,E] f32, device.
 *   correction_bias [E] f32, device, or NULL.  Sigmoid only; it shifts the selection keys
 *                   and never the weights.
 *   topk_ids        [T,k] int32, device, written: chosen experts in descending key order
 *                   (ties: lower expert index).
 *   topk_weights    [T,k] f32, device, written: score of each chosen expert (softmax
 *                   probability or sigmoid), divided by the chosen scores' sum if
 *                   renormalize, times routed_scaling_factor.
 * Selection keys: softmax selects on the f32 logit; sigmoid on f32(f32(sigmoid(g)) + bias).
 * A group's score is the f32 sum of its two largest keys; groups and experts tie to the lower
 * index.  Scores and weights are computed in double and rounded to f32 once.
 * Errors: MOE_ERR_NULL (gating/ids/weights/p NULL), MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED,
 * MOE_ERR_LAUNCH.  Only p's T, E, k, scoring, renormalize, grouping and scaling are read. */
int moe_route(const float *gating_output, const float *correction_bias, const moe_params_t *p,
              int32_t *topk_ids, float *topk_weights, void *stream);

/* ---------------------------------------------------------------------------------------
 * moe_align_sort -- expert histogram, padded prefix sum and stable permutation of the routes
 * (TileOPs "MoE" page, MoEPermuteAlignFwd on topk_ids [T,K] i32; MoEPostPermuteFwd's
 * inverse_indices [T*K]; block_m = 1 is that page's tight packing with alignment 1).
 *   topk_ids          [T,k] int32, device.  Route r = t*k + j.  Ids outside [0,E) are
 *                     skipped.  Repeated ids of one token are each counted.
 *   block_m           row tile, 1..1024: every expert's segment is padded up to a multiple.
 *   sorted_route_ids  [T*k + E*(block_m-1)] int32, device, written: route r of each row of
 *                     the expert-contiguous order, routes of one expert in increasing r;
 *                     padding and unused rows hold -1.
 *   expert_offsets    [E+1] int32, device, written: first row of each expert's padded
 *                     segment; expert_offsets[E] = total padded rows.
 *   tile_expert       [T*k/block_m + E] int32, device, written: expert of each block_m-row
 *                     tile, -1 past the last tile.
 *   inverse_pos       [T*k] int32, device, written: row of route r, -1 for skipped routes.
 *   n_tiles           [1] int32, device, written: number of tiles (expert_offsets[E]/block_m).
 *   workspace         device scratch of at least moe_align_sort_workspace_bytes(T, k, E,
 *                     block_m) bytes, 4-byte aligned, owned by the caller; contents on entry
 *                     are ignored and on return unspecified (the sort/workspace buffers that
 *                     the FlashInfer BF16-activation MoE PR preallocates).  May be NULL when
 *                     that size is 0.
 * Up to 1024 routes one workgroup does everything; above that the workspace holds a
 * chunks x E table of per-chunk expert counts (chunks of 1024 routes) and the sort runs as
 * three launches: per-chunk histograms, one workgroup for the padded layout, then every
 * chunk's stable scatter at once.  The outputs are the same either way.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (T < 0, k < 1, E < 1), MOE_ERR_UNSUPPORTED
 * (E > 1024, block_m outside 1..1024, T*k >= 2^30, a misaligned workspace),
 * MOE_ERR_WORKSPACE (workspace_bytes below the size query), MOE_ERR_LAUNCH. */
int moe_align_sort(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                   int32_t *sorted_route_ids, int32_t *expert_offsets, int32_t *tile_expert,
                   int32_t *inverse_pos, int32_t *n_tiles, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Bytes of workspace moe_align_sort needs for T*k routes and E experts: 0 up to 1024 routes,
 * else 4 * ceil(T*k / 1024) * E.  Returns 0 for arguments moe_align_sort would reject. */
size_t moe_align_sort_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t block_m);

/* ---------------------------------------------------------------------------------------
 * Workspace of the fused entry points: device memory the caller allocates (256-byte aligned)
 * and passes in.  Its size depends on p (T, H, E, F, k, path) and shared_inter; contents on
 * entry are ignored and on return are unspecified.  One workspace must not be used by two
 * calls that can run at the same time. */
size_t fused_moe_workspace_bytes(const moe_params_t *p, int32_t shared_inter);

/* fused_moe_fwd -- the whole pass (TileOPs "MoE" page, FusedMoEFwd: hidden_states [T,H],
 * gating_output [T,E] f32, w_gate_up [E,2F,H], w_down [E,H,F], optional correction_bias [E]).
 *   hidden_states  [T,H] bf16.
 *   gating_output  [T,E] f32.
 *   w_gate_up      [E,2F,H] bf16: rows [0,F) of each expert are the gate projection,
 *                  rows [F,2F) the up projection.
 *   w_down         [E,H,F] bf16.
 *   correction_bias [E] f32 or NULL.
 *   out            [T,H] bf16, written (every row; no prior clear needed).
 *   topk_ids_out   [T,k] int32 or NULL: receives the routing.
 *   topk_weights_out [T,k] f32 or NULL: receives the route weights.
 *   workspace / workspace_bytes: see fused_moe_workspace_bytes.
 * The intermediate h is rounded to bf16 after SiLU(gate)*up, and expert output rows are
 * rounded to bf16 before the f32 weighted combine.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
 * MOE_ERR_LAUNCH. */
int fused_moe_fwd(const uint16_t *hidden_states, const float *gating_output,
                  const uint16_t *w_gate_up, const uint16_t *w_down,
                  const float *correction_bias, const moe_params_t *p, uint16_t *out,
                  int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                  size_t workspace_bytes, void *stream);

/* fused_moe_fwd_noalloc -- fused_moe_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, which instead is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES (128 MiB) of device memory inside the library, one per GPU, held
 * until the process ends.  The call allocates nothing; its first call on a device (with that
 * device current, and the stream on it) looks up the array's device address.  Every call on a
 * GPU uses that GPU's one array, so calls that can overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls in one stream's order are fine.  Results
 * are bit-identical to fused_moe_fwd's.
 * Errors: as fused_moe_fwd; MOE_ERR_WORKSPACE when fused_moe_workspace_bytes(p, 0) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (checked before anything is enqueued; the Qwen3 decode and batch
 * workloads fit, 4096-token DeepSeek-V3 prefill does not); MOE_ERR_LAUNCH if the array's
 * address cannot be looked up. */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
int fused_moe_fwd_noalloc(const uint16_t *hidden_states, const float *gating_output,
                          const uint16_t *w_gate_up, const uint16_t *w_down,
                          const float *correction_bias, const moe_params_t *p, uint16_t *out,
                          int32_t *topk_ids_out, float *topk_weights_out, void *stream);

/* fused_moe_shared_fwd -- fused_moe_fwd plus a shared expert added unweighted (TileOPs "MoE"
 * page, FusedMoESharedExpertFwd: shared_w_gate_up [2S,H], shared_w_down [H,S]).
 *   shared_w_gate_up [2S,H] bf16 (rows [0,S) gate, [S,2S) up); shared_w_down [H,S] bf16;
 *   shared_inter S >= 64, S % 64 == 0.  The routed scaling factor does not apply to it.
 * The shared expert needs no routing, so its two GEMMs run on a second stream of the
 * library's (one per device, default priority, made on first use) on three eighths of the
 * CUs, beside the routing and the routed GEMMs on `stream`; an event forks that stream from
 * `stream` at the call and another joins it back before the combine.  The call therefore
 * stays ordered on `stream` (and can be captured into a graph from it).  The stages of
 * fused_moe_experts_stage run the same kernels in order on one stream, with the same results.
 * Other arguments and errors as fused_moe_fwd. */
int fused_moe_shared_fwd(const uint16_t *hidden_states, const float *gating_output,
                         const uint16_t *w_gate_up, const uint16_t *w_down,
                         const float *correction_bias, const uint16_t *shared_w_gate_up,
                         const uint16_t *shared_w_down, int32_t shared_inter,
                         const moe_params_t *p, uint16_t *out, int32_t *topk_ids_out,
                         float *topk_weights_out, void *workspace, size_t workspace_bytes,
                         void *stream);

/* fused_moe_experts_fwd -- the pass with the routing given (TileOPs "MoE" page,
 * FusedMoEExpertsFwd: hidden_states [T,H], w_gate_up, w_down, topk_weights [T,K] f32,
 * topk_ids [T,K] i32).  topk_ids may hold -1 (skipped) and repeated ids (each counted).
 * Only p's T, H, E, F, k and path are read.  Workspace as fused_moe_fwd's with the same p.
 * Errors as fused_moe_fwd. */
int fused_moe_experts_fwd(const uint16_t *hidden_states, const uint16_t *w_gate_up,
                          const uint16_t *w_down, const int32_t *topk_ids,
                          const float *topk_weights, const moe_params_t *p, uint16_t *out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * fused_moe_experts_stage -- one step of the expert part of the pass, on the caller's
 * workspace, so that each step can be timed or checked on its own.  Calling the stages
 * MOE_STAGE_ALIGN, MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_SHARED (only with a shared
 * expert) and MOE_STAGE_COMBINE in that order, on one stream with one workspace, enqueues
 * exactly the kernels of fused_moe_experts_fwd (or of the expert part of
 * fused_moe_shared_fwd), with the same results.
 *   MOE_STAGE_ALIGN    sorted path: moe_align_sort into the workspace; direct path: nothing.
 *   MOE_STAGE_GATE_UP  gate-up grouped GEMM with the SiLU(gate)*up epilogue -> h (workspace)
 *                      (TileOPs "MoE" page, MoEGroupedGemmFwd activation=silu_and_mul).
 *   MOE_STAGE_DOWN     down grouped GEMM -> expert output rows (workspace)
 *                      (MoEGroupedGemmFwd on w_down [E,H,F]).
 *   MOE_STAGE_SHARED   shared expert's dense SwiGLU MLP -> its output rows (workspace)
 *                      (SharedExpertMLPFwd).
 *   MOE_STAGE_COMBINE  weighted combine -> out (MoEPostPermuteFwd).
 * Arguments as fused_moe_experts_fwd, plus the shared weights (NULL and shared_inter 0 when
 * there is no shared expert); each stage reads only what it needs, the others may be NULL.
 * The workspace size is fused_moe_workspace_bytes(p, shared_inter).
 * Errors as fused_moe_experts_fwd; an unknown stage, or MOE_STAGE_SHARED without a shared
 * expert, is MOE_ERR_UNSUPPORTED. */
enum {
    MOE_STAGE_ALIGN = 1,
    MOE_STAGE_GATE_UP = 2,
    MOE_STAGE_DOWN = 3,
    MOE_STAGE_SHARED = 4,
    MOE_STAGE_COMBINE = 5
};
int fused_moe_experts_stage(int stage, const uint16_t *hidden_states, const uint16_t *w_gate_up,
                            const uint16_t *w_down, const int32_t *topk_ids,
                            const float *topk_weights, const uint16_t *shared_w_gate_up,
                            const uint16_t *shared_w_down, int32_t shared_inter,
                            const moe_params_t *p, uint16_t *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * fused_moe_mxfp4_fwd -- fused_moe_fwd with MXFP4 expert weights and bf16 activations (W4A16;
 * FlashInfer BF16-activation PR: 4-bit expert weights with BF16 activations, here in the OCP MX
 * format that gfx950 converts natively).  Weights in MXFP4: blocks of 32 consecutive elements
 * along the reduction dimension share one E8M0 scale; each element is an e2m1 code.
 *   w_gate_up_q      [E, 2F, H/2] uint8: two e2m1 codes per byte, element 2i in the low
 *                    nibble of byte i (e2m1: sign, 2 exponent bits with bias 1, 1 mantissa
 *                    bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *   w_gate_up_scale  [E, 2F, H/32] uint8: E8M0 scales, 2^(s-127); 255 is NaN.
 *   w_down_q         [E, H, F/2] uint8; w_down_scale [E, H, F/32] uint8.
 * Expert weight (e, n, k) = e2m1(code) * 2^(scale - 127); everything else as fused_moe_fwd
 * (rows [0,F) of w_gate_up are gate, [F,2F) up).  For scales up to 252 the dequantised
 * weights are exact in bf16, so the sums are those of the bf16 pass on those weights.  Needs p->dtype == MOE_DTYPE_BF16,
 * H % 128 == 0 and F % 128 == 0; 16-byte aligned hidden_states, the code tensors, out and the
 * workspace, 4-byte aligned scale tensors.  No shared expert.
 * Kernels by routed rows per expert (T*k/E): up to 8, weight streaming in 16-row passes; up to
 * 64 (48 with grouped routing, whose busiest experts take far more than the mean), 64-row
 * tiles, each wave dequantising its weight rows into its MFMA operands; above, with
 * H and F multiples of 256, 256 x 256 tiles whose weights arrive as codes and scales by DMA and
 * are dequantised by each wave into its MFMA operands (the bf16 pass's prefill tile otherwise).
 * Workspace: fused_moe_mxfp4_workspace_bytes(p) bytes.
 * Errors: as fused_moe_fwd. */
size_t fused_moe_mxfp4_workspace_bytes(const moe_params_t *p);
int fused_moe_mxfp4_fwd(const uint16_t *hidden_states, const float *gating_output,
                        const uint8_t *w_gate_up_q, const uint8_t *w_gate_up_scale,
                        const uint8_t *w_down_q, const uint8_t *w_down_scale,
                        const float *correction_bias, const moe_params_t *p, uint16_t *out,
                        int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                        size_t workspace_bytes, void *stream);

/* fused_moe_mxfp4_stage -- one step of fused_moe_mxfp4_fwd's expert part with the routing given
 * (topk_ids / topk_weights [T,k] as fused_moe_experts_fwd takes them): MOE_STAGE_ALIGN,
 * MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_COMBINE in that order enqueue exactly the expert
 * kernels of the fused call (for per-kernel timing and tests).  A stage checks only the
 * pointers it reads.  MOE_STAGE_SHARED: MOE_ERR_UNSUPPORTED. */
int fused_moe_mxfp4_stage(int stage, const uint16_t *hidden_states, const uint8_t *w_gate_up_q,
                          const uint8_t *w_gate_up_scale, const uint8_t *w_down_q,
                          const uint8_t *w_down_scale, const int32_t *topk_ids,
                          const float *topk_weights, const moe_params_t *p, uint16_t *out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * fused_moe_fp8_fwd -- fused_moe_fwd with FP8 expert weights: OCP e4m3 codes with f32 scales
 * per 128 x 128 weight block (TileOPs "MoE" page, MoEGroupedGemmFP8Fwd's b / b_scale), and the
 * bf16 activations quantised per 1 x 128 group on the way in (moe_quant_fp8's rule).
 *   w_gate_up        [E, 2F, H] uint8 e4m3 (rows [0,F) gate, [F,2F) up);
 *   w_gate_up_scale  [E, 2F/128, H/128] f32;
 *   w_down           [E, H, F] uint8 e4m3; w_down_scale [E, H/128, F/128] f32.
 * The pass: route; the routes in expert order (align with block_m 1); each token's x row
 * quantised once (moe_quant_fp8); the gate-up GEMM as moe_grouped_gemm_fp8_contiguous on the
 * routes' rows (a route reads its token's codes; bf16 gate and up); h = bf16(SiLU(gate) * up)
 * quantised the same way; the down GEMM (bf16
 * rows); the weighted combine of fused_moe_fwd.  Needs p->dtype == MOE_DTYPE_BF16,
 * H % 128 == 0, F % 128 == 0, no shared expert; 16-byte aligned hidden_states, weights, out
 * and workspace, 4-byte aligned scales.
 * p->path: MOE_PATH_DIRECT computes the same values with no align and no quantiser launches:
 * each GEMM reads the routes from topk_ids and quantises its own rows by the same rule (the
 * decoding form for a few tokens).  It needs T*k <= 64 and H, F multiples of 256 small enough
 * for one workgroup's LDS to hold 16 quantised rows (K up to 9472), else MOE_ERR_UNSUPPORTED.
 * AUTO takes it when it is allowed and T*k <= 8*E; SORTED never.
 * Workspace: fused_moe_fp8_workspace_bytes(p) bytes (depends on the path taken).
 * Errors: as fused_moe_fwd. */
size_t fused_moe_fp8_workspace_bytes(const moe_params_t *p);
int fused_moe_fp8_fwd(const uint16_t *hidden_states, const float *gating_output,
                      const uint8_t *w_gate_up, const float *w_gate_up_scale,
                      const uint8_t *w_down, const float *w_down_scale,
                      const float *correction_bias, const moe_params_t *p, uint16_t *out,
                      int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                      size_t workspace_bytes, void *stream);

/* fused_moe_fp8_stage -- one step of fused_moe_fp8_fwd's expert part with the routing given:
 * MOE_STAGE_ALIGN (expert order and the quantised x rows; direct path: nothing),
 * MOE_STAGE_GATE_UP, MOE_STAGE_DOWN (h quantised, then the down GEMM), MOE_STAGE_COMBINE, in
 * that order, enqueue exactly the expert kernels of the fused call.  A stage checks only the
 * pointers it reads (hidden_states: ALIGN on the sorted path, GATE_UP on the direct one).
 * MOE_STAGE_SHARED: MOE_ERR_UNSUPPORTED. */
int fused_moe_fp8_stage(int stage, const uint16_t *hidden_states, const uint8_t *w_gate_up,
                        const float *w_gate_up_scale, const uint8_t *w_down,
                        const float *w_down_scale, const int32_t *topk_ids,
                        const float *topk_weights, const moe_params_t *p, uint16_t *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * Masked layout: the expert MLPs of one expert-parallel shard (TileOPs "MoE" page,
 * MoEGroupedGemmFwd with a: [E, layout.max_m, K] and layout_metadata [E] i32, workload
 * ds-v3-ep8-masked; MoEPrePermuteFwd's num_local_experts).  Local expert e owns the row block
 * a[e, 0:max_m, :] whose first masked_m[e] rows are the tokens routed to it (placed there by the
 * exchange between GPUs); the remaining rows of the block are ignored.
 *   a          [E, max_m, H] bf16.
 *   masked_m   [E] int32, device: rows in use per expert; clamped to [0, max_m] on the device.
 *   w_gate_up  [E, 2F, H] bf16 (rows [0,F) gate, [F,2F) up); w_down [E, H, F] bf16.
 *   out        [E, max_m, H] bf16: row i of expert e is written for i < masked_m[e] with
 *              bf16( bf16(SiLU(gate) * up) W_down^T ); the other rows are not touched.  There
 *              are no route weights: weighting and summing a token's rows belongs to the caller
 *              after the return exchange.
 *   E in 1..1024, max_m >= 0 (0: nothing is enqueued), H % 64 == 0, F % 64 == 0,
 *   E * max_m < 2^30; a, the weights, out and the workspace 16-byte aligned.
 * Workspace: fused_moe_masked_workspace_bytes(E, max_m, H, F) bytes (0 when nothing is to do).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E < 1, max_m < 0, H < 1 or F < 1),
 * MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH. */
size_t fused_moe_masked_workspace_bytes(int32_t E, int32_t max_m, int32_t H, int32_t F);
int fused_moe_masked_fwd(const uint16_t *a, const int32_t *masked_m, const uint16_t *w_gate_up,
                         const uint16_t *w_down, int32_t E, int32_t max_m, int32_t H, int32_t F,
                         uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);

/* fused_moe_masked_stage -- one step of fused_moe_masked_fwd with the same arguments:
 * MOE_STAGE_ALIGN (the expert-contiguous layout of the rows in use, into the workspace),
 * MOE_STAGE_GATE_UP (-> h in the workspace), MOE_STAGE_DOWN (-> out).  The three in that order
 * enqueue exactly the kernels of fused_moe_masked_fwd.  Other stages: MOE_ERR_UNSUPPORTED. */
int fused_moe_masked_stage(int stage, const uint16_t *a, const int32_t *masked_m,
                           const uint16_t *w_gate_up, const uint16_t *w_down, int32_t E,
                           int32_t max_m, int32_t H, int32_t F, uint16_t *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * moe_grouped_gemm_fp8 -- block-scaled FP8 grouped GEMM of the masked layout (TileOPs "MoE"
 * page, MoEGroupedGemmFP8Fwd: a [E, layout.max_m, K] and b [E, N, K] in fp8e4m3, a_scale
 * [E, layout.max_m, ceil_div(K, 128)] f32, b_scale [E, ceil_div(N, 128), ceil_div(K, 128)] f32,
 * layout_metadata [E] i32):
 *   out[e, m, n] = bf16( sum_kb a_scale[e,m,kb] * b_scale[e,n/128,kb]
 *                        * sum_{k in block kb} a[e,m,k] * b[e,n,k] )   for m < masked_m[e].
 *   a        [E, max_m, K] uint8: OCP e4m3 codes (S.EEEE.MMM, bias 7, no infinities).
 *   a_scale  [E, max_m, K/128] f32; b [E, N, K] uint8 e4m3; b_scale [E, ceil(N/128), K/128] f32.
 *   masked_m [E] int32, device: rows in use per expert, clamped to [0, max_m] on the device.
 *   out      [E, max_m, N] bf16: rows m < masked_m[e] written, the other rows untouched.
 * A block's products are summed by the MFMA (whose internal sum carries about 15 fraction bits
 * relative to the sum of the products' magnitudes, not a full f32 sum), scaled in f32 and
 * accumulated in f32; NaN codes (S.1111.111) propagate.  Needs E >= 1, max_m >= 0 (0: nothing is enqueued),
 * N % 64 == 0, K % 128 == 0, E * ceil(max_m/64) * ceil(N/256) < 2^30, 16-byte aligned a, b,
 * out and 4-byte aligned scales.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E < 1, max_m < 0, N < 1, K < 1), MOE_ERR_UNSUPPORTED
 * (N % 64, K % 128, E * max_m >= 2^30, the tile count, alignment), MOE_ERR_LAUNCH. */
int moe_grouped_gemm_fp8(const uint8_t *a, const float *a_scale, const uint8_t *b,
                         const float *b_scale, const int32_t *masked_m, int32_t E, int32_t max_m,
                         int32_t N, int32_t K, uint16_t *out, void *stream);

/* moe_grouped_gemm_fp8_contiguous -- the same GEMM on the contiguous layout (TileOPs "MoE"
 * page, layout=contiguous(packing=tight, metadata_kind=physical_psum) of its grouped GEMMs):
 * the rows of all experts stacked in one matrix, expert e owning rows
 * [expert_offsets[e], expert_offsets[e+1]).
 *   out[r, n] = bf16( sum_kb a_scale[r,kb] * b_scale[e,n/128,kb]
 *                     * sum_{k in block kb} a[r,k] * b[e,n,k] )   for r in expert e's rows.
 *   a               [P, K] uint8 e4m3; a_scale [P, K/128] f32.
 *   b, b_scale      as moe_grouped_gemm_fp8.
 *   expert_offsets  [E+1] int32, device: non-decreasing prefix sums of the rows per expert
 *                   (each clamped to [0, P] on the device; a decreasing pair gives no rows).
 *   out             [P, N] bf16: rows of some expert written, the others untouched.
 * Same arithmetic as moe_grouped_gemm_fp8.  Needs E in 1..1024, 0 <= P < 2^30 (0: nothing is
 * enqueued), (ceil(P/64) + E) * ceil(N/256) < 2^30, N % 64 == 0, K % 128 == 0, 16-byte aligned
 * a, b, out and 4-byte aligned scales and offsets.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E < 1, P < 0, N < 1, K < 1), MOE_ERR_UNSUPPORTED,
 * MOE_ERR_LAUNCH. */
int moe_grouped_gemm_fp8_contiguous(const uint8_t *a, const float *a_scale, const uint8_t *b,
                                    const float *b_scale, const int32_t *expert_offsets,
                                    int32_t E, int32_t P, int32_t N, int32_t K, uint16_t *out,
                                    void *stream);

/* moe_quant_fp8 -- bf16 activations to the e4m3 codes and 1 x 128 group scales that the FP8
 * grouped GEMMs take as a / a_scale (TileOPs "MoE" page, MoEGroupedGemmFP8Fwd: a_scale
 * [.., ceil_div(K, 128)] f32; the page gives the scales' shape, this library's rule is):
 *   s[r,g]  = amax_{k in group g} |x[r,k]| / 448   (IEEE f32 division; 1 for an all-zero group)
 *   q[r,k]  = the e4m3 code nearest to x[r,k] / s[r,g] (IEEE f32 division), ties to the even
 *             code, magnitudes from 448 up saturated to 448.
 *   x [M, K] bf16 (16-byte aligned), q [M, K] uint8 (8-byte aligned), scale [M, ceil(K/128)]
 *   f32; the last group of a row may be partial.  Needs M >= 0 (0: nothing is enqueued),
 *   K % 8 == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (M < 0, K < 1), MOE_ERR_UNSUPPORTED (K % 8, alignment),
 * MOE_ERR_LAUNCH. */
int moe_quant_fp8(const uint16_t *x, int32_t M, int32_t K, uint8_t *q, float *scale,
                  void *stream);

/* ---- measurement: the HBM streaming-read ceiling
 *
 * Not a step of the pass: the plain sequential read that the expert GEMMs' weight streams are
 * measured against (a roofline is reported against the published HBM peak; this is the rate
 * the same CUs reach on a pure read, so it gives the achievable share of that peak).
 *
 * moe_stream_read_sink_words() is the number of uint32 words moe_stream_read writes to sink
 * (G = one per CU of the current device).  moe_stream_read enqueues one read of bytes bytes of
 * buf (device memory, 16-byte aligned, bytes a multiple of 16) with 16-byte non-temporal loads
 * by G 512-thread workgroups sweeping the buffer in 8 KB blocks (block q read by workgroup
 * q % G); sink[b] receives the xor of the 32-bit words workgroup b read (so the loads cannot be
 * elided).  bytes = 0: nothing is enqueued.
 * Errors: MOE_ERR_NULL (buf or sink NULL with bytes > 0), MOE_ERR_UNSUPPORTED (alignment, bytes
 * % 16), MOE_ERR_LAUNCH. */
int moe_stream_read_sink_words(void);
int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
