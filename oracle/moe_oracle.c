/*
 * moe_oracle.c -- CPU oracle of the fused mixture-of-experts (MoE) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct definition that the
 * GPU library is checked against.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it; the product path never does.  It shares no source, header,
 * table or helper with the GPU library and includes no HIP header.
 *
 * What it computes (sources: the TileOPs "MoE" benchmark page, op signatures of FusedMoEFwd,
 * FusedMoESharedExpertFwd, FusedTopKFwd, MoEPermuteAlignFwd and MoEPostPermuteFwd):
 *   route     gating logits -> top-k expert ids and f32 route weights
 *   align     stable counting sort of the routes by expert, each expert padded to block_m rows
 *   experts   out[t] = RNE_bf16( sum_j w[t,j] * SwiGLU_{id[t,j]}(x[t]) + SharedSwiGLU(x[t]) )
 *   fp8 grouped GEMM (MoEGroupedGemmFP8Fwd, masked layout, e4m3 operands with f32 scales per
 *             1 x 128 activation block and per 128 x 128 weight block; and the same GEMM on
 *             the contiguous layout of the page's bf16 grouped GEMMs)
 *   fp8 quant bf16 activations -> e4m3 codes with one f32 scale per 1 x 128 group
 *   mxfp4     dequantisation of MXFP4 expert weights (e2m1 codes, E8M0 block scales)
 *
 * Precision: every floating-point quantity is double; results are rounded exactly once at the
 * end (route weights to f32, outputs to bf16 with round-to-nearest-even).  The only f32
 * arithmetic is the selection key of sigmoid scoring (score rounded to f32 plus the f32 bias)
 * and the two divisions of the fp8 quantiser (group scale and quotient), which is where those
 * integer decisions are defined in f32 on both sides.
 *
 * Readings of the pages that this file adopts where they are silent are listed in the
 * comments of the function that applies them.
 *
 * Every function returns 0 on success and a negative value for an argument it rejects.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_SOFTMAX 0
#define ORACLE_SIGMOID 1

/* ---------------------------------------------------------------- number formats */

/* bf16 bit pattern -> double (exact: bf16 is the upper half of an IEEE binary32). */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bf16 bit pattern, one rounding, round-to-nearest-even.
 * bf16 keeps 8 significant bits and binary32's exponent range (normal >= 2^-126, subnormal
 * quantum 2^-133).  The value is scaled so that one unit in the last bf16 place is 1, rounded
 * with nearbyint (the default mode is to-nearest-even), and scaled back; the result is exactly
 * representable in binary32, whose upper 16 bits are then the bf16 pattern. */
uint16_t oracle_double_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    double r;
    if (v == 0.0) {
        r = v;
    } else {
        int e;
        (void)frexp(v, &e);               /* |v| = m * 2^e, m in [0.5, 1) */
        int q_exp = (e - 1 >= -126) ? (e - 8) : -133;  /* exponent of one ulp */
        double q = nearbyint(ldexp(v, -q_exp));
        r = ldexp(q, q_exp);
        if (fabs(r) > 3.38953138925153547590470800371487866880e+38) /* largest finite bf16 */
            r = (v > 0) ? INFINITY : -INFINITY;
    }
    float f = (float)r;                   /* exact */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- routing
 *
 * Per token (TileOPs "MoE" page, FusedTopKFwd and FusedMoEFwd attributes top_k, scoring_func,
 * renormalize, num_expert_group, topk_group, routed_scaling_factor; correction_bias [E] f32):
 *  1. scores s_e: softmax over the row (the default when no scoring_func is given) or the
 *     logistic sigmoid 1/(1+exp(-g_e)), in double.
 *  2. selection keys k_e (f32): softmax selects on the raw logit g_e (softmax is strictly
 *     increasing along a row, so the chosen set is the same); sigmoid selects on
 *     f32(f32(s_e) + bias_e) -- the bias steers the choice only.
 *  3. grouped top-k (DeepSeek-style): the E experts form num_expert_group contiguous groups; a
 *     group's score is the f32 sum of its two largest keys (its largest key when a group has one
 *     expert); the topk_group best groups stay eligible, ties to the lower group index.
 *  4. top-k over eligible experts by key, ties to the lower expert index; ids are listed in
 *     descending key order.
 *  5. weights: the unbiased scores of the chosen experts; divided by their sum when
 *     renormalize is set; then multiplied by routed_scaling_factor; rounded to f32 once.
 */

/* "a ranks before b" for selection: larger key first, then lower index. */
static int ranks_before(float key_a, int idx_a, float key_b, int idx_b)
{
    if (key_a != key_b)
        return key_a > key_b;
    return idx_a < idx_b;
}

int oracle_route(const float *gating, const float *bias, int T, int E, int k, int scoring,
                 int renormalize, int num_expert_group, int topk_group, double rsf,
                 int32_t *topk_ids, float *topk_weights)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E)
        return -2;
    if (scoring != ORACLE_SOFTMAX && scoring != ORACLE_SIGMOID)
        return -3;
    if (num_expert_group <= 0 || E % num_expert_group != 0 || topk_group <= 0 ||
        topk_group > num_expert_group)
        return -3;
    const int group_size = E / num_expert_group;
    if (k > topk_group * group_size)
        return -3;

    double *score = malloc(sizeof(double) * (size_t)E);
    float *key = malloc(sizeof(float) * (size_t)E);
    int *eligible = malloc(sizeof(int) * (size_t)E);
    int *taken = malloc(sizeof(int) * (size_t)E);
    float *gscore = malloc(sizeof(float) * (size_t)num_expert_group);
    int *gkept = malloc(sizeof(int) * (size_t)num_expert_group);
    if (!score || !key || !eligible || !taken || !gscore || !gkept) {
        free(score); free(key); free(eligible); free(taken); free(gscore); free(gkept);
        return -4;
    }

    for (int t = 0; t < T; ++t) {
        const float *g = gating + (size_t)t * E;

        /* 1-2: scores and selection keys */
        if (scoring == ORACLE_SOFTMAX) {
            double m = g[0];
            for (int e = 1; e < E; ++e)
                if (g[e] > m)
                    m = g[e];
            double z = 0.0;
            for (int e = 0; e < E; ++e)
                z += exp((double)g[e] - m);
            for (int e = 0; e < E; ++e) {
                score[e] = exp((double)g[e] - m) / z;
                key[e] = g[e];
            }
        } else {
            for (int e = 0; e < E; ++e) {
                score[e] = 1.0 / (1.0 + exp(-(double)g[e]));
                float s32 = (float)score[e];
                float b = bias ? bias[e] : 0.0f;
                key[e] = s32 + b; /* f32 add */
            }
        }

        /* 3: group filter */
        for (int e = 0; e < E; ++e)
            eligible[e] = 1;
        if (num_expert_group > 1) {
            for (int gi = 0; gi < num_expert_group; ++gi) {
                const int e0 = gi * group_size;
                int best = e0;
                for (int e = e0 + 1; e < e0 + group_size; ++e)
                    if (ranks_before(key[e], e, key[best], best))
                        best = e;
                if (group_size == 1) {
                    gscore[gi] = key[best];
                } else {
                    int second = -1;
                    for (int e = e0; e < e0 + group_size; ++e) {
                        if (e == best)
                            continue;
                        if (second < 0 || ranks_before(key[e], e, key[second], second))
                            second = e;
                    }
                    gscore[gi] = key[best] + key[second]; /* f32 add */
                }
                gkept[gi] = 0;
            }
            for (int n = 0; n < topk_group; ++n) {
                int pick = -1;
                for (int gi = 0; gi < num_expert_group; ++gi) {
                    if (gkept[gi])
                        continue;
                    if (pick < 0 || ranks_before(gscore[gi], gi, gscore[pick], pick))
                        pick = gi;
                }
                gkept[pick] = 1;
            }
            for (int e = 0; e < E; ++e)
                eligible[e] = gkept[e / group_size];
        }

        /* 4: top-k by repeated selection of the best remaining eligible expert */
        for (int e = 0; e < E; ++e)
            taken[e] = 0;
        int32_t *ids = topk_ids + (size_t)t * k;
        for (int j = 0; j < k; ++j) {
            int pick = -1;
            for (int e = 0; e < E; ++e) {
                if (!eligible[e] || taken[e])
                    continue;
                if (pick < 0 || ranks_before(key[e], e, key[pick], pick))
                    pick = e;
            }
            taken[pick] = 1;
            ids[j] = pick;
        }

        /* 5: weights */
        double sum = 0.0;
        for (int j = 0; j < k; ++j)
            sum += score[ids[j]];
        for (int j = 0; j < k; ++j) {
            double w = score[ids[j]];
            if (renormalize)
                w = w / sum;
            w = w * rsf;
            topk_weights[(size_t)t * k + j] = (float)w;
        }
    }

    free(score); free(key); free(eligible); free(taken); free(gscore); free(gkept);
    return 0;
}

/* ---------------------------------------------------------------- align / sort
 *
 * Expert histogram -> per-expert row counts padded up to block_m -> exclusive prefix sum ->
 * stable placement of every route (route r = t*k + j, in increasing r) into its expert's
 * segment (TileOPs "MoE" page, MoEPermuteAlignFwd on topk_ids [T, K]; the contiguous layout
 * with physical prefix-sum metadata; block_m = 1 is that page's tight packing).
 * Ids outside [0, E) -- the -1 padding routes of the aiter MI308 decoding PR, "Changes" -- are
 * left out: their inverse position is -1.  Unused slots of sorted_route_ids hold -1.
 * Output sizes: sorted_route_ids [P + E*(block_m-1)], expert_offsets [E+1],
 * tile_expert [P/block_m + E] (tile i covers rows [i*block_m, (i+1)*block_m), -1 past the
 * last tile), inverse_pos [P], n_tiles [1], with P = T*k.
 */
int oracle_align_sort(const int32_t *topk_ids, int T, int k, int E, int block_m,
                      int32_t *sorted_route_ids, int32_t *expert_offsets, int32_t *tile_expert,
                      int32_t *inverse_pos, int32_t *n_tiles)
{
    if (T < 0 || k <= 0 || E <= 0 || block_m <= 0)
        return -2;
    const long P = (long)T * k;
    const long slots = P + (long)E * (block_m - 1);
    const long tiles_cap = P / block_m + E;

    long *count = calloc((size_t)E, sizeof(long));
    long *next = calloc((size_t)E, sizeof(long));
    if (!count || !next) {
        free(count); free(next);
        return -4;
    }
    for (long r = 0; r < P; ++r) {
        int e = topk_ids[r];
        if (e >= 0 && e < E)
            count[e] += 1;
    }
    expert_offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        long padded = (count[e] + block_m - 1) / block_m * block_m;
        expert_offsets[e + 1] = (int32_t)(expert_offsets[e] + padded);
    }
    for (long s = 0; s < slots; ++s)
        sorted_route_ids[s] = -1;
    for (int e = 0; e < E; ++e)
        next[e] = expert_offsets[e];
    for (long r = 0; r < P; ++r) {
        int e = topk_ids[r];
        if (e >= 0 && e < E) {
            sorted_route_ids[next[e]] = (int32_t)r;
            inverse_pos[r] = (int32_t)next[e];
            next[e] += 1;
        } else {
            inverse_pos[r] = -1;
        }
    }
    const long tiles = expert_offsets[E] / block_m;
    *n_tiles = (int32_t)tiles;
    for (long i = 0; i < tiles_cap; ++i)
        tile_expert[i] = -1;
    for (int e = 0; e < E; ++e)
        for (long i = expert_offsets[e] / block_m; i < expert_offsets[e + 1] / block_m; ++i)
            tile_expert[i] = e;

    free(count); free(next);
    return 0;
}

/* ---------------------------------------------------------------- experts and combine
 *
 * For each requested token t (TileOPs "MoE" page, FusedMoEFwd / FusedMoESharedExpertFwd
 * tensor signatures w_gate_up [E, 2F, H], w_down [E, H, F], shared_w_gate_up [2S, H],
 * shared_w_down [H, S]; MoEGroupedGemmFwd activation=silu_and_mul; MoEPostPermuteFwd weighted
 * combine):
 *   for each route j with e = id[t,j] in [0, E)  (other ids are skipped, as the aiter MI308
 *   decoding PR does for -1 routes):
 *     u_f = sum_h x[t,h] W_gu[e, f, h],  v_f = sum_h x[t,h] W_gu[e, F+f, h]     (f < F)
 *     a_f = silu(u_f) * v_f,  silu(z) = z / (1 + exp(-z))
 *     y_h = sum_f a_f W_d[e, h, f]
 *     acc_h += w[t,j] * y_h
 *   with a shared expert (S > 0) the same SwiGLU MLP on S_gu / S_d is added, unweighted.
 *   out[t,h] = RNE_bf16(acc_h).
 * Readings: rows [0, F) of w_gate_up are the gate, rows [F, 2F) the up projection; no
 * intermediate is rounded.
 *
 * token_list (n_tokens entries, or NULL for tokens 0..n_tokens-1) selects which tokens to
 * evaluate; output row i belongs to token_list[i].  acc_out (double, may be NULL) receives the
 * unrounded sums, out_bf16 (may be NULL) the rounded output.  num_threads <= 0 uses the OpenMP
 * default.  The token loop is the only parallel loop; each token is computed by one thread in
 * a fixed order, so results do not depend on the thread count.
 */
/* IEEE binary16 bit pattern -> double (exact): 1 sign, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent 0 encodes subnormals f/1024 * 2^-14; exponent 31 is inf (f = 0) or NaN. */
static double f16_to_double(uint16_t b)
{
    const int sign = b >> 15, e = (b >> 10) & 31, f = b & 1023;
    double mag;
    if (e == 31)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -24);
    else
        mag = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -mag : mag;
}

/* double -> binary16 bit pattern, one rounding, round-to-nearest-even: the value is rounded to a
 * multiple of its binade's quantum (2^(E-10) for 2^E <= |v| < 2^(E+1), E >= -14; 2^-24 below
 * 2^-14), then encoded; a result past the largest finite 65504 is infinity. */
uint16_t oracle_double_to_f16(double v)
{
    if (v != v)
        return 0x7E00;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                 /* a in [2^(ex-1), 2^ex) */
    const int E = ex - 1;
    const double q = E < -14 ? ldexp(1.0, -24) : ldexp(1.0, E - 10);
    const double r = nearbyint(a / q) * q;
    if (r > 65504.0)
        return sign | 0x7C00;
    if (r < ldexp(1.0, -14))
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    int er;
    const double m = frexp(r, &er); /* r = m 2^er, m in [0.5, 1) */
    const int e_field = er - 1 + 15;
    const int frac = (int)((2.0 * m - 1.0) * 1024.0);
    return sign | (uint16_t)(e_field << 10) | (uint16_t)frac;
}

/* element type of the expert pass: 0 bf16, 1 f16 (both as 16-bit patterns) */
static double elem_to_double(uint16_t b, int dtype)
{
    return dtype == 1 ? f16_to_double(b) : bf16_to_double(b);
}

static void swiglu_mlp_accumulate(int dtype, const double *x, const uint16_t *w_gu,
                                  const uint16_t *w_d,
                                  int H, int F, double weight, double *a, double *acc)
{
    for (int f = 0; f < F; ++f) {
        const uint16_t *wg = w_gu + (size_t)f * H;
        const uint16_t *wu = w_gu + (size_t)(F + f) * H;
        double u = 0.0, v = 0.0;
        for (int h = 0; h < H; ++h) {
            u += x[h] * elem_to_double(wg[h], dtype);
            v += x[h] * elem_to_double(wu[h], dtype);
        }
        a[f] = u / (1.0 + exp(-u)) * v;
    }
    for (int h = 0; h < H; ++h) {
        const uint16_t *wd = w_d + (size_t)h * F;
        double y = 0.0;
        for (int f = 0; f < F; ++f)
            y += a[f] * elem_to_double(wd[f], dtype);
        acc[h] += weight * y;
    }
}

/* The experts and combine for element type dtype (0 bf16, 1 f16 -- the TileOPs "MoE" page's
 * FusedMoEFwd qwen3-235b-decode row runs both): inputs decoded exactly, everything in double,
 * the output rounded once to the same type (nearest even). */
int oracle_experts_dt(int dtype, const uint16_t *x, const uint16_t *w_gate_up,
                      const uint16_t *w_down, const int32_t *topk_ids, const float *topk_weights,
                      const uint16_t *shared_w_gate_up, const uint16_t *shared_w_down, int S,
                      int H, int E, int F, int k, const int32_t *token_list, int n_tokens,
                      double *acc_out, uint16_t *out_bits, int num_threads)
{
    if (dtype != 0 && dtype != 1)
        return -3;
    if (H <= 0 || E <= 0 || F <= 0 || k <= 0 || n_tokens < 0 || S < 0)
        return -2;
    if (S > 0 && (!shared_w_gate_up || !shared_w_down))
        return -1;
    const int a_len = (F > S) ? F : S;
    int status = 0;

#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
    for (int i = 0; i < n_tokens; ++i) {
        const int t = token_list ? token_list[i] : i;
        double *xd = malloc(sizeof(double) * (size_t)H);
        double *a = malloc(sizeof(double) * (size_t)(a_len > 0 ? a_len : 1));
        double *acc = calloc((size_t)H, sizeof(double));
        if (!xd || !a || !acc) {
            free(xd); free(a); free(acc);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -4;
            continue;
        }
        for (int h = 0; h < H; ++h)
            xd[h] = elem_to_double(x[(size_t)t * H + h], dtype);
        for (int j = 0; j < k; ++j) {
            const int e = topk_ids[(size_t)t * k + j];
            if (e < 0 || e >= E)
                continue;
            swiglu_mlp_accumulate(dtype, xd, w_gate_up + (size_t)e * 2 * F * H,
                                  w_down + (size_t)e * H * F, H, F,
                                  (double)topk_weights[(size_t)t * k + j], a, acc);
        }
        if (S > 0)
            swiglu_mlp_accumulate(dtype, xd, shared_w_gate_up, shared_w_down, H, S, 1.0, a, acc);
        for (int h = 0; h < H; ++h) {
            if (acc_out)
                acc_out[(size_t)i * H + h] = acc[h];
            if (out_bits)
                out_bits[(size_t)i * H + h] =
                    dtype == 1 ? oracle_double_to_f16(acc[h]) : oracle_double_to_bf16(acc[h]);
        }
        free(xd); free(a); free(acc);
    }
    return status;
}

/* The bf16 pass (the element type of every FusedMoEFwd workload but one). */
int oracle_experts(const uint16_t *x, const uint16_t *w_gate_up, const uint16_t *w_down,
                   const int32_t *topk_ids, const float *topk_weights,
                   const uint16_t *shared_w_gate_up, const uint16_t *shared_w_down, int S,
                   int H, int E, int F, int k, const int32_t *token_list, int n_tokens,
                   double *acc_out, uint16_t *out_bf16, int num_threads)
{
    return oracle_experts_dt(0, x, w_gate_up, w_down, topk_ids, topk_weights, shared_w_gate_up,
                             shared_w_down, S, H, E, F, k, token_list, n_tokens, acc_out,
                             out_bf16, num_threads);
}

/* ---------------------------------------------------------------- fp8 grouped GEMM */

/* OCP FP8 E4M3 ("e4m3fn") code -> double, from the format's definition: 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; there are
 * no infinities, and S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 * (TileOPs "MoE" page, MoEGroupedGemmFP8Fwd: dtype=fp8e4m3.) */
double oracle_fp8_e4m3_to_double(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* The grouped GEMM of the masked layout with block scales (TileOPs "MoE" page,
 * MoEGroupedGemmFP8Fwd: a [E, layout.max_m, K] e4m3 with a_scale [E, layout.max_m,
 * ceil_div(K, 128)] f32; b [E, N, K] e4m3 with b_scale [E, ceil_div(N, 128), ceil_div(K, 128)]
 * f32; layout_metadata [E] i32 = rows in use per expert):
 *   out[e, m, n] = RNE_bf16( sum_kb a_scale[e, m, kb] * b_scale[e, n / 128, kb]
 *                            * sum_{k in block kb} a[e, m, k] * b[e, n, k] )
 * for m < clamp(masked_m[e], 0, max_m); other rows are left as they are.  Reading: the scale
 * of a block multiplies the exact product sum of that block's decoded codes (the dequantised
 * operands' dot product), and the output is bf16.  Everything in double, one rounding. */
int oracle_grouped_gemm_fp8(const uint8_t *a, const float *a_scale, const uint8_t *b,
                            const float *b_scale, const int32_t *masked_m, int E, int max_m,
                            int N, int K, uint16_t *out, double *acc_out)
{
    if (E < 1 || max_m < 0 || N < 1 || K < 1)
        return -1;
    const int KB = (K + 127) / 128, NB = (N + 127) / 128;
    for (int e = 0; e < E; ++e) {
        int rows = masked_m[e];
        rows = rows < 0 ? 0 : (rows > max_m ? max_m : rows);
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic)
#endif
        for (int mn = 0; mn < rows * N; ++mn) {
            const int m = mn / N, n = mn % N;
            const uint8_t *ar = a + ((size_t)e * max_m + m) * K;
            const uint8_t *br = b + ((size_t)e * N + n) * K;
            double total = 0.0;
            for (int kb = 0; kb < KB; ++kb) {
                double block = 0.0;
                for (int k = kb * 128; k < K && k < kb * 128 + 128; ++k)
                    block += oracle_fp8_e4m3_to_double(ar[k]) * oracle_fp8_e4m3_to_double(br[k]);
                const double sa = a_scale[((size_t)e * max_m + m) * KB + kb];
                const double sb = b_scale[((size_t)e * NB + n / 128) * KB + kb];
                total += sa * sb * block;
            }
            const size_t o = ((size_t)e * max_m + m) * N + n;
            out[o] = oracle_double_to_bf16(total);
            if (acc_out)
                acc_out[o] = total;
        }
    }
    return 0;
}

/* double -> OCP e4m3 code: the finite e4m3 value nearest to v, ties to the code with an even
 * mantissa (round to nearest even), magnitudes beyond the largest finite value 448 saturate to
 * it (the format has no infinity; its one NaN pattern per sign is never produced).  Written from
 * the definition: the 127 non-negative finite codes are scanned for the nearest value.  NaN in
 * gives the NaN code 0x7F.  The sign of v (also of -0.0) is kept. */
uint8_t oracle_fp8_e4m3_encode(double v)
{
    if (v != v)
        return 0x7F;
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs(v);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(oracle_fp8_e4m3_to_double((uint8_t)c) - a);
        /* strictly nearer, or as near and even (codes ascend with value, so a tie is between c-1
         * and c, and the even one of the two wins) */
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* Per-token 1 x 128 group quantisation of bf16 activations to e4m3 with one f32 scale per group
 * (the a / a_scale pair of TileOPs "MoE" page, MoEGroupedGemmFP8Fwd: a_scale
 * [..., ceil_div(K, 128)] f32).  The pages give the scale's shape, not its rule; reading: the
 * group's scale is s = fl32(amax / 448) with amax the largest |x| of the group (s = 1 for an
 * all-zero group), and each value's code is the e4m3 nearest to fl32(x / s) (both divisions in
 * f32, as a quantised code is decided in the kernel's precision).  x [M, K] bf16 bits,
 * q [M, K] codes, scale [M, ceil(K / 128)]; the last group of a row may be partial. */
int oracle_quant_fp8_1x128(const uint16_t *x, int M, int K, uint8_t *q, float *scale)
{
    if (M < 0 || K < 1)
        return -1;
    const int G = (K + 127) / 128;
    for (int r = 0; r < M; ++r) {
        for (int g = 0; g < G; ++g) {
            const int k0 = 128 * g, k1 = k0 + 128 < K ? k0 + 128 : K;
            float amax = 0.0f;
            for (int k = k0; k < k1; ++k) {
                const float v = fabsf((float)bf16_to_double(x[(size_t)r * K + k]));
                amax = v > amax ? v : amax;
            }
            volatile float s = amax / 448.0f;
            if (amax == 0.0f)
                s = 1.0f;
            scale[(size_t)r * G + g] = s;
            for (int k = k0; k < k1; ++k) {
                volatile float t = (float)bf16_to_double(x[(size_t)r * K + k]) / s;
                q[(size_t)r * K + k] = oracle_fp8_e4m3_encode((double)t);
            }
        }
    }
    return 0;
}

/* The same block-scaled grouped GEMM on the contiguous layout (TileOPs "MoE" page,
 * layout=contiguous(packing=tight, metadata_kind=physical_psum)): the rows of all experts are
 * stacked in a [P, K], expert e owning rows [offsets[e], offsets[e+1]) (offsets [E+1], the
 * prefix sums of the rows per expert); a_scale [P, ceil(K/128)] f32.  Row r of expert e:
 *   out[r, n] = RNE_bf16( sum_kb a_scale[r, kb] * b_scale[e, n / 128, kb]
 *                         * sum_{k in block kb} a[r, k] * b[e, n, k] ).
 * Rows outside every expert's range are left as they are.  Everything in double. */
int oracle_grouped_gemm_fp8_contig(const uint8_t *a, const float *a_scale, const uint8_t *b,
                                   const float *b_scale, const int32_t *offsets, int E, int P,
                                   int N, int K, uint16_t *out, double *acc_out)
{
    if (E < 1 || P < 0 || N < 1 || K < 1)
        return -1;
    const int KB = (K + 127) / 128, NB = (N + 127) / 128;
    for (int e = 0; e < E; ++e) {
        int r0 = offsets[e], r1 = offsets[e + 1];
        r0 = r0 < 0 ? 0 : (r0 > P ? P : r0);
        r1 = r1 < r0 ? r0 : (r1 > P ? P : r1);
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic)
#endif
        for (int rn = 0; rn < (r1 - r0) * N; ++rn) {
            const int r = r0 + rn / N, n = rn % N;
            const uint8_t *ar = a + (size_t)r * K;
            const uint8_t *br = b + ((size_t)e * N + n) * K;
            double total = 0.0;
            for (int kb = 0; kb < KB; ++kb) {
                double block = 0.0;
                for (int k = kb * 128; k < K && k < kb * 128 + 128; ++k)
                    block += oracle_fp8_e4m3_to_double(ar[k]) * oracle_fp8_e4m3_to_double(br[k]);
                total += (double)a_scale[(size_t)r * KB + kb] *
                         (double)b_scale[((size_t)e * NB + n / 128) * KB + kb] * block;
            }
            out[(size_t)r * N + n] = oracle_double_to_bf16(total);
            if (acc_out)
                acc_out[(size_t)r * N + n] = total;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- MXFP4 weights */

/* OCP MX e2m1 code (4 bits) -> double: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent 0 encodes the subnormal m * 0.5; no infinities or NaN.  Magnitudes 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6. */
double oracle_e2m1_to_double(uint8_t code)
{
    const int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* OCP MX E8M0 scale byte -> double: 2^(s - 127); 255 is NaN. */
double oracle_e8m0_to_double(uint8_t s)
{
    return s == 255 ? NAN : ldexp(1.0, (int)s - 127);
}

/* MXFP4 weights -> double (the FlashInfer BF16-activation PR's 4-bit expert weights with 16-bit
 * activations, in the OCP MX layout): rows of K elements, two e2m1 codes per byte (element 2i
 * in the low nibble of byte i, reading of the packing order), one E8M0 scale per 32 consecutive
 * elements.  q [rows, K/2], scale [rows, K/32], out [rows, K]; K % 32 == 0. */
int oracle_mxfp4_dequant(const uint8_t *q, const uint8_t *scale, int rows, int K, double *out)
{
    if (rows < 0 || K < 32 || K % 32 != 0)
        return -1;
    for (int r = 0; r < rows; ++r)
        for (int k = 0; k < K; ++k) {
            const uint8_t byte = q[(size_t)r * (K / 2) + k / 2];
            const uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
            out[(size_t)r * K + k] = oracle_e2m1_to_double(code) *
                                     oracle_e8m0_to_double(scale[(size_t)r * (K / 32) + k / 32]);
        }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The roundings above applied to n values (the Python wrappers' array form). */
void oracle_double_to_bf16_n(const double *v, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_bf16(v[i]);
}

void oracle_double_to_f16_n(const double *v, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_f16(v[i]);
}
