// moe_route_dev.h -- per-token top-k / grouped top-k routing on one wave (gfx950, wave64).
//
// Computes what the TileOPs "MoE" page's FusedTopKFwd op computes (gating_output [T,E] f32,
// top_k, renormalize, scoring_func, correction_bias [E] f32, num_expert_group, topk_group,
// routed_scaling_factor):
//   - selection keys in f32: the logit for softmax; f32(f32(sigmoid(g)) + bias) for sigmoid,
//     the sigmoid evaluated in double and rounded once;
//   - grouped top-k: a group scores the f32 sum of its two largest keys, the topk_group best
//     groups stay eligible (ties to the lower group);
//   - top-k by key over eligible experts, ties to the lower expert index, ids in descending
//     key order;
//   - weights: unbiased scores of the chosen experts in double, renormalised if asked, times
//     the routed scaling factor, rounded to f32 once.
//
// Layout: lane l of a token's wave holds experts e = 64*i + l (i < SLOTS), so the row load is
// coalesced.  Selection runs on 64-bit keys (order-preserving f32 bits << 32 | ~index): the
// wave maximum is the best expert with the lower-index tie-break built in, so every step is
// exact integer comparison and the result is bit-identical to any correct implementation.
#pragma once

#include "moe_device.h"

namespace moe_route_dev {


__device__ __forceinline__ uint32_t ordered_bits(float f)
{
    if (f == 0.0f)
        f = 0.0f;  // -0 and +0 are the same key
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t select_key(float key, int idx)
{
    return ((uint64_t)ordered_bits(key) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

__device__ __forceinline__ int select_index(uint64_t key)
{
    return (int)(0xffffffffu - (uint32_t)key);
}

// v of the lane that DPP control CTRL selects within this lane's row of 16 (every lane of the
// row has a source under the controls used here)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum over the 64 lanes, returned to every lane.  Within each row of 16 lanes four DPP
// exchanges (lane ^ 1, lane ^ 2, then the mirror images within 8 and within 16 lanes) leave the
// row's maximum in all its lanes; the four rows' maxima are then read as scalars.  DPP moves
// run on the VALU, not through the LDS crossbar that a general lane shuffle takes.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
    v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
    return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)),
                   max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

// Routes token t with one wave (lane = lane index).  s_key: E floats of LDS owned by this wave
// (used when n_group > 1).  ids_copy: optional second destination of the ids (LDS).
template <int SLOTS>
__device__ __forceinline__ void route_token(
    const float *__restrict__ gating, const float *__restrict__ bias, int t, int E, int k,
    int sigmoid, int renormalize, int n_group, int topk_group, float rsf, float *s_key, int lane,
    int32_t *__restrict__ ids_out, float *__restrict__ weights_out, int32_t *ids_copy)
{
    const float *g = gating + (size_t)t * E;

    float key[SLOTS];
    double sig[SLOTS];      // sigmoid: the unbiased score in double, kept for the weights
    uint32_t eligible = 0;  // bit i: slot i holds an eligible expert
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
        const int e = 64 * i + lane;
        key[i] = 0.0f;
        sig[i] = 0.0;
        if (e < E) {
            const float gv = g[e];
            if (sigmoid) {
                sig[i] = 1.0 / (1.0 + exp(-(double)gv));
                key[i] = (float)sig[i] + (bias ? bias[e] : 0.0f);
            } else {
                key[i] = gv;
            }
            eligible |= 1u << i;
        }
    }

    const int gs = n_group > 1 ? E / n_group : 0;
    if (n_group > 1 && gs <= 64 && (gs & (gs - 1)) == 0 && n_group <= 64) {
        // Groups of a power-of-two size up to 64 lie within one slot's lanes: the two largest
        // keys of each group by a butterfly over its gs lanes, merging (largest, second) pairs,
        // all slots at once.  A group scores b1 + b2 (b1 alone for single-expert groups), as
        // the scan below; which of two equal keys is "first" does not change the sum.
        float b1[SLOTS], b2[SLOTS];
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            // a NaN key never counts (the scan's strict comparisons skip it too)
            b1[i] = (64 * i + lane < E && key[i] == key[i]) ? key[i] : -INFINITY;
            b2[i] = -INFINITY;
        }
        for (int off = 1; off < gs; off <<= 1) {
#pragma unroll
            for (int i = 0; i < SLOTS; ++i) {
                const float o1 = __shfl_xor(b1[i], off);
                const float o2 = __shfl_xor(b2[i], off);
                const float hi = fmaxf(b1[i], o1), lo = fminf(b1[i], o1);
                b2[i] = fmaxf(lo, fmaxf(b2[i], o2));
                b1[i] = hi;
            }
        }
        // group gi = (64 * i + lane) / gs: its pair sits in every lane of its segment; lane
        // gi < n_group gathers group gi's from the segment's first lane (every lane runs the
        // shuffles; the others discard the result)
        const int e0 = lane < n_group ? lane * gs : 0;  // first expert of group `lane`
        const int slot = e0 >> 6, src = e0 & 63;
        float s1 = -INFINITY, s2 = -INFINITY;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const float v1 = __shfl(b1[i], src), v2 = __shfl(b2[i], src);
            if (i == slot) {
                s1 = v1;
                s2 = v2;
            }
        }
        uint64_t gkey = 0;
        if (lane < n_group)
            gkey = select_key(gs == 1 ? s1 : s1 + s2, lane);
        uint64_t kept = 0;  // bit gi: group gi kept
        for (int n = 0; n < topk_group; ++n) {
            const uint64_t best = wave_max_u64(gkey);
            const int gi = select_index(best);
            kept |= 1ull << gi;
            if (lane == gi)
                gkey = 0;
        }
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int e = 64 * i + lane;
            if (e < E && !((kept >> (e / gs)) & 1ull))
                eligible &= ~(1u << i);
        }
    } else if (n_group > 1) {
        // group scores: lane gi < n_group scans its contiguous group of E/n_group experts
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int e = 64 * i + lane;
            if (e < E)
                s_key[e] = key[i];
        }
        moe_wave_sync();
        uint64_t gkey = 0;
        if (lane < n_group) {
            float b1 = -INFINITY, b2 = -INFINITY;
            for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
                const float v = s_key[e];
                if (v > b1) {
                    b2 = b1;
                    b1 = v;
                } else if (v > b2) {
                    b2 = v;
                }
            }
            const float score = (gs == 1) ? b1 : b1 + b2;
            gkey = select_key(score, lane);
        }
        uint64_t kept = 0;  // bit gi: group gi kept
        for (int n = 0; n < topk_group; ++n) {
            const uint64_t best = wave_max_u64(gkey);
            const int gi = select_index(best);
            kept |= 1ull << gi;
            if (lane == gi)
                gkey = 0;
        }
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int e = 64 * i + lane;
            if (e < E && !((kept >> (e / gs)) & 1ull))
                eligible &= ~(1u << i);
        }
    }

    // top-k: k rounds of a wave-wide maximum over the remaining eligible experts
    int my_id = -1;
    int first_id = 0;  // wave-uniform: the best expert overall
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            if ((eligible >> i) & 1u) {
                const uint64_t c = select_key(key[i], 64 * i + lane);
                best = c > best ? c : best;
            }
        }
        best = wave_max_u64(best);
        const int e = select_index(best);
        if ((e & 63) == lane)
            eligible &= ~(1u << (e >> 6));
        if (lane == j)
            my_id = e;
        if (j == 0)
            first_id = e;
    }

    // weights: lane j < k owns route j.  Softmax keys are the logits themselves, so the logits
    // the weights need come from the registers that hold them (no second read of the row).
    // Softmax is never grouped, so the first chosen expert holds the row's largest logit.
    double m = 0.0;
    if (!sigmoid) {
        const int fe = __builtin_amdgcn_readfirstlane(first_id);  // wave-uniform already
        float mv = 0.0f;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i)
            if (i == (fe >> 6))
                mv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key[i]), fe & 63));
        m = (double)mv;
    }
    double s = 0.0;
    if (sigmoid) {
        // the chosen expert's sigmoid from the lane and slot that computed it
        const int src = my_id < 0 ? 0 : (my_id & 63), slot = my_id < 0 ? 0 : (my_id >> 6);
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const double v = __shfl(sig[i], src);
            if (i == slot && lane < k)
                s = v;
        }
    } else {
        const int src = my_id < 0 ? 0 : (my_id & 63), slot = my_id < 0 ? 0 : (my_id >> 6);
        float gl = 0.0f;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const float v = __shfl(key[i], src);
            if (i == slot)
                gl = v;
        }
        if (lane < k)
            s = exp((double)gl - m);
    }
    double denom = 1.0;
    if (renormalize) {
        denom = wave_sum_f64(s);
    } else if (!sigmoid) {
        // full softmax denominator over all experts
        double z = 0.0;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int e = 64 * i + lane;
            if (e < E)
                z += exp((double)key[i] - m);
        }
        denom = wave_sum_f64(z);
    }
    if (lane < k) {
        const double w = s / denom * (double)rsf;
        ids_out[(size_t)t * k + lane] = my_id;
        weights_out[(size_t)t * k + lane] = (float)w;
        if (ids_copy)
            ids_copy[(size_t)t * k + lane] = my_id;
    }
}


}  // namespace moe_route_dev
