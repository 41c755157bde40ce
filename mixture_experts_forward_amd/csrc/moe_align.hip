// moe_align.hip -- expert histogram, padded prefix sum and stable permutation of routes.
//
// Computes the expert-contiguous route order of the TileOPs "MoE" page's MoEPermuteAlignFwd
// (topk_ids [T,K] i32 -> per-expert prefix sums of the contiguous layout) together with the
// inverse map of its MoEPostPermuteFwd (inverse_indices [T*K]): every expert's routes in
// increasing route index r = t*k + j, each expert's segment padded up to block_m rows.
//
// Rounds of 1024 routes (one workgroup of 16 waves) do the stable scatter: a route's row = its
// expert's running base + the count of the same expert in earlier waves of the round (per-wave
// histograms packed as two 16-bit counters per word) + its rank among earlier lanes of its own
// wave (LDS broadcast compare).  Two drivers:
//   - one workgroup for everything (the public moe_align_sort, and up to 1024 routes): LDS
//     histogram with integer atomics (order-independent, so deterministic), block-wide scan of
//     the padded counts (expert_offsets, tile_expert, n_tiles, the -1 fill of padding slots),
//     then the rounds in order;
//   - three launches over chunks of 1024 routes when a caller provides a count table of
//     chunks x E ints (the fused pass): per-chunk histograms, one workgroup that turns them
//     into per-chunk prefix counts per expert and lays out the padded segments, then all
//     chunks' rounds at once.
// Every slot of sorted_route_ids and tile_expert is written exactly once.
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_plan.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxExperts = 1024;
static_assert(kThreads == moe::kAlignChunk, "a chunk of the chunked align is one workgroup");

struct AlignSmem {
    int count[kMaxExperts];
    int base[kMaxExperts];
    int first[kMaxExperts];  // expert's first row (its segment start)
    uint32_t hist[kWaves][kMaxExperts / 2];  // two 16-bit counters per word
    alignas(16) int round_ids[kThreads];
    int wave_total[kWaves];
    int wave_cost[kWaves];
    int total;
};

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off);
        if (lane >= off)
            v += o;
    }
    return v;
}

// Padded exclusive scan of sm.count[0..E) (thread e owns expert e): writes expert_offsets,
// tile_expert, n_tiles and the -1 padding of sorted_ids; leaves each expert's first row in
// sm.base (sm.count unchanged).
__device__ __forceinline__ void write_schedule(int E, int bm, int c, int excl_rows,
                                               moe::TileSchedule *__restrict__ sched,
                                               AlignSmem &sm);

// The per-XCD tile ranges of the layout (moe::TileSchedule): thread e < E holds expert e's
// routed rows c and its first padded row excl_rows; sm.total is the padded row count.  Each
// expert's cost (its row tiles' 5*bm/4 + their rows) is scanned; range boundary p (1..7) falls
// in the expert whose cost interval holds p/8 of the total, at the matching fraction of its row
// tiles.  Also zeroes the counters.
__device__ __forceinline__ void write_schedule(int E, int bm, int c, int excl_rows,
                                               moe::TileSchedule *__restrict__ sched,
                                               AlignSmem &sm)
{
    constexpr int P = moe::kSchedParts;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int te = (c + bm - 1) / bm;  // row tiles of expert tid (0 past E)
    const int cost = te * (5 * bm / 4) + c;
    int incl = wave_inclusive_scan(cost, lane);
    if (lane == 63)
        sm.wave_cost[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
        before += w < wv ? sm.wave_cost[w] : 0;
        total += sm.wave_cost[w];
    }
    incl += before;
    const int excl = incl - cost;
    const float row_tiles = (float)(sm.total / bm);
    if (tid <= P)
        sched->queue[tid] = 0;
    if (total == 0) {
        if (tid <= P)
            sched->bounds[tid] = 0.0f;
        return;
    }
    if (tid == 0) {
        sched->bounds[0] = 0.0f;
        sched->bounds[P] = row_tiles;
    }
    if (tid < E && cost > 0) {
        for (int p = 1; p < P; ++p) {
            const double target = (double)total * p / P;
            if ((double)excl < target && target <= (double)incl) {
                const double f = (target - excl) / cost;
                sched->bounds[p] = (float)(excl_rows / bm + f * te);
            }
        }
    }
}

__device__ __forceinline__ void scan_layout(int E, int bm, int slots, int tiles_cap,
                                            int32_t *__restrict__ sorted_ids,
                                            int32_t *__restrict__ offsets,
                                            int32_t *__restrict__ tile_expert,
                                            int32_t *__restrict__ n_tiles,
                                            moe::TileSchedule *__restrict__ sched, bool balanced,
                                            AlignSmem &sm)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int c = (tid < E) ? sm.count[tid] : 0;
    const int padded = (c + bm - 1) / bm * bm;
    int incl = wave_inclusive_scan(padded, lane);
    if (lane == 63)
        sm.wave_total[wv] = incl;
    __syncthreads();
    int before_wave = 0;
    for (int w = 0; w < wv; ++w)
        before_wave += sm.wave_total[w];
    incl += before_wave;
    const int excl = incl - padded;
    if (tid < E) {
        offsets[tid] = excl;
        sm.base[tid] = excl;
        sm.first[tid] = excl;
    }
    if (tid == E - 1) {
        offsets[E] = incl;
        *n_tiles = incl / bm;
        sm.total = incl;
    }
    __syncthreads();
    if (sched)
        write_schedule(E, bm, c, excl, sched, sm);
    // padding rows and tile table of expert e, by wave e % 16 (lanes share the slots)
    for (int e = wv; e < E; e += kWaves) {
        const int b = sm.base[e], ce = sm.count[e];
        const int pe = (ce + bm - 1) / bm * bm;
        if (balanced && ce > 0) {
            // tile j's rows are a prefix of it: q + 1 rows in the first rem tiles, q after
            const int te = pe / bm, q = ce / te, rem = ce % te;
            for (int j = 0; j < te; ++j) {
                const int t0 = b + j * bm;
                for (int s = t0 + q + (j < rem ? 1 : 0) + lane; s < t0 + bm; s += 64)
                    sorted_ids[s] = -1;
            }
        } else {
            for (int s = b + ce + lane; s < b + pe; s += 64)
                sorted_ids[s] = -1;
        }
        for (int i = b / bm + lane; i < (b + pe) / bm; i += 64)
            tile_expert[i] = e;
    }
    const int total = sm.total;
    for (int s = total + tid; s < slots; s += kThreads)
        sorted_ids[s] = -1;
    for (int i = total / bm + tid; i < tiles_cap; i += kThreads)
        tile_expert[i] = -1;
}

// Row of an expert's route of rank p (0-based, in route order) in the balanced layout: the
// expert's ce routes fill its te = ceil(ce / bm) tiles as evenly as they can (the first
// ce % te tiles one row more), each tile's rows a prefix of it.
__device__ __forceinline__ int balanced_row(int first, int p, int ce, int bm)
{
    const int te = (ce + bm - 1) / bm;
    const int q = ce / te, rem = ce % te;
    const int big = (q + 1) * rem;  // routes in the first rem tiles
    const int j = p < big ? p / (q + 1) : rem + (p - big) / q;
    const int start = p < big ? j * (q + 1) : big + (j - rem) * q;
    return first + j * bm + (p - start);
}

// Stable scatter of routes [r0, r0 + 1024): route r of expert e goes to row sm.base[e] + (its
// rank among this round's routes of e), or with bal (the tile height) to the balanced row of
// that rank (sm.first and sm.count: the expert's first row and route count).  With advance,
// sm.base moves past the round's routes.  sm.hist must be zero on entry and is zero again on
// return.
__device__ __forceinline__ void scatter_round(const int32_t *__restrict__ ids, int P, int E,
                                              int r0, bool advance, int bal,
                                              int32_t *__restrict__ sorted_ids,
                                              int32_t *__restrict__ inverse, AlignSmem &sm)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int half_words = (E + 1) / 2;
    const int r = r0 + tid;
    int e = (r < P) ? ids[r] : -1;
    const bool valid = (e >= 0 && e < E);
    if (!valid)
        e = -1;
    sm.round_ids[tid] = e;
    __syncthreads();
    int rank = 0;
    if (valid) {
        const int4 *w4 = reinterpret_cast<const int4 *>(&sm.round_ids[wv * 64]);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int4 v = w4[q];
            rank += (4 * q + 0 < lane && v.x == e);
            rank += (4 * q + 1 < lane && v.y == e);
            rank += (4 * q + 2 < lane && v.z == e);
            rank += (4 * q + 3 < lane && v.w == e);
        }
        atomicAdd(&sm.hist[wv][e >> 1], 1u << ((e & 1) * 16));
    }
    __syncthreads();
    if (valid) {
        int before = 0;
        for (int w = 0; w < wv; ++w)
            before += (sm.hist[w][e >> 1] >> ((e & 1) * 16)) & 0xffff;
        int pos = sm.base[e] + before + rank;
        if (bal)
            pos = balanced_row(sm.first[e], pos - sm.first[e], sm.count[e], bal);
        sorted_ids[pos] = r;
        inverse[r] = pos;
    } else if (r < P) {
        inverse[r] = -1;
    }
    __syncthreads();
    if (advance && tid < E) {
        int sum = 0;
        for (int w = 0; w < kWaves; ++w)
            sum += (sm.hist[w][tid >> 1] >> ((tid & 1) * 16)) & 0xffff;
        sm.base[tid] += sum;
    }
    __syncthreads();
    for (int x = tid; x < kWaves * half_words; x += kThreads)
        sm.hist[x / half_words][x % half_words] = 0;
    // the next round's first barrier orders this clear before its atomics
}

// The whole align/sort by one 1024-thread workgroup.
__device__ __forceinline__ void align_block(const int32_t *__restrict__ ids, int P, int E, int bm,
                                            int slots, int tiles_cap,
                                            int32_t *__restrict__ sorted_ids,
                                            int32_t *__restrict__ offsets,
                                            int32_t *__restrict__ tile_expert,
                                            int32_t *__restrict__ inverse,
                                            int32_t *__restrict__ n_tiles,
                                            moe::TileSchedule *__restrict__ sched, bool balanced,
                                            AlignSmem &sm)
{
    const int tid = threadIdx.x;
    const int half_words = (E + 1) / 2;
    if (tid < E)
        sm.count[tid] = 0;
    for (int x = tid; x < kWaves * half_words; x += kThreads)
        sm.hist[x / half_words][x % half_words] = 0;
    __syncthreads();
    for (int r = tid; r < P; r += kThreads) {
        const int e = ids[r];
        if (e >= 0 && e < E)
            atomicAdd(&sm.count[e], 1);
    }
    __syncthreads();
    scan_layout(E, bm, slots, tiles_cap, sorted_ids, offsets, tile_expert, n_tiles, sched,
                balanced, sm);
    for (int r0 = 0; r0 < P; r0 += kThreads)
        scatter_round(ids, P, E, r0, true, balanced ? bm : 0, sorted_ids, inverse, sm);
}

// Chunked driver, launch 1: histogram of chunk b (routes [1024b, 1024b + 1024)) into
// counts[b*E + e].
__global__ __launch_bounds__(kThreads) void k_align_hist(const int32_t *__restrict__ ids, int P,
                                                         int E, int32_t *__restrict__ counts)
{
    __shared__ int cnt[kMaxExperts];
    const int tid = threadIdx.x;
    if (tid < E)
        cnt[tid] = 0;
    __syncthreads();
    const int r = blockIdx.x * kThreads + tid;
    if (r < P) {
        const int e = ids[r];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid < E)
        counts[blockIdx.x * E + tid] = cnt[tid];
}

// Chunked driver, launch 2 (one workgroup): per-expert totals and the padded layout;
// counts[b*E + e] becomes the number of expert e's routes in chunks before b (balanced: and
// counts[chunks*E + e] its total).  The counts are read 16 chunks at a time so that their
// loads overlap.
__global__ __launch_bounds__(kThreads) void k_align_scan(int32_t *__restrict__ counts,
                                                         int chunks, int E, int bm, int slots,
                                                         int tiles_cap,
                                                         int32_t *__restrict__ sorted_ids,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ tile_expert,
                                                         int32_t *__restrict__ n_tiles,
                                                         moe::TileSchedule *__restrict__ sched,
                                                         int balanced)
{
    constexpr int kBatch = 16;
    __shared__ AlignSmem sm;
    const int tid = threadIdx.x;
    if (tid < E) {
        int run = 0;
        for (int b0 = 0; b0 < chunks; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                c[u] = (b0 + u < chunks) ? counts[(b0 + u) * E + tid] : 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (b0 + u < chunks)
                    counts[(b0 + u) * E + tid] = run;
                run += c[u];
            }
        }
        sm.count[tid] = run;
        if (balanced)
            counts[(size_t)chunks * E + tid] = run;
    }
    __syncthreads();
    scan_layout(E, bm, slots, tiles_cap, sorted_ids, offsets, tile_expert, n_tiles, sched,
                balanced != 0, sm);
}

// Chunked driver, launch 3: the round of chunk b, its routes of expert e starting at rank
// (routes of e in earlier chunks) of the expert's rows from expert_offsets[e] on (bal: the
// tile height of the balanced layout, whose totals follow the chunk table).
__global__ __launch_bounds__(kThreads) void k_align_scatter(const int32_t *__restrict__ ids,
                                                            int P, int E, int chunks,
                                                            const int32_t *__restrict__ counts,
                                                            const int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted_ids,
                                                            int32_t *__restrict__ inverse,
                                                            int bal)
{
    __shared__ AlignSmem sm;
    const int tid = threadIdx.x;
    const int half_words = (E + 1) / 2;
    if (tid < E) {
        sm.first[tid] = offsets[tid];
        sm.base[tid] = offsets[tid] + counts[blockIdx.x * E + tid];
        sm.count[tid] = bal ? counts[(size_t)chunks * E + tid] : 0;
    }
    for (int x = tid; x < kWaves * half_words; x += kThreads)
        sm.hist[x / half_words][x % half_words] = 0;
    __syncthreads();
    scatter_round(ids, P, E, blockIdx.x * kThreads, false, bal, sorted_ids, inverse, sm);
}

__global__ __launch_bounds__(kThreads) void k_align_sort(
    const int32_t *__restrict__ ids, int P, int E, int bm, int slots, int tiles_cap,
    int32_t *__restrict__ sorted_ids, int32_t *__restrict__ offsets,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ inverse,
    int32_t *__restrict__ n_tiles, moe::TileSchedule *__restrict__ sched, int balanced)
{
    __shared__ AlignSmem sm;
    align_block(ids, P, E, bm, slots, tiles_cap, sorted_ids, offsets, tile_expert, inverse,
                n_tiles, sched, balanced != 0, sm);
}

}  // namespace

namespace moe {

void launch_align_sort(const int32_t *ids, int P, int E, int block_m, int32_t *sorted_ids,
                       int32_t *offsets, int32_t *tile_expert, int32_t *inverse, int32_t *n_tiles,
                       int32_t *scratch, hipStream_t stream, TileSchedule *sched, bool balanced)
{
    const int slots = P + E * (block_m - 1);
    const int tiles_cap = P / block_m + E;
    const int bal = balanced ? 1 : 0;
    if (scratch == nullptr || P <= kThreads) {
        hipLaunchKernelGGL(k_align_sort, dim3(1), dim3(kThreads), 0, stream, ids, P, E, block_m,
                           slots, tiles_cap, sorted_ids, offsets, tile_expert, inverse, n_tiles,
                           sched, bal);
        return;
    }
    const int chunks = (P + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_align_hist, dim3(chunks), dim3(kThreads), 0, stream, ids, P, E,
                       scratch);
    hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(kThreads), 0, stream, scratch, chunks, E,
                       block_m, slots, tiles_cap, sorted_ids, offsets, tile_expert, n_tiles,
                       sched, bal);
    hipLaunchKernelGGL(k_align_scatter, dim3(chunks), dim3(kThreads), 0, stream, ids, P, E,
                       chunks, scratch, offsets, sorted_ids, inverse, balanced ? block_m : 0);
}

}  // namespace moe
