// select.hip -- pooled-key block scoring and the query-aware / query-agnostic block selection.
//
// "NOSA: Native and Offloadable Sparse Attention":
//   [P1] paperlayer.ai summary §2.1 (query-aware selection scores by query-key similarity;
//        query-agnostic selection ranks cache units by a query-independent score and keeps a
//        fixed eviction pattern), §3.1 (budget split between the two subsets; sub-block mean
//        pooling then block max pooling), App. A (per step: select, fetch misses, attend),
//        App. E (adjacent selections overlap in at least ke entries);
//   [P4] gist.science technical summary, Method 1 (strict eviction: a unit left out at one step
//        is never selected again by the query-agnostic part; locality >= ke / k).
//
// Scoring.  Every lane builds its slice of the group query qs = sum of the row's G query heads
//   (fp32) straight from global memory, no barrier involved; with 256 threads the pooled-key
//   loads go out first and the query's loads (four heads at a time, all in flight) overlap them.
//   Eight lanes share one fp32 sub-block row (16-byte loads, 128 contiguous bytes per lane group
//   and load), reduce with three DPP adds and max-pool the block's sub-blocks with DPP and lane
//   swaps; each wave keeps four groups of eight rows in flight.
// Selection (one workgroup per row, in LDS).
//   Gamma_e: the sink and window blocks (if any), plus the best blocks by eviction score among
//            all other visible blocks (first step) or among the previous score-ranked members
//            and the blocks that left the window since (strict eviction);
//   Gamma_q: top-kq by block score among the visible blocks outside Gamma_e.
//   Exact top-k on unique 64-bit keys (order-preserving score bits, then the inverted block id,
//   so equal scores go to the lower id): rows of up to 64 blocks are ranked in registers, one
//   block per lane, with the counting shared by the waves; rows of up to 512 blocks rank every
//   candidate against all others in LDS, several lanes sharing each count; longer rows first drop
//   every key below a bound taken from the maxima of at most 256 chunks and rank the survivors
//   (radix select as the fallback).  Outputs are compacted in ascending block id.  The
//   selection's workgroup barriers wait for LDS only.
// Launch plans (chosen on the host).  "fused": one workgroup (256 or 1024 threads) scores a
//   whole row and selects from LDS.  "parts": several workgroups (256 threads, or 512 for rows
//   over 1024 blocks) score slices of a row into the workspace while one more workgroup per row
//   picks Gamma_e from the eviction scores; a second kernel (1024 threads per row) picks Gamma_q
//   (and, in the one-call offloaded step, then builds the row's cache map), unless the one-call
//   decode step ranks it inside its attention launch.  No workgroup ever
//   waits on another inside a kernel.
#include "cache_core.h"
#include "select_core.h"

namespace nosa {


// One workgroup scores a whole row, keeps the scores in LDS and selects.
template <typename T, int D, int SPB, int NT>
__global__ __launch_bounds__(NT) void score_select_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SelectShared<NT> sh;
    const int row = blockIdx.x;
    const RowLds L = carve<NT>(dyn, a.n_blocks);
    const bool short_row = a.n_blocks <= kWaveRowMax;
    float e[kEvPre];
    ev_load<NT>(a, row, e);
    const int pid = prev_agn(a, row, short_row ? (int)(threadIdx.x & 63) : (int)threadIdx.x);
    score_range<T, D, SPB, NT>(a, row, 0, a.n_blocks, L.sc, nullptr);
    ev_store<NT>(a, row, L, a.n_blocks, e);
    __syncthreads();
    if (short_row) {   // one block per lane, ranked in registers
        select_row64<NT>(a, row, L, nullptr, pid);
        return;
    }
    select_agnostic<NT>(a, row, L, sh, pid);
    select_query<NT>(a, row, L, sh, true);
}

// Grid rows x (parts + 1): one workgroup per row (absent in scores-only mode) computes the row's
// Gamma_e from the eviction scores and writes it to agn_state, while `parts` workgroups per row
// score slices of the row's blocks into the global score buffer.
template <typename T, int D, int SPB, int NT>
__global__ __launch_bounds__(NT) void score_part_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SelectShared<NT> sh;
    // Workgroups [0, rows) compute Gamma_e (none in scores-only mode); the scoring parts follow.
    // Dispatched first, the Gamma_e workgroups issue their eviction-score loads before the
    // scoring parts fill the memory queues with pooled keys.
    const int n_agn = a.scores_only ? 0 : a.rows;
    const bool agn_wg = (int)blockIdx.x < n_agn;
    const int idx = (int)blockIdx.x - n_agn;
    const int row = agn_wg ? (int)blockIdx.x : idx / a.parts, part = agn_wg ? a.parts : idx - row * a.parts;
    if (agn_wg) {
        const RowLds L = carve<NT>(dyn, a.n_blocks);
        float e[kEvPre];
        ev_load<NT>(a, row, e);
        const int pid = prev_agn(a, row, threadIdx.x);
        ev_store<NT>(a, row, L, a.n_blocks, e);
        // The ranking shares its CU with the scoring workgroups: give it issue priority.
        __builtin_amdgcn_s_setprio(2);
        select_agnostic<NT>(a, row, L, sh, pid);
        compact_outputs<NT>(a.n_blocks, L.inE, L.inE, a.ke > 0 ? a.agn + (size_t)row * a.ke : nullptr, a.ke,
                            nullptr, 0, sh);
        return;
    }
    const int blk_lo = part * a.blocks_per_part;
    const int blk_hi = min(a.n_blocks, blk_lo + a.blocks_per_part);
    score_range<T, D, SPB, NT>(a, row, blk_lo, blk_hi, nullptr, a.scores + (size_t)row * a.scores_stride);
}

// Gamma_q of row `row` scored by score_part_kernel (Gamma_e is already in agn_state), by the NT
// threads of one workgroup, in the dynamic LDS `dyn`; writes the row's selection.
template <int NT>
__device__ __forceinline__ void pick_row(const SelectArgs &a, int row, unsigned char *dyn, SelectShared<NT> &sh) {
    const int tid = threadIdx.x;
    const RowLds L = carve<NT>(dyn, a.n_blocks);
    const float *gscore = a.scores + (size_t)row * a.scores_stride;
    const int32_t *agn = a.agn + (size_t)row * a.ke;
    // the first NT Gamma_e ids are loaded together with the scores (one memory round trip) and
    // marked after the clear; any further ids are read after the barrier
    const int id0 = tid < a.ke ? agn[tid] : -1;
    scores_to_lds<NT>(gscore, a.n_blocks, L);
    __syncthreads();
    if (id0 >= 0 && id0 < a.n_blocks) L.inE[id0] = 1;
    for (int j = tid + NT; j < a.ke; j += NT) {
        const int id = agn[j];
        if (id >= 0 && id < a.n_blocks) L.inE[id] = 1;
    }
    __syncthreads();
    select_query<NT>(a, row, L, sh, false);
}

// Gamma_q of rows scored by score_part_kernel: one workgroup per row.
template <int NT>
__global__ __launch_bounds__(NT) void pick_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SelectShared<NT> sh;
    pick_row<NT>(a, blockIdx.x, dyn, sh);
}

// pick_kernel, then the row's cache map (cache_map_row, by wave 0) from the selection just written:
// the one-call offloaded step folds the map into the pick instead of launching it on its own.
template <int NT>
__global__ __launch_bounds__(NT) void pick_map_kernel(SelectArgs a, CacheArgs c) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SelectShared<NT> sh;
    pick_row<NT>(a, blockIdx.x, dyn, sh);
    // the row's selection (global stores of every wave) is visible to the workgroup after the
    // barrier; the pick's LDS is free again
    __syncthreads();
    if (threadIdx.x < 64) cache_map_row(c, blockIdx.x, threadIdx.x, dyn);
}

template <class K>
static hipError_t allow_lds(K kern, size_t dyn) {
    if (dyn <= 48 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
}

template <typename T, int D, int SPB>
static hipError_t launch_select_t(const SelectArgs &a, int rows, int fused_threads, int part_threads,
                                  hipStream_t st) {
    hipError_t e;
    if (a.parts == 1 && !a.scores_only) {
        if (fused_threads == 1024) {
            const size_t dyn = row_lds_bytes<1024>(a.n_blocks);
            auto kern = score_select_kernel<T, D, SPB, 1024>;
            if ((e = allow_lds(kern, dyn)) != hipSuccess) return e;
            kern<<<dim3((unsigned)rows), dim3(1024), dyn, st>>>(a);
        } else {
            const size_t dyn = row_lds_bytes<256>(a.n_blocks);
            auto kern = score_select_kernel<T, D, SPB, 256>;
            if ((e = allow_lds(kern, dyn)) != hipSuccess) return e;
            kern<<<dim3((unsigned)rows), dim3(256), dyn, st>>>(a);
        }
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)(rows * (a.parts + (a.scores_only ? 0 : 1)));
    if (part_threads == 512) {
        const size_t dyn0 = a.scores_only ? 0 : row_lds_bytes<512>(a.n_blocks);
        if ((e = allow_lds(score_part_kernel<T, D, SPB, 512>, dyn0)) != hipSuccess) return e;
        score_part_kernel<T, D, SPB, 512><<<dim3(grid), dim3(512), dyn0, st>>>(a);
    } else {
        const size_t dyn0 = a.scores_only ? 0 : row_lds_bytes<256>(a.n_blocks);
        if ((e = allow_lds(score_part_kernel<T, D, SPB, 256>, dyn0)) != hipSuccess) return e;
        score_part_kernel<T, D, SPB, 256><<<dim3(grid), dim3(256), dyn0, st>>>(a);
    }
    if ((e = hipGetLastError()) != hipSuccess || a.scores_only || a.no_pick) return e;
    // 1024 threads even for short rows: with 256, each thread ranks a whole candidate and the pick
    // takes longer (measured on MI355X at 256 blocks per row: 18.8 vs 17.1 us for the selection).
    const size_t dyn = row_lds_bytes<1024>(a.n_blocks);
    if ((e = allow_lds(pick_kernel<1024>, dyn)) != hipSuccess) return e;
    pick_kernel<1024><<<dim3((unsigned)rows), dim3(1024), dyn, st>>>(a);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_select_d(int spb, const SelectArgs &a, int rows, int fused_threads, int part_threads,
                                  hipStream_t st) {
    switch (spb) {
        case 1: return launch_select_t<T, D, 1>(a, rows, fused_threads, part_threads, st);
        case 2: return launch_select_t<T, D, 2>(a, rows, fused_threads, part_threads, st);
        case 4: return launch_select_t<T, D, 4>(a, rows, fused_threads, part_threads, st);
        default: return launch_select_t<T, D, 8>(a, rows, fused_threads, part_threads, st);
    }
}

hipError_t launch_pick_map(const SelectArgs &a, const CacheArgs &c, int rows, hipStream_t st) {
    size_t dyn = row_lds_bytes<1024>(a.n_blocks);
    if (cache_map_lds_bytes(c.C, c.k) > dyn) dyn = cache_map_lds_bytes(c.C, c.k);
    hipError_t e = allow_lds(pick_map_kernel<1024>, dyn);
    if (e != hipSuccess) return e;
    pick_map_kernel<1024><<<dim3((unsigned)rows), dim3(1024), dyn, st>>>(a, c);
    return hipGetLastError();
}

hipError_t launch_select(int dtype, int d, int spb, const SelectArgs &a, int rows, int fused_threads,
                         int part_threads, hipStream_t st) {
    if (dtype == 1)
        return d == 128 ? launch_select_d<uint16_t, 128>(spb, a, rows, fused_threads, part_threads, st)
                        : launch_select_d<uint16_t, 64>(spb, a, rows, fused_threads, part_threads, st);
    return d == 128 ? launch_select_d<float, 128>(spb, a, rows, fused_threads, part_threads, st)
                    : launch_select_d<float, 64>(spb, a, rows, fused_threads, part_threads, st);
}

}  // namespace nosa
