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
// Scoring (256 threads, 4 waves).  The group query qs = sum of the row's G query heads (fp32) is
//   dotted with every pooled sub-block key; eight lanes share one fp32 sub-block row (16-byte
//   loads, 128 contiguous bytes per lane group and load), reduce with three DPP adds and
//   max-pool the block's sub-blocks with DPP / lane swaps.  Each wave keeps four row groups of
//   loads in flight.
// Selection (one workgroup per row, in LDS).
//   Gamma_e: top-ke by eviction score among all visible blocks (first step) or among the
//            previous Gamma_e plus the newly visible blocks (strict eviction);
//   Gamma_q: top-kq by block score among the visible blocks outside Gamma_e.
//   Exact top-k on unique 64-bit keys (order-preserving score bits, then the inverted block id,
//   so equal scores go to the lower id): rows of up to 512 blocks rank every candidate against
//   all others in one pass; longer rows use a radix select (four 8-bit digit passes over an LDS
//   histogram) with the id tie rule applied by a scan.  Outputs are compacted in ascending id.
// Launch plans.  A row that one workgroup scores (parts == 1) is scored and selected by that
//   workgroup ("fused").  Longer rows are scored by `parts` workgroups into the workspace and
//   selected by a second kernel with one workgroup per row; no cross-workgroup synchronisation
//   happens inside a kernel.
#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;          // sub-block groups per wave kept in flight
constexpr int kRankMaxBlocks = 512; // rows up to this length use the one-pass rank selection

struct SelectShared {
    uint32_t hist[256];
    int scan[4];
    int bcast[4];
};

__device__ __forceinline__ uint64_t composite_key(uint32_t k, int id) {
    return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// Marks the kk best candidates (key descending, id ascending) in mark[0..n).
// keybuf: LDS scratch of n uint64 (used by the rank path).
template <class KeyF, class CandF>
__device__ void topk_mark(int n, int kk, KeyF key, CandF cand, uint8_t *mark, uint64_t *keybuf, SelectShared &sh) {
    if (kk <= 0) return;
    const int tid = threadIdx.x;
    if (n <= kRankMaxBlocks) {
        // rank of each candidate among all candidates; unique keys, non-candidates hold 0
        for (int i = tid; i < n; i += kThreads) keybuf[i] = cand(i) ? composite_key(key(i), i) : 0ull;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint64_t ki = keybuf[i];
            if (ki == 0ull) continue;
            int r = 0;
            for (int j = 0; j < n; ++j) r += keybuf[j] > ki ? 1 : 0;
            if (r < kk) mark[i] = 1;
        }
        __syncthreads();
        return;
    }
    uint32_t prefix = 0, pmask = 0;
    int need = kk;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        sh.hist[tid] = 0u;
        if (tid == 0) { sh.bcast[0] = 0; sh.bcast[1] = 0; }
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            if (cand(i)) {
                const uint32_t kv = key(i);
                if ((kv & pmask) == prefix) atomicAdd(&sh.hist[(kv >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        const int d = 255 - tid;
        const int cnt = (int)sh.hist[d];
        const int ge = block_incl_scan256(cnt, sh.scan);   // candidates with digit >= d
        const int gt = ge - cnt;
        if (gt < need && need <= ge) { sh.bcast[0] = d; sh.bcast[1] = gt; }
        __syncthreads();
        prefix |= (uint32_t)sh.bcast[0] << shift;
        pmask |= 0xFFu << shift;
        need -= sh.bcast[1];
        __syncthreads();
    }
    // prefix is the kk-th largest key; take every larger key and the `need` lowest ids equal to it.
    const uint32_t T = prefix;
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int eq = 0;
    for (int i = lo; i < hi; ++i)
        if (cand(i) && key(i) == T) ++eq;
    int rank = block_incl_scan256(eq, sh.scan) - eq;
    for (int i = lo; i < hi; ++i) {
        if (!cand(i)) continue;
        const uint32_t kv = key(i);
        if (kv > T) {
            mark[i] = 1;
        } else if (kv == T) {
            if (rank < need) mark[i] = 1;
            ++rank;
        }
    }
    __syncthreads();
}

// Writes the ids i < n with flag(i) in ascending order to out[0..cap), padding with -1.
template <class F>
__device__ void compact_ids(int n, F flag, int32_t *out, int cap, SelectShared &sh) {
    const int tid = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int cnt = 0;
    for (int i = lo; i < hi; ++i) cnt += flag(i) ? 1 : 0;
    const int incl = block_incl_scan256(cnt, sh.scan);
    int pos = incl - cnt;
    for (int i = lo; i < hi; ++i)
        if (flag(i)) {
            if (pos < cap) out[pos] = i;
            ++pos;
        }
    if (tid == kThreads - 1) sh.bcast[2] = incl;
    __syncthreads();
    for (int p = sh.bcast[2] + tid; p < cap; p += kThreads) out[p] = -1;
    __syncthreads();
}

// LDS layout of the selection phase for a row of n blocks.
struct RowLds {
    float *sc;          // [n] block scores
    uint8_t *inE;       // [n]
    uint8_t *inQ;       // [n]
    uint64_t *keys;     // [n] (rank path, rows of up to kRankMaxBlocks blocks)
};

__host__ __device__ inline size_t row_lds_bytes(int n) {
    const size_t n16 = (size_t)((n + 15) & ~15);
    return (n <= kRankMaxBlocks ? 8 * n16 : 0) + 4 * n16 + 2 * n16;
}

__device__ inline RowLds carve(unsigned char *dyn, int n) {
    const int n16 = (n + 15) & ~15;
    const int off = n <= kRankMaxBlocks ? 8 * n16 : 0;
    RowLds L;
    L.keys = n <= kRankMaxBlocks ? (uint64_t *)dyn : nullptr;
    L.sc = (float *)(dyn + off);
    L.inE = dyn + off + 4 * n16;
    L.inQ = L.inE + n16;
    return L;
}

// Selection of one row from the block scores in L.sc (all threads of the workgroup).
__device__ void select_row(const SelectArgs &a, int row, const RowLds &L, SelectShared &sh) {
    const int tid = threadIdx.x;
    const int n = a.n_blocks;
    for (int i = tid; i < n; i += kThreads) {
        L.inE[i] = 0;
        L.inQ[i] = 0;
    }
    __syncthreads();

    // Gamma_e: query-agnostic subset under strict eviction
    const int n_prev = a.n_prev;
    const bool fresh = (n_prev == 0);
    if (!fresh)
        for (int j = tid; j < a.ke; j += kThreads) {
            const int id = a.agn[(size_t)row * a.ke + j];
            if (id >= 0 && id < n_prev) L.inQ[id] = 1;   // previous Gamma_e (inQ reused as scratch)
        }
    __syncthreads();
    const float *evr = a.ev + (size_t)row * a.n_blocks_max;
    uint8_t *prevE = L.inQ;
    topk_mark(
        n, a.ke, [&](int i) { return order_key(evr[i]); },
        [&](int i) { return fresh || prevE[i] || i >= n_prev; }, L.inE, L.keys, sh);
    for (int i = tid; i < n; i += kThreads) L.inQ[i] = 0;
    __syncthreads();

    // Gamma_q: query-aware subset over the complement of Gamma_e
    const uint8_t *inE = L.inE;
    const float *sc = L.sc;
    topk_mark(
        n, a.kq, [&](int i) { return order_key(sc[i]); }, [&](int i) { return !inE[i]; }, L.inQ, L.keys, sh);

    // outputs, ascending block id
    const int k = a.kq + a.ke;
    if (a.ke > 0) compact_ids(n, [&](int i) { return L.inE[i] != 0; }, a.agn + (size_t)row * a.ke, a.ke, sh);
    compact_ids(n, [&](int i) { return (L.inE[i] | L.inQ[i]) != 0; }, a.sel + (size_t)row * k, k, sh);
}

}  // namespace

// Scores the blocks [part * blocks_per_part, ...) of one row; FUSED: the workgroup owns the whole
// row, keeps the scores in LDS and selects.
template <typename T, int D, int SPB, bool FUSED>
__global__ __launch_bounds__(256) void score_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ __align__(16) float qs[D];
    __shared__ SelectShared sh;

    constexpr int CPLS = D / 32;   // 16-byte chunks per lane of one fp32 sub-block row
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = blockIdx.x / a.parts, part = blockIdx.x - row * a.parts;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const int n = a.n_blocks;
    RowLds L;
    if (FUSED) L = carve(dyn, n);

    for (int c = tid; c < D; c += kThreads) {
        float s = 0.0f;
        for (int h = 0; h < a.G; ++h) s += load_elem<T>(a.q, ((size_t)(b * a.Hq + g * a.G + h)) * D + c);
        qs[c] = s;
    }
    __syncthreads();

    const int r8 = lane >> 3, c8 = lane & 7;
    float4 qv[CPLS];
#pragma unroll
    for (int i = 0; i < CPLS; ++i) qv[i] = *(const float4 *)&qs[(c8 + 8 * i) * 4];
    const int blk_lo = part * a.blocks_per_part;
    const int blk_hi = min(n, blk_lo + a.blocks_per_part);
    const int sb_lo = blk_lo * SPB, sb_hi = blk_hi * SPB;
    const int ngroups = (sb_hi - sb_lo + 7) >> 3;   // groups of 8 sub-blocks
    const float *kprow = a.kp + (size_t)row * a.n_blocks_max * SPB * D;
    float *gscore = a.scores + (size_t)row * a.scores_stride;
    for (int g0 = w; g0 < ngroups; g0 += 4 * kUnroll) {
        float4 x[kUnroll][CPLS];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = sb_lo + (g0 + 4 * u) * 8 + r8;
            const bool v = (g0 + 4 * u < ngroups) && (j < sb_hi);
#pragma unroll
            for (int i = 0; i < CPLS; ++i)
                x[u][i] = v ? *(const float4 *)(kprow + (size_t)j * D + (c8 + 8 * i) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = sb_lo + (g0 + 4 * u) * 8 + r8;
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < CPLS; ++i) {
                s = fmaf(x[u][i].x, qv[i].x, s);
                s = fmaf(x[u][i].y, qv[i].y, s);
                s = fmaf(x[u][i].z, qv[i].z, s);
                s = fmaf(x[u][i].w, qv[i].w, s);
            }
            s += dpp<kDppQuadXor1>(s);
            s += dpp<kDppQuadXor2>(s);
            s += dpp<kDppRowHalfMirror>(s);     // every lane of the 8-lane group holds u[j]
            if (SPB >= 2) s = fmaxf(s, dpp<kDppRowMirror>(s));
            if (SPB >= 4) s = fmaxf(s, xor_lane(s, 16));
            if (SPB >= 8) s = fmaxf(s, xor_lane(s, 32));
            const bool v = (g0 + 4 * u < ngroups) && (j < sb_hi);
            if (v && (lane % (8 * SPB)) == 0) {
                const int blk = j / SPB;
                if (FUSED) L.sc[blk] = s;
                else gscore[blk] = s;
            }
        }
    }
    if (!FUSED) return;
    __syncthreads();
    select_row(a, row, L, sh);
}

// Selection of rows scored by score_kernel<..., false>: one workgroup per row.
__global__ __launch_bounds__(256) void pick_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SelectShared sh;
    const int row = blockIdx.x;
    const RowLds L = carve(dyn, a.n_blocks);
    const float *gscore = a.scores + (size_t)row * a.scores_stride;
    for (int i = threadIdx.x; i < a.n_blocks; i += kThreads) L.sc[i] = gscore[i];
    __syncthreads();
    select_row(a, row, L, sh);
}

size_t select_lds_bytes(int n_blocks) { return row_lds_bytes(n_blocks); }

template <class K>
static hipError_t allow_lds(K kern, size_t dyn) {
    if (dyn <= 48 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
}

template <typename T, int D, int SPB>
static hipError_t launch_select_t(const SelectArgs &a, int rows, hipStream_t st) {
    hipError_t e;
    if (a.parts == 1 && !a.scores_only) {
        const size_t dyn = row_lds_bytes(a.n_blocks);
        auto kern = score_kernel<T, D, SPB, true>;
        if ((e = allow_lds(kern, dyn)) != hipSuccess) return e;
        kern<<<dim3((unsigned)rows), dim3(kThreads), dyn, st>>>(a);
        return hipGetLastError();
    }
    score_kernel<T, D, SPB, false><<<dim3((unsigned)(rows * a.parts)), dim3(kThreads), 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess || a.scores_only) return e;
    const size_t dyn = row_lds_bytes(a.n_blocks);
    if ((e = allow_lds(pick_kernel, dyn)) != hipSuccess) return e;
    pick_kernel<<<dim3((unsigned)rows), dim3(kThreads), dyn, st>>>(a);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_select_d(int spb, const SelectArgs &a, int rows, hipStream_t st) {
    switch (spb) {
        case 1: return launch_select_t<T, D, 1>(a, rows, st);
        case 2: return launch_select_t<T, D, 2>(a, rows, st);
        case 4: return launch_select_t<T, D, 4>(a, rows, st);
        default: return launch_select_t<T, D, 8>(a, rows, st);
    }
}

hipError_t launch_select(int dtype, int d, int spb, const SelectArgs &a, int rows, hipStream_t st) {
    if (dtype == 1) return d == 128 ? launch_select_d<uint16_t, 128>(spb, a, rows, st) : launch_select_d<uint16_t, 64>(spb, a, rows, st);
    return d == 128 ? launch_select_d<float, 128>(spb, a, rows, st) : launch_select_d<float, 64>(spb, a, rows, st);
}

}  // namespace nosa
