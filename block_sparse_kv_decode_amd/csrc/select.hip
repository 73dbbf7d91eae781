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
// Kernel shape: grid = rows x parts, 256 threads (4 waves of 64).
//   Scoring.  The group query qs = sum of the row's G query heads (float32) is dotted with every
//   pooled sub-block key; eight lanes share one 512-byte fp32 sub-block row (four 16-byte loads
//   each, fully coalesced), reduce with three DPP adds, and max-pool the block's sub-blocks with
//   DPP / lane swaps.  Each wave keeps four row groups in flight.
//   Selection.  One workgroup per row (the part that arrives last when parts > 1, found with an
//   agent-scope counter) selects in LDS:
//     Gamma_e: top-ke by eviction score among all visible blocks (first step) or among the
//              previous Gamma_e plus newly visible blocks (strict eviction);
//     Gamma_q: top-kq by block score among visible blocks outside Gamma_e.
//   Top-k is an exact radix select over order-preserving 32-bit keys (four 8-bit digit passes
//   with an LDS histogram), followed by a workgroup scan that gives equal keys to the lowest
//   block ids.  Outputs are compacted in ascending block id by another scan.
#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // sub-block groups per wave kept in flight

struct SelectShared {
    uint32_t hist[256];
    int scan[4];
    int bcast[4];
    int last;
};

// Marks the kk best candidates (key descending, id ascending) in mark[0..n).
template <class KeyF, class CandF>
__device__ void topk_mark(int n, int kk, KeyF key, CandF cand, uint8_t *mark, SelectShared &sh) {
    if (kk <= 0) return;
    const int tid = threadIdx.x;
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

}  // namespace

template <typename T, int D, int SPB>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ __align__(16) float qs[D];
    __shared__ SelectShared sh;

    constexpr int CPLS = D / 32;   // 16-byte chunks per lane of one fp32 sub-block row
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = blockIdx.x / a.parts, part = blockIdx.x - row * a.parts;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const int n = a.n_blocks;
    const bool fused = (a.parts == 1) && !a.scores_only;

    const int npad = (n + 15) & ~15;
    float *sc = (float *)dyn;                 // [n] block scores of this row (selection phase)
    uint8_t *inE = dyn + 4 * npad;            // [n] Gamma_e membership
    uint8_t *inQ = inE + npad;                // [n] Gamma_q membership (old Gamma_e first)

    // ---- group query ---------------------------------------------------------------------
    for (int c = tid; c < D; c += kThreads) {
        float s = 0.0f;
        for (int h = 0; h < a.G; ++h) s += load_elem<T>(a.q, ((size_t)(b * a.Hq + g * a.G + h)) * D + c);
        qs[c] = s;
    }
    __syncthreads();

    // ---- scoring of this part's blocks -----------------------------------------------------
    {
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
                    x[u][i] = v ? *(const float4 *)(kprow + (size_t)j * D + (c8 + 8 * i) * 4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
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
                    if (fused) sc[blk] = s;
                    else gscore[blk] = s;
                }
            }
        }
    }
    if (a.scores_only) return;

    // ---- one workgroup per row continues ---------------------------------------------------
    if (!fused) {
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const uint32_t prev = atomicAdd(&a.cnt[row], 1u);
            sh.last = (prev == (uint32_t)(a.parts - 1));
        }
        __syncthreads();
        if (!sh.last) return;
        __threadfence();
        const float *gscore = a.scores + (size_t)row * a.scores_stride;
        for (int i = tid; i < n; i += kThreads) sc[i] = load_agent(gscore + i);
        if (tid == 0) __hip_atomic_store(&a.cnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int i = tid; i < n; i += kThreads) {
        inE[i] = 0;
        inQ[i] = 0;
    }
    __syncthreads();

    // ---- Gamma_e: query-agnostic subset under strict eviction -------------------------------
    const int k = a.kq + a.ke;
    const int n_prev = a.n_prev;
    const bool fresh = (n_prev == 0);
    if (!fresh)
        for (int j = tid; j < a.ke; j += kThreads) {
            const int id = a.agn[(size_t)row * a.ke + j];
            if (id >= 0 && id < n_prev) inQ[id] = 1;   // previous Gamma_e
        }
    __syncthreads();
    const float *evr = a.ev + (size_t)row * a.n_blocks_max;
    topk_mark(
        n, a.ke, [&](int i) { return order_key(evr[i]); },
        [&](int i) { return fresh || inQ[i] || i >= n_prev; }, inE, sh);
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) inQ[i] = 0;
    __syncthreads();

    // ---- Gamma_q: query-aware subset over the complement ----------------------------------
    topk_mark(
        n, a.kq, [&](int i) { return order_key(sc[i]); }, [&](int i) { return !inE[i]; }, inQ, sh);
    __syncthreads();

    // ---- outputs, ascending block id --------------------------------------------------------
    if (a.ke > 0) compact_ids(n, [&](int i) { return inE[i] != 0; }, a.agn + (size_t)row * a.ke, a.ke, sh);
    compact_ids(n, [&](int i) { return (inE[i] | inQ[i]) != 0; }, a.sel + (size_t)row * k, k, sh);
}

size_t select_lds_bytes(int n_blocks) {
    const size_t npad = (size_t)((n_blocks + 15) & ~15);
    return 4 * npad + 2 * npad;
}

template <typename T, int D, int SPB>
static hipError_t launch_select_t(const SelectArgs &a, int rows, hipStream_t st) {
    const size_t dyn = a.scores_only ? 0 : select_lds_bytes(a.n_blocks);
    auto kern = select_kernel<T, D, SPB>;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    kern<<<dim3((unsigned)(rows * a.parts)), dim3(kThreads), dyn, st>>>(a);
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
