// decode.hip -- split-K GQA flash decoding over the selected KV blocks.
//
// "NOSA: Native and Offloadable Sparse Attention", [P1] paperlayer.ai summary App. A: after the
// selection and the transfer of missed blocks, attention runs over the KV cache; [P1] §2.2: most
// of the decode time goes to attention.  The pages give no formula; this is standard scaled
// dot-product attention restricted to the tokens of the k selected blocks.
//
// Grid: rows x S splits; a workgroup (4 waves) walks the blocks [sp*nbs, sp*nbs + nbs) of its
// row's block table.  Wave w owns tokens [16w, 16w + 16) of every block, so the four waves run
// with no barrier until the end of the split, each with its own online-softmax state for the G
// query heads of the row (the G heads reuse every K/V byte: the GQA saving).
//   QK, bf16 : one 16x16x32 bf16 MFMA per 32 dims: A = the wave's 16 key rows (each lane loads a
//              16-byte chunk; four lanes cover 64 contiguous bytes of a row), B = the G query
//              heads (columns G..15 zero), fp32 accumulate.  The G x 16 products of a block are a
//              small dense contraction; on the matrix cores it frees the VALU for the softmax and
//              P.V, and keeps q in 16 registers instead of 64.
//   QK, fp32 : VALU dot products, 4 lanes per key row, reduced with two DPP adds.
//   softmax  : scores in the log2 domain (scale * log2 e folded in).  The running max only moves
//              when some lane's score exceeds it (a wave-wide vote), so most blocks skip the
//              cross-lane max and the accumulator rescale.
//   P.V      : the wave's 16 V rows are loaded as contiguous 1 KiB lines; a lane owns one 16-byte
//              column chunk of several rows and accumulates G x chunk fp32 outputs (VALU FMAs:
//              V would need a transpose to feed the matrix cores).  Probabilities travel through
//              16 x G floats of LDS.
//   Prefetch : K and V of the next blocks are loaded into registers while a block is computed
//              (two blocks ahead for bf16, one for fp32).  A split reads its block ids once, 64
//              to a register (one per lane), so no block's loads wait on a table read.
// End of split: lane reduction, a 4-wave merge through LDS, then either the final output
// (one split) or a (max, sum, acc) partial in the workspace, merged by combine_kernel with the same
// online-softmax rule.  No workgroup waits on another.  A launch may fill only some of a row's
// partial slots (slots [s0, s0 + S) of St): the offload step attends the cache hits in one launch
// while the missed blocks are still in transit, and the missed blocks in a second launch that
// reads their slots straight from the miss list (entry stride 2, per-row count), and one combine
// merges both.
#include "gather_core.h"
#include "nosa_device.h"
#include "nosa_internal.h"
#include "select_core.h"

namespace nosa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kTokPerWave = kBlockTokens / kWaves;   // 16

template <typename T, int D>
struct Geom {
    static constexpr int EB = (int)sizeof(T);
    static constexpr int EPC = 16 / EB;              // elements per 16-byte chunk
    static constexpr int RB = D * EB;                // bytes per token row
    static constexpr int NC = RB / 16;               // chunks per token row
    static constexpr int CPL = NC / 4;               // chunks per lane per 16-token slice
    static constexpr int TPI = 64 / NC;              // tokens per wave-wide V load
    static_assert(NC == 8 || NC == 16 || NC == 32, "unsupported row size");
};

__device__ __forceinline__ float dot16_f32(const uint4 &a, const uint4 &b, float acc) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
    return acc;
}

__device__ __forceinline__ void unpack16(const uint4 &x, float *v, uint16_t) {
    v[0] = bf16_lo(x.x); v[1] = bf16_hi(x.x);
    v[2] = bf16_lo(x.y); v[3] = bf16_hi(x.y);
    v[4] = bf16_lo(x.z); v[5] = bf16_hi(x.z);
    v[6] = bf16_lo(x.w); v[7] = bf16_hi(x.w);
}
__device__ __forceinline__ void unpack16(const uint4 &x, float *v, float) {
    v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y);
    v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Entries [j0, j1) of a split's block table (tab[j * stride]), held 64 at a time in one register
// of the wave: lane l holds entry base + l.  id(j) must be called with uniform, non-decreasing j
// in [j0, j1); crossing into the next 64 entries reloads the window.
struct TableWindow {
    const int32_t *tab;
    int stride, j1, lane, base, v;
    __device__ __forceinline__ TableWindow(const int32_t *t, int s, int j0, int j1_, int ln)
        : tab(t), stride(s), j1(j1_), lane(ln), base(j0) {
        v = fetch();
    }
    __device__ __forceinline__ int fetch() const {
        const int jj = base + lane;
        return jj < j1 ? tab[(size_t)jj * stride] : -1;
    }
    __device__ __forceinline__ int id(int j) {
        if (j - base >= 64) {
            base += 64 * ((j - base) >> 6);
            v = fetch();
        }
        return __builtin_amdgcn_readlane(v, j - base);
    }
};

// acc[h][e] += p[tok][h] * V[tok][chunk e] over this lane's PV tokens of the block.
template <typename T, int D, int G>
__device__ __forceinline__ void pv_accumulate(const float (*pl)[G], int tpv, const uint4 (&vv)[Geom<T, D>::CPL],
                                              float (&acc)[G][Geom<T, D>::EPC]) {
    using Gm = Geom<T, D>;
#pragma unroll
    for (int i = 0; i < Gm::CPL; ++i) {
        const int tok = i * Gm::TPI + tpv;
        float p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) p[h] = pl[tok][h];
        float v[Gm::EPC];
        unpack16(vv[i], v, T());
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < Gm::EPC; ++e) acc[h][e] = fmaf(p[h], v[e], acc[h][e]);
    }
}

template <int D, int G>
struct SplitShared {
    __align__(16) float p[kWaves][kTokPerWave][G];
    float m[kWaves][G], l[kWaves][G];
    __align__(16) float acc[kWaves][G][D];
};

// End of a split: reduce the lane accumulators, merge the 4 waves, write the output (S == 1) or
// the split's (max, sum, acc) partial.  m_h / l_h: this wave's per-head running max / sum.
template <typename T, int D, int G>
__device__ __forceinline__ void finish_split(const DecodeArgs &a, int row, int sp, const float (&m_h)[G],
                                             const float (&l_h)[G], float (&acc)[G][Geom<T, D>::EPC],
                                             SplitShared<D, G> &sh) {
    using Gm = Geom<T, D>;
    constexpr int NC = Gm::NC, EPC = Gm::EPC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cpv = lane % NC, tpv = lane / NC;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            float x = acc[h][e];
            if (NC <= 8) x += dpp<kDppRowRor8>(x);
            if (NC <= 16) x += xor_lane(x, 16);
            x += xor_lane(x, 32);
            acc[h][e] = x;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            sh.m[w][h] = m_h[h];
            sh.l[w][h] = l_h[h];
        }
    }
    if (tpv == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) sh.acc[w][h][cpv * EPC + e] = acc[h][e];
    }
    __syncthreads();
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const size_t out_base = (size_t)(b * a.Hq + g * G) * D;
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D, dd = idx - h * D;
        float M = sh.m[0][h];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sh.m[ww][h]);
        float L = 0.0f, A = 0.0f;
        if (M != -INFINITY) {     // else the split saw no block: empty partial (M = -inf, L = A = 0)
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = fast_exp2(sh.m[ww][h] - M);
                L = fmaf(sh.l[ww][h], f, L);
                A = fmaf(sh.acc[ww][h][dd], f, A);
            }
        }
        if (a.direct) {
            store_elem<T>(a.out, out_base + idx, L > 0.0f ? A / L : 0.0f);   // a row with no valid block: 0
        } else {
            float *part = a.part + ((size_t)(row * a.St + a.s0 + sp) * G + h) * (D + 2);
            part[2 + dd] = A;
            if (dd == 0) {
                part[0] = M;
                part[1] = L;
            }
        }
    }
}

}  // namespace

// ---- bf16: QK on the matrix cores -----------------------------------------------------------
// Where this lane's K and V chunks of a block lie: wave w covers tokens [16w, 16w + 16); K in the
// MFMA A layout (lane = key row j16 of k-group grp), V as contiguous 1 KiB lines (PV layout).
template <int D>
struct BlockAddr {
    using Gm = Geom<uint16_t, D>;
    static constexpr int KS = D / 32, CPL = Gm::CPL, RB = Gm::RB;
    const char *kbase, *vbase;
    int kofs[KS], vofs[CPL];
    __device__ __forceinline__ BlockAddr(const DecodeArgs &a, int row) {
        const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
        const int j16 = lane & 15, grp = lane >> 4;
        const int cpv = lane % Gm::NC, tpv = lane / Gm::NC;
        const size_t rowb = (size_t)row * a.store_blocks * blk_bytes() + (size_t)w * kTokPerWave * RB;
        kbase = (const char *)a.k + rowb;
        vbase = (const char *)a.v + rowb;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kofs[ks] = j16 * RB + (4 * ks + grp) * 16;
#pragma unroll
        for (int i = 0; i < CPL; ++i) vofs[i] = (i * Gm::TPI + tpv) * RB + cpv * 16;
    }
    static constexpr size_t blk_bytes() { return (size_t)kBlockTokens * RB; }
    // Issues the loads of block blk (false, and no loads, for an id outside the store).
    __device__ __forceinline__ bool issue(const DecodeArgs &a, int blk, uint4 (&kk)[KS], uint4 (&vv)[CPL]) const {
        if ((unsigned)blk >= (unsigned)a.store_blocks) return false;
        const char *kp = kbase + (size_t)blk * blk_bytes();
        const char *vp = vbase + (size_t)blk * blk_bytes();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kk[ks] = *(const uint4 *)(kp + kofs[ks]);
#pragma unroll
        for (int i = 0; i < CPL; ++i) vv[i] = *(const uint4 *)(vp + vofs[i]);
        return true;
    }
};

// The MFMA B operand of a row's query: lane (j16, grp) holds dims 32 ks + 8 grp .. + 8 of head
// j16 (zero for j16 >= G).  A caller that attends only after other work (scoring, ranking) loads
// it first, so that the split's first K/V loads do not wait behind a query round trip.
template <int D>
struct QFrag {
    bf16x8_t qb[D / 32];
};

template <int D, int G>
__device__ __forceinline__ void load_qfrag(const DecodeArgs &a, int row, QFrag<D> &f) {
    constexpr int RB = D * 2;
    const int lane = threadIdx.x & 63, j16 = lane & 15, grp = lane >> 4;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const char *qrow = (const char *)a.q + (size_t)(b * a.Hq + g * G + (j16 < G ? j16 : 0)) * RB;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (j16 < G) x = *(const uint4 *)(qrow + (4 * ks + grp) * 16);
        f.qb[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
}

// Two blocks whose loads a caller issued ahead of the split (the split's first two entries).
template <int D>
struct PreBlocks {
    uint4 k0[D / 32], v0[D / 32], k1[D / 32], v1[D / 32];
    bool o0 = false, o1 = false;
};

// One split: entries [j0, j1) of the row's table (tab[j * tab_stride], block ids into the store),
// written as partial slot sp of the row (or the output itself when a.direct).  With PRE, the loads
// of entries j0 and j0 + 1 were already issued into *pre.  qf: the row's query fragment, loaded by
// the caller (else loaded here).
template <int D, int G, bool PRE = false>
__device__ __forceinline__ void decode_mfma_split(const DecodeArgs &a, int row, int sp, const int32_t *tab,
                                                  int tab_stride, int j0, int j1, SplitShared<D, G> &sh,
                                                  PreBlocks<D> *pre = nullptr, const QFrag<D> *qf = nullptr) {
    using Gm = Geom<uint16_t, D>;
    constexpr int KS = D / 32;                        // 32-dim MFMA steps
    constexpr int CPL = Gm::CPL, EPC = Gm::EPC, NC = Gm::NC;
    static_assert(CPL == KS, "bf16 rows: one V chunk per MFMA step");

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int j16 = lane & 15, grp = lane >> 4;       // MFMA layout: column (head) / k-group
    const int tpv = lane / NC;                        // PV layout

    // B operand: q of head j16 (zero columns beyond G), dims 32 ks + 8 grp .. + 8
    QFrag<D> qown;
    if (!qf) {
        load_qfrag<D, G>(a, row, qown);
        qf = &qown;
    }
    bf16x8_t qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = qf->qb[ks];

    const BlockAddr<D> ba(a, row);

    float m = -INFINITY;          // running max of head j16 (lanes j16 < G)
    float lq = 0.0f;              // running sum of p over this lane's 4 tokens of head j16
    float acc[G][EPC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;
    float(*pl)[G] = sh.p[w];
    const float sl2 = a.sl2;

    auto process = [&](const uint4(&kk)[KS], const uint4(&vv)[CPL]) {
        floatx4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[ks]), qb[ks], c, 0, 0, 0);
        // lane holds S[token 4 grp + e][head j16]
        float z[4];
        bool up = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = c[e] * sl2;
            up |= (j16 < G) && (z[e] > m);
        }
        const bool rescale = __any(up);
        float alpha = 1.0f;
        if (rescale) {
            float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
            bm = fmaxf(bm, xor_lane(bm, 16));
            bm = fmaxf(bm, xor_lane(bm, 32));
            const float mn = fmaxf(m, bm);
            alpha = fast_exp2(m - mn);
            m = mn;
        }
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = fast_exp2(z[e] - m);
            ps += z[e];
        }
        lq = rescale ? fmaf(lq, alpha, ps) : lq + ps;
        if (j16 < G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) pl[4 * grp + e][j16] = z[e];
        }
        wave_lds_sync();
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ah = readlane_f(alpha, h);
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[h][e] *= ah;
            }
        }
        pv_accumulate<uint16_t, D, G>(pl, tpv, vv, acc);
        wave_lds_sync();
    };

    // The split's block ids, 64 at a time, one per lane: a block's K/V loads take its id with a
    // lane read (j is uniform) instead of waiting on a table load of their own.
    TableWindow tw(tab, tab_stride, j0, j1, lane);
    auto load = [&](int j, uint4(&kk)[KS], uint4(&vv)[CPL]) -> bool { return ba.issue(a, tw.id(j), kk, vv); };

    // three register buffers: blocks j+1 and j+2 are in flight while block j is computed
    uint4 kb0[KS], vb0[CPL], kb1[KS], vb1[CPL], kb2[KS], vb2[CPL];
    int j = j0;
    bool o0, o1;
    if (PRE) {
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            kb0[i] = pre->k0[i];
            vb0[i] = pre->v0[i];
            kb1[i] = pre->k1[i];
            vb1[i] = pre->v1[i];
        }
        o0 = pre->o0;
        o1 = pre->o1;
    } else {
        o0 = (j < j1) ? load(j, kb0, vb0) : false;
        o1 = (j + 1 < j1) ? load(j + 1, kb1, vb1) : false;
    }
    bool o2 = false;
    while (j < j1) {
        if (j + 2 < j1) o2 = load(j + 2, kb2, vb2);
        if (o0) process(kb0, vb0);
        if (++j >= j1) break;
        if (j + 2 < j1) o0 = load(j + 2, kb0, vb0);
        if (o1) process(kb1, vb1);
        if (++j >= j1) break;
        if (j + 2 < j1) o1 = load(j + 2, kb1, vb1);
        if (o2) process(kb2, vb2);
        ++j;
    }

    // per-head max and sum of this wave: lanes j16 = h of the four k-groups
    float lt = lq;
    lt += xor_lane(lt, 16);
    lt += xor_lane(lt, 32);
    float m_h[G], l_h[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_h[h] = readlane_f(m, h);
        l_h[h] = readlane_f(lt, h);
    }
    finish_split<uint16_t, D, G>(a, row, sp, m_h, l_h, acc, sh);
}

// Entries [j0, j1) of split sp of a row.  With a per-row entry count (the missed blocks of an
// offloaded step) the row's entries are spread evenly over the S splits, so that a few misses are
// attended side by side instead of one after another by the first split (measured on MI355X in the
// bs16/16K offload loop, about 3 misses per row in 4 splits: 0.254 against 0.259 ms per step; the
// miss launch took 13 us with fixed ranges).
__device__ __forceinline__ int2 split_range(const DecodeArgs &a, int row, int sp) {
    if (!a.count) {
        const int j0 = sp * a.nbs;
        return make_int2(j0, min(a.k_sel, j0 + a.nbs));
    }
    const int n_use = min(a.k_sel, max(a.count[row], 0));
    const int nb = (n_use + a.S - 1) / a.S;
    const int j0 = sp * nb;
    return make_int2(j0, min(n_use, j0 + nb));
}

template <int D, int G>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeArgs a) {
    __shared__ SplitShared<D, G> sh;
    const int row = blockIdx.x / a.S, sp = blockIdx.x - row * a.S;
    const int2 jr = split_range(a, row, sp);
    decode_mfma_split<D, G>(a, row, sp, a.table + (size_t)row * a.k_sel * a.tab_stride, a.tab_stride, jr.x, jr.y,
                            sh);
}

// ---- offloaded KV: the gather and the attention over the cache hits in one launch ----------
// Workgroups [0, n_gather) run the persistent gather of the missed blocks (gather_blocks); the rest
// are decode_mfma_kernel's splits over the hit-only table.  The two roles share no data: the hits'
// slots are not written by this step's gather.  One launch on one stream overlaps them with no
// cross-stream event between map, gather and attention; the launch after it (the missed blocks)
// is ordered behind both.  The gather's workgroups come first in dispatch order.
template <int D, int G>
__global__ __launch_bounds__(256, 2) void hit_gather_kernel(DecodeArgs a, GatherArgs g, int n_gather) {
    extern __shared__ __align__(16) unsigned char dyn[];   // the gather's start[rows + 1]
    __shared__ SplitShared<D, G> sh;
    __shared__ int wsum[kGatherThreads / 64];
    if ((int)blockIdx.x < n_gather) {
        gather_blocks(g, blockIdx.x, n_gather, (int *)dyn, wsum);
        return;
    }
    const int bid = blockIdx.x - n_gather;
    const int row = bid / a.S, sp = bid - row * a.S;
    const int2 jr = split_range(a, row, sp);
    decode_mfma_split<D, G>(a, row, sp, a.table + (size_t)row * a.k_sel * a.tab_stride, a.tab_stride, jr.x, jr.y,
                            sh);
}

// ---- fp32: QK on the VALU ------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256, (G >= 8 || D > 64) ? 1 : 2) void decode_valu_kernel(DecodeArgs a) {
    using Gm = Geom<float, D>;
    constexpr int CPL = Gm::CPL, EPC = Gm::EPC, NC = Gm::NC, RB = Gm::RB, TPI = Gm::TPI;
    __shared__ SplitShared<D, G> sh;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = blockIdx.x / a.S, sp = blockIdx.x - row * a.S;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const int sub = lane & 3, tq = lane >> 2;          // QK layout: 4 lanes per key row
    const int cpv = lane % NC, tpv = lane / NC;        // PV layout
    const int2 jr = split_range(a, row, sp);
    const int j0 = jr.x, j1 = jr.y;

    uint4 qf[G][CPL];
    {
        const char *qrow = (const char *)a.q + (size_t)(b * a.Hq + g * G) * RB;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < CPL; ++i) qf[h][i] = *(const uint4 *)(qrow + h * RB + (sub + 4 * i) * 16);
    }
    const size_t blk_bytes = (size_t)kBlockTokens * RB;
    const char *kbase = (const char *)a.k + (size_t)row * a.store_blocks * blk_bytes + (size_t)w * kTokPerWave * RB;
    const char *vbase = (const char *)a.v + (size_t)row * a.store_blocks * blk_bytes + (size_t)w * kTokPerWave * RB;
    int kofs[CPL], vofs[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        kofs[i] = tq * RB + (sub + 4 * i) * 16;
        vofs[i] = (i * TPI + tpv) * RB + cpv * 16;
    }

    float m[G], lq[G], acc[G][EPC];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        lq[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;
    }
    float(*pl)[G] = sh.p[w];
    const float sl2 = a.sl2;

    auto process = [&](const uint4(&kk)[CPL], const uint4(&vv)[CPL]) {
        float z[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) s = dot16_f32(qf[h][i], kk[i], s);
            s += dpp<kDppQuadXor1>(s);
            s += dpp<kDppQuadXor2>(s);
            z[h] = s * sl2;
        }
        bool up = false;
#pragma unroll
        for (int h = 0; h < G; ++h) up |= z[h] > m[h];
        float alpha[G];
        const bool rescale = __any(up);
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float bm = fmaxf(z[h], dpp<kDppRowRor4>(z[h]));
                bm = fmaxf(bm, dpp<kDppRowRor8>(bm));
                bm = fmaxf(bm, xor_lane(bm, 16));
                bm = fmaxf(bm, xor_lane(bm, 32));
                const float mn = fmaxf(m[h], bm);
                alpha[h] = fast_exp2(m[h] - mn);
                m[h] = mn;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float p = fast_exp2(z[h] - m[h]);
            lq[h] = rescale ? fmaf(lq[h], alpha[h], p) : lq[h] + p;
            z[h] = p;
        }
        if (sub == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) pl[tq][h] = z[h];
        }
        wave_lds_sync();
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha[h];
        }
        pv_accumulate<float, D, G>(pl, tpv, vv, acc);
        wave_lds_sync();
    };

    const int32_t *tab = a.table + (size_t)row * a.k_sel * a.tab_stride;
    TableWindow tw(tab, a.tab_stride, j0, j1, lane);
    auto load = [&](int j, uint4(&kk)[CPL], uint4(&vv)[CPL]) -> bool {
        const int blk = tw.id(j);
        if ((unsigned)blk >= (unsigned)a.store_blocks) return false;
        const char *kp = kbase + (size_t)blk * blk_bytes;
        const char *vp = vbase + (size_t)blk * blk_bytes;
#pragma unroll
        for (int i = 0; i < CPL; ++i) kk[i] = *(const uint4 *)(kp + kofs[i]);
#pragma unroll
        for (int i = 0; i < CPL; ++i) vv[i] = *(const uint4 *)(vp + vofs[i]);
        return true;
    };
    uint4 kc[CPL], vc[CPL], kn[CPL], vn[CPL];
    int j = j0;
    bool okc = (j < j1) ? load(j, kc, vc) : false, okn = false;
    while (j < j1) {
        if (j + 1 < j1) okn = load(j + 1, kn, vn);
        if (okc) process(kc, vc);
        if (++j >= j1) break;
        if (j + 1 < j1) okc = load(j + 1, kc, vc);
        if (okn) process(kn, vn);
        ++j;
    }

    float m_h[G], l_h[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float x = lq[h];                  // identical in the 4 lanes of a key row
        x += dpp<kDppRowRor4>(x);
        x += dpp<kDppRowRor8>(x);
        x += xor_lane(x, 16);
        x += xor_lane(x, 32);
        l_h[h] = x;
        m_h[h] = m[h];
    }
    finish_split<float, D, G>(a, row, sp, m_h, l_h, acc, sh);
}

// ---- the decode step with the query-aware pick inside the attention launch -------------------
// Grid rows x (S_e + S_q), bf16.  Once the scoring kernel has written the block scores and
// Gamma_e (agn_state), a row's S_e Gamma_e splits (partial slots 0 .. S_e - 1) attend the Gamma_e
// blocks straight away, while each of its S_q Gamma_q splits (slots S_e ..) ranks the row's Gamma_q
// in LDS (the one in slot S_e also writes the row's selection, the ascending union) and then
// attends its slice of Gamma_q.  Attention does not
// depend on the order of the blocks, so the pick hides under the Gamma_e splits' streaming instead
// of taking a kernel of its own.  Every split writes partial slot sp; combine_kernel merges them.
// Workgroup ids are split-major, Gamma_q splits first: ids [0, S_q * rows) are the Gamma_q splits
// of every row, then the Gamma_e splits.  Consecutive ids go to the eight XCDs in turn, so with
// row-major ids and S_e + S_q dividing 8 each XCD would hold one role only: half of them streaming
// Gamma_e from the start and finishing first, the other half ranking and then forming the tail,
// each phase on half the chip's paths to memory.  Split-major ids give every XCD an equal share of
// both roles, and the rankings are dispatched first.  (Measured on MI355X at bs16/16K: 62.2 against
// 63.8 us per step; 62.7 with the Gamma_e splits first.)
template <int D, int G>
__global__ __launch_bounds__(256, 2) void step_decode_kernel(DecodeArgs a, SelectArgs s, int S_e, int S_q) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SplitShared<D, G> sh;
    __shared__ SelectShared<256> ssh;
    const int St = S_e + S_q, rows = gridDim.x / St;
    const int si = blockIdx.x / rows, row = blockIdx.x - si * rows;
    const int sp = si < S_q ? S_e + si : si - S_q;   // partial slot: Gamma_e splits first
    if (sp < S_e) {
        const int j0 = sp * a.nbs, j1 = min(s.ke, j0 + a.nbs);
        decode_mfma_split<D, G>(a, row, sp, s.agn + (size_t)row * s.ke, 1, j0, j1, sh);
        return;
    }
    const int n = s.n_blocks, tid = threadIdx.x;
    // the query fragment first: the split's first K/V loads then wait for nothing older
    QFrag<D> qf;
    load_qfrag<D, G>(a, row, qf);
    const RowLds L = carve<256>(dyn, n);
    int32_t *qlist = (int32_t *)(dyn + row_lds_bytes<256>(n));   // [kq] Gamma_q, ascending
    const float *gscore = s.scores + (size_t)row * s.scores_stride;
    const int32_t *agn = s.agn + (size_t)row * s.ke;
    const int k = s.kq + s.ke;
    // the first Gamma_q split writes the row's selection
    int32_t *selrow = sp == S_e ? s.sel + (size_t)row * k : nullptr;
    // The ranking shares its CU with streaming attention workgroups: give it issue priority.
    __builtin_amdgcn_s_setprio(2);
    if (!reg_pick_fits<256>(n, s.kq, s.ke) ||
        !pick_query_regs<256>(gscore, n, agn, s.ke, s.kq, L.keys, qlist, selrow, ssh)) {
        // Gamma_e ids loaded together with the scores (one memory round trip), marked after the clear
        constexpr int kAgnPer = 2;   // ids per thread in flight; more are read after the barrier
        int ids[kAgnPer];
#pragma unroll
        for (int r = 0; r < kAgnPer; ++r) {
            const int j = tid + r * 256;
            ids[r] = j < s.ke ? agn[j] : -1;
        }
        scores_to_lds<256>(gscore, n, L);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kAgnPer; ++r)
            if (ids[r] >= 0 && ids[r] < n) L.inE[ids[r]] = 1;
        for (int j = tid + kAgnPer * 256; j < s.ke; j += 256) {
            const int id = agn[j];
            if (id >= 0 && id < n) L.inE[id] = 1;
        }
        __syncthreads();
        topk_mark<256>(
            n, s.kq, [&](int i) { return order_key(L.sc[i]); }, [&](int i) { return !L.inE[i]; }, L.inQ, L.keys,
            ssh);
        // one pass: Gamma_q (ascending) into LDS, and the selection
        compact_outputs<256>(n, L.inQ, L.inE, qlist, s.kq, selrow, selrow ? k : 0, ssh);
    }
    __builtin_amdgcn_s_setprio(0);
    // qlist complete in LDS; the selection's global stores need not have landed
    wg_barrier();
    const int j0 = (sp - S_e) * a.nbs, j1 = min(s.kq, j0 + a.nbs);
    decode_mfma_split<D, G>(a, row, sp, qlist, 1, j0, j1, sh, nullptr, &qf);
}

// ---- the decode step in one workgroup per row ----------------------------------------------
// Grid rows, bf16, for plans where one 256-thread workgroup scores and selects a row and a single
// split attends it (many rows, short rows): the workgroup scores its row, selects (writing
// agn_state and the selection), and attends the selected blocks straight after, so each row's
// attention starts when its own selection is done rather than when the slowest row's is.  Rows
// of up to 64 blocks are selected in registers (select_row64); on longer rows the loads of the
// first two Gamma_e blocks go out before the Gamma_q ranking and land during it.
template <int D, int G, int SPB>
__global__ __launch_bounds__(256, 2) void row_step_kernel(DecodeArgs a, SelectArgs s) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ SplitShared<D, G> sh;
    __shared__ SelectShared<256> ssh;
    const int row = blockIdx.x;
    const int n = s.n_blocks, k = s.kq + s.ke;
    const RowLds L = carve<256>(dyn, n);
    int32_t *wl = (int32_t *)(dyn + row_lds_bytes<256>(n));   // [k]: Gamma_e, then Gamma_q, each ascending
    // the query fragment first: attention's first K/V loads then wait for nothing older
    QFrag<D> qf;
    load_qfrag<D, G>(a, row, qf);
    float e[kEvPre];
    ev_load<256>(s, row, e);
    const int pid = prev_agn(s, row, n <= kWaveRowMax ? (int)(threadIdx.x & 63) : (int)threadIdx.x);
    score_range<uint16_t, D, SPB, 256>(s, row, 0, n, L.sc, nullptr);
    ev_store<256>(s, row, L, n, e);
    wg_barrier();
    if (n <= kWaveRowMax) {
        // a row of up to 64 blocks: lane i of each wave holds block i, the waves share the ranking
        select_row64<256>(s, row, L, wl, pid);
        wg_barrier();
        decode_mfma_split<D, G>(a, row, 0, wl, 1, 0, k, sh, nullptr, &qf);
        return;
    }
    select_agnostic<256>(s, row, L, ssh, pid);
    compact_outputs<256>(n, L.inE, L.inE, wl, s.ke, nullptr, 0, ssh);
    wg_barrier();
    // The first two Gamma_e blocks' loads go out now and stay in flight through the Gamma_q
    // ranking, whose barriers wait for LDS only.  (Not at d 128 with 8 query heads per KV head:
    // holding the two blocks through the ranking would spill registers.)
    constexpr bool kPre = !(D == 128 && G == 8);
    PreBlocks<D> pre;
    if (kPre && s.ke >= 2) {
        const BlockAddr<D> ba(a, row);
        pre.o0 = ba.issue(a, wl[0], pre.k0, pre.v0);
        pre.o1 = ba.issue(a, wl[1], pre.k1, pre.v1);
    }
    select_query<256>(s, row, L, ssh, true);
    compact_outputs<256>(n, L.inQ, L.inQ, wl + s.ke, s.kq, nullptr, 0, ssh);
    wg_barrier();
    if (kPre && s.ke >= 2)
        decode_mfma_split<D, G, kPre>(a, row, 0, wl, 1, 0, k, sh, &pre, &qf);
    else
        decode_mfma_split<D, G>(a, row, 0, wl, 1, 0, k, sh, nullptr, &qf);
}

bool row_step_fits(int n_blocks, int k) {
    return row_lds_bytes<256>(n_blocks) + 4 * (size_t)k <= kRowStepMaxLds;
}

// Merges the St split partials (max, sum, acc) of one (row, head) into the output; thread = dim.
// Empty partials (max = -inf) carry nothing and are passed over.  The partials are read kChunk
// splits at a time, every load issued before any is used (one memory round trip per chunk rather
// than two per split); each chunk is folded in against the largest max seen so far.
template <typename T, int D, int G, int kChunk>
__global__ __launch_bounds__(D) void combine_kernel(DecodeArgs a) {
    const int row = blockIdx.x / G, h = blockIdx.x - row * G;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const int dd = threadIdx.x;
    const float *rp = a.part + ((size_t)row * a.St * G + h) * (D + 2);
    const size_t stride = (size_t)G * (D + 2);
    float M = -INFINITY, L = 0.0f, A = 0.0f;
    for (int s0 = 0; s0 < a.St; s0 += kChunk) {
        float hd[kChunk], as[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            // slots past St re-read the last slot (no branch between the loads) and count as empty;
            // even lanes load the slot's max, odd lanes its sum (vector loads, waited for in order)
            const float *ps = rp + (size_t)min(s0 + u, a.St - 1) * stride;
            hd[u] = ps[dd & 1];
            as[u] = ps[2 + dd];
        }
        float ms[kChunk], ls[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            ms[u] = s0 + u < a.St ? readlane_f(hd[u], 0) : -INFINITY;
            ls[u] = readlane_f(hd[u], 1);
        }
        float mc = M;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) mc = fmaxf(mc, ms[u]);
        const float fo = M == -INFINITY ? 0.0f : fast_exp2(M - mc);   // L = A = 0 while M is -inf
        L *= fo;
        A *= fo;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const bool live = ms[u] != -INFINITY;
            const float f = fast_exp2(ms[u] - mc);
            L = live ? fmaf(ls[u], f, L) : L;
            A = live ? fmaf(as[u], f, A) : A;
        }
        M = mc;
    }
    // a row with no valid block in any slot (L = 0) yields 0
    store_elem<T>(a.out, (size_t)(b * a.Hq + g * G + h) * D + dd, L > 0.0f ? A / L : 0.0f);
}

static hipError_t mark(hipEvent_t ev, hipStream_t st) { return ev ? hipEventRecord(ev, st) : hipSuccess; }

// The merge reads up to 16 partial slots per memory round trip: 8 at a time when a row has no more
// (fewer loads), else 16 (one round trip for the fused step's 16 splits at bs4/128K).
template <typename T, int D, int G>
static hipError_t launch_combine(const DecodeArgs &a, int rows, hipStream_t st) {
    if (a.St <= 8)
        combine_kernel<T, D, G, 8><<<dim3((unsigned)(rows * G)), dim3(D), 0, st>>>(a);
    else
        combine_kernel<T, D, G, 16><<<dim3((unsigned)(rows * G)), dim3(D), 0, st>>>(a);
    return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, int rows, hipStream_t st, bool merge, const KernelMarks &m) {
    hipError_t e = mark(m.start, st);
    if (e != hipSuccess) return e;
    if (sizeof(T) == 2)
        decode_mfma_kernel<D, G><<<dim3((unsigned)(rows * a.S)), dim3(256), 0, st>>>(a);
    else
        decode_valu_kernel<D, G><<<dim3((unsigned)(rows * a.S)), dim3(256), 0, st>>>(a);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(m.stop, st);
    if (e != hipSuccess || a.direct || !merge) return e;
    return launch_combine<T, D, G>(a, rows, st);
}

template <typename T, int D>
static hipError_t launch_decode_d(int G, const DecodeArgs &a, int rows, hipStream_t st, bool merge,
                                  const KernelMarks &m) {
    switch (G) {
        case 1: return launch_decode_t<T, D, 1>(a, rows, st, merge, m);
        case 2: return launch_decode_t<T, D, 2>(a, rows, st, merge, m);
        case 4: return launch_decode_t<T, D, 4>(a, rows, st, merge, m);
        default: return launch_decode_t<T, D, 8>(a, rows, st, merge, m);
    }
}

template <int D, int G>
static hipError_t launch_step_t(const DecodeArgs &a, const SelectArgs &s, int rows, int S_e, int S_q,
                                hipStream_t st, const KernelMarks &m) {
    const size_t dyn = row_lds_bytes<256>(s.n_blocks) + 4 * (size_t)s.kq;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)step_decode_kernel<D, G>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipError_t e = mark(m.start, st);
    if (e != hipSuccess) return e;
    step_decode_kernel<D, G><<<dim3((unsigned)(rows * (S_e + S_q))), dim3(256), dyn, st>>>(a, s, S_e, S_q);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(m.stop, st);
    if (e != hipSuccess) return e;
    return launch_combine<uint16_t, D, G>(a, rows, st);
}

template <int D>
static hipError_t launch_step_d(int G, const DecodeArgs &a, const SelectArgs &s, int rows, int S_e, int S_q,
                                hipStream_t st, const KernelMarks &m) {
    switch (G) {
        case 1: return launch_step_t<D, 1>(a, s, rows, S_e, S_q, st, m);
        case 2: return launch_step_t<D, 2>(a, s, rows, S_e, S_q, st, m);
        case 4: return launch_step_t<D, 4>(a, s, rows, S_e, S_q, st, m);
        default: return launch_step_t<D, 8>(a, s, rows, S_e, S_q, st, m);
    }
}

hipError_t launch_step_decode(int d, int G, const DecodeArgs &a, const SelectArgs &s, int rows, int S_e, int S_q,
                              hipStream_t st, const KernelMarks &m) {
    return d == 128 ? launch_step_d<128>(G, a, s, rows, S_e, S_q, st, m)
                    : launch_step_d<64>(G, a, s, rows, S_e, S_q, st, m);
}

template <int D, int G, int SPB>
static hipError_t launch_row_step_t(const DecodeArgs &a, const SelectArgs &s, int rows, hipStream_t st,
                                    const KernelMarks &m) {
    const size_t dyn = row_lds_bytes<256>(s.n_blocks) + 4 * (size_t)(s.kq + s.ke);
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)row_step_kernel<D, G, SPB>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipError_t e = mark(m.start, st);
    if (e != hipSuccess) return e;
    row_step_kernel<D, G, SPB><<<dim3((unsigned)rows), dim3(256), dyn, st>>>(a, s);
    e = hipGetLastError();
    return e == hipSuccess ? mark(m.stop, st) : e;
}

template <int D, int G>
static hipError_t launch_row_step_g(int spb, const DecodeArgs &a, const SelectArgs &s, int rows, hipStream_t st,
                                    const KernelMarks &m) {
    switch (spb) {
        case 1: return launch_row_step_t<D, G, 1>(a, s, rows, st, m);
        case 2: return launch_row_step_t<D, G, 2>(a, s, rows, st, m);
        case 4: return launch_row_step_t<D, G, 4>(a, s, rows, st, m);
        default: return launch_row_step_t<D, G, 8>(a, s, rows, st, m);
    }
}

template <int D>
static hipError_t launch_row_step_d(int G, int spb, const DecodeArgs &a, const SelectArgs &s, int rows,
                                    hipStream_t st, const KernelMarks &m) {
    switch (G) {
        case 1: return launch_row_step_g<D, 1>(spb, a, s, rows, st, m);
        case 2: return launch_row_step_g<D, 2>(spb, a, s, rows, st, m);
        case 4: return launch_row_step_g<D, 4>(spb, a, s, rows, st, m);
        default: return launch_row_step_g<D, 8>(spb, a, s, rows, st, m);
    }
}

hipError_t launch_row_step(int d, int G, int spb, const DecodeArgs &a, const SelectArgs &s, int rows,
                           hipStream_t st, const KernelMarks &m) {
    return d == 128 ? launch_row_step_d<128>(G, spb, a, s, rows, st, m)
                    : launch_row_step_d<64>(G, spb, a, s, rows, st, m);
}

template <int D, int G>
static hipError_t launch_hit_gather_t(const DecodeArgs &a, const GatherArgs &g, int rows, hipStream_t st) {
    static_assert(kGatherThreads == 256, "the gather role runs in the attention's 256-thread workgroups");
    const size_t dyn = sizeof(int) * (size_t)(g.rows + 1);
    hit_gather_kernel<D, G><<<dim3((unsigned)(kGatherWorkgroups + rows * a.S)), dim3(256), dyn, st>>>(
        a, g, kGatherWorkgroups);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_hit_gather_d(int G, const DecodeArgs &a, const GatherArgs &g, int rows, hipStream_t st) {
    switch (G) {
        case 1: return launch_hit_gather_t<D, 1>(a, g, rows, st);
        case 2: return launch_hit_gather_t<D, 2>(a, g, rows, st);
        case 4: return launch_hit_gather_t<D, 4>(a, g, rows, st);
        default: return launch_hit_gather_t<D, 8>(a, g, rows, st);
    }
}

hipError_t launch_hit_gather(int d, int G, const DecodeArgs &a, const GatherArgs &g, int rows, hipStream_t st) {
    return d == 128 ? launch_hit_gather_d<128>(G, a, g, rows, st) : launch_hit_gather_d<64>(G, a, g, rows, st);
}

// merge: run combine_kernel over the St partial slots after this launch (unless direct).
hipError_t launch_decode(int dtype, int d, int G, const DecodeArgs &a, int rows, hipStream_t st, bool merge,
                         const KernelMarks &m) {
    if (dtype == 1)
        return d == 128 ? launch_decode_d<uint16_t, 128>(G, a, rows, st, merge, m)
                        : launch_decode_d<uint16_t, 64>(G, a, rows, st, merge, m);
    return d == 128 ? launch_decode_d<float, 128>(G, a, rows, st, merge, m)
                    : launch_decode_d<float, 64>(G, a, rows, st, merge, m);
}

}  // namespace nosa
