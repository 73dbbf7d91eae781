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
//   QK layout : 4 lanes per token, each holding CPL 16-byte chunks (64 contiguous bytes per
//               token and load); q . K with packed bf16 dot products (fp32 FMAs for fp32 data),
//               reduced over the 4 lanes with two DPP adds.
//   softmax   : scores in the log2 domain (scale * log2 e folded in), block max over the wave's
//               16 tokens (DPP + lane swaps), running max / sum per head, exp2.
//   PV layout : the wave's 16 V rows are loaded as fully contiguous 1 KiB lines; a lane owns one
//               16-byte column chunk of several tokens and accumulates G x (chunk) fp32 outputs.
//               The probabilities travel from the QK layout through 16 x G floats of LDS.
//   Prefetch  : K and V of block j+1 are loaded into registers while block j is computed.
// End of split: lane reduction, a 4-wave merge through LDS, then either the final output
// (S = 1) or a (max, sum, acc) partial in the workspace, merged by combine_kernel (one
// workgroup per row) with the same online-softmax rule.  No workgroup waits on another.
#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

namespace {

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

__device__ __forceinline__ float dot16(const uint4 &a, const uint4 &b, float acc, uint16_t) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
    return acc;
}
__device__ __forceinline__ float dot16(const uint4 &a, const uint4 &b, float acc, float) {
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

template <typename T, int D, int G>
struct WaveState {
    float m[G];                          // running max (log2 domain), wave-uniform
    float lq[G];                         // running sum of p for this lane's QK token
    float acc[G][Geom<T, D>::EPC];       // running sum of p * V for this lane's PV column chunk
};

// One 64-token block: this wave's 16-token slice.
template <typename T, int D, int G>
__device__ __forceinline__ void process_block(WaveState<T, D, G> &st, const uint4 (&qf)[G][Geom<T, D>::CPL],
                                              const uint4 (&kk)[Geom<T, D>::CPL], const uint4 (&vv)[Geom<T, D>::CPL],
                                              float (*pl)[G], float sl2, int sub, int tq, int tpv) {
    using Gm = Geom<T, D>;
    float z[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < Gm::CPL; ++i) s = dot16(qf[h][i], kk[i], s, T());
        s += dpp<kDppQuadXor1>(s);
        s += dpp<kDppQuadXor2>(s);
        z[h] = s * sl2;
    }
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float bm = fmaxf(z[h], dpp<kDppRowRor4>(z[h]));
        bm = fmaxf(bm, dpp<kDppRowRor8>(bm));
        bm = fmaxf(bm, xor_lane(bm, 16));
        bm = fmaxf(bm, xor_lane(bm, 32));
        const float mn = fmaxf(st.m[h], bm);
        alpha[h] = fast_exp2(st.m[h] - mn);
        st.m[h] = mn;
        const float p = fast_exp2(z[h] - mn);
        st.lq[h] = fmaf(st.lq[h], alpha[h], p);
        z[h] = p;
    }
    if (sub == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) pl[tq][h] = z[h];
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < Gm::EPC; ++e) st.acc[h][e] *= alpha[h];
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
            for (int e = 0; e < Gm::EPC; ++e) st.acc[h][e] = fmaf(p[h], v[e], st.acc[h][e]);
    }
    wave_lds_sync();
}

}  // namespace

template <typename T, int D, int G>
__global__ __launch_bounds__(256, (G >= 8 || sizeof(T) * D > 256) ? 1 : 2) void decode_kernel(DecodeArgs a) {
    using Gm = Geom<T, D>;
    constexpr int CPL = Gm::CPL, EPC = Gm::EPC, NC = Gm::NC, RB = Gm::RB, TPI = Gm::TPI;
    __shared__ __align__(16) float p_lds[kWaves][kTokPerWave][G];
    __shared__ float w_m[kWaves][G], w_l[kWaves][G];
    __shared__ __align__(16) float w_acc[kWaves][G][D];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = blockIdx.x / a.S, sp = blockIdx.x - row * a.S;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const int sub = lane & 3, tq = lane >> 2;          // QK layout
    const int cpv = lane % NC, tpv = lane / NC;        // PV layout
    const int j0 = sp * a.nbs, j1 = min(a.k_sel, j0 + a.nbs);

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

    WaveState<T, D, G> st;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.m[h] = -INFINITY;
        st.lq[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) st.acc[h][e] = 0.0f;
    }

    const int32_t *tab = a.table + (size_t)row * a.k_sel;
    uint4 kc[CPL], vc[CPL], kn[CPL], vn[CPL];
    auto load = [&](int j, uint4(&kk)[CPL], uint4(&vv)[CPL]) -> bool {
        const int blk = tab[j];
        if ((unsigned)blk >= (unsigned)a.store_blocks) return false;
        const char *kp = kbase + (size_t)blk * blk_bytes;
        const char *vp = vbase + (size_t)blk * blk_bytes;
#pragma unroll
        for (int i = 0; i < CPL; ++i) kk[i] = *(const uint4 *)(kp + kofs[i]);
#pragma unroll
        for (int i = 0; i < CPL; ++i) vv[i] = *(const uint4 *)(vp + vofs[i]);
        return true;
    };

    float(*pl)[G] = p_lds[w];
    int j = j0;
    bool okc = (j < j1) ? load(j, kc, vc) : false, okn = false;
    while (j < j1) {
        if (j + 1 < j1) okn = load(j + 1, kn, vn);
        if (okc) process_block<T, D, G>(st, qf, kc, vc, pl, a.sl2, sub, tq, tpv);
        if (++j >= j1) break;
        if (j + 1 < j1) okc = load(j + 1, kc, vc);
        if (okn) process_block<T, D, G>(st, qf, kn, vn, pl, a.sl2, sub, tq, tpv);
        ++j;
    }

    // ---- reduce within the wave ----------------------------------------------------------
    float l[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float x = st.lq[h];                  // identical in the 4 lanes of a token
        x += dpp<kDppRowRor4>(x);
        x += dpp<kDppRowRor8>(x);
        x += xor_lane(x, 16);
        x += xor_lane(x, 32);
        l[h] = x;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            float x = st.acc[h][e];
            if (NC <= 8) x += dpp<kDppRowRor8>(x);
            if (NC <= 16) x += xor_lane(x, 16);
            x += xor_lane(x, 32);
            st.acc[h][e] = x;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            w_m[w][h] = st.m[h];
            w_l[w][h] = l[h];
        }
    }
    if (tpv == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPC; ++e) w_acc[w][h][cpv * EPC + e] = st.acc[h][e];
    }
    __syncthreads();

    // ---- merge the 4 waves -----------------------------------------------------------------
    const size_t out_base = (size_t)(b * a.Hq + g * G) * D;
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D, dd = idx - h * D;
        float M = w_m[0][h];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, w_m[ww][h]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = fast_exp2(w_m[ww][h] - M);
            L = fmaf(w_l[ww][h], f, L);
            A = fmaf(w_acc[ww][h][dd], f, A);
        }
        if (a.S == 1) {
            store_elem<T>(a.out, out_base + idx, A / L);
        } else {
            float *part = a.part + ((size_t)(row * a.S + sp) * G + h) * (D + 2);
            part[2 + dd] = A;
            if (dd == 0) {
                part[0] = M;
                part[1] = L;
            }
        }
    }
}

// Merges the S split partials (max, sum, acc) of every row into the output.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const size_t out_base = (size_t)(b * a.Hq + g * G) * D;
    const float *rp = a.part + (size_t)row * a.S * G * (D + 2);
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int h = idx / D, dd = idx - h * D;
        float M = -INFINITY;
        for (int s = 0; s < a.S; ++s) M = fmaxf(M, rp[(size_t)(s * G + h) * (D + 2)]);
        float L = 0.0f, A = 0.0f;
        for (int s = 0; s < a.S; ++s) {
            const float *ps = rp + (size_t)(s * G + h) * (D + 2);
            const float f = fast_exp2(ps[0] - M);
            L = fmaf(ps[1], f, L);
            A = fmaf(ps[2 + dd], f, A);
        }
        store_elem<T>(a.out, out_base + idx, A / L);
    }
}

template <typename T, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, int rows, hipStream_t st) {
    decode_kernel<T, D, G><<<dim3((unsigned)(rows * a.S)), dim3(256), 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.S == 1) return e;
    combine_kernel<T, D, G><<<dim3((unsigned)rows), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(int G, const DecodeArgs &a, int rows, hipStream_t st) {
    switch (G) {
        case 1: return launch_decode_t<T, D, 1>(a, rows, st);
        case 2: return launch_decode_t<T, D, 2>(a, rows, st);
        case 4: return launch_decode_t<T, D, 4>(a, rows, st);
        default: return launch_decode_t<T, D, 8>(a, rows, st);
    }
}

hipError_t launch_decode(int dtype, int d, int G, const DecodeArgs &a, int rows, hipStream_t st) {
    if (dtype == 1) return d == 128 ? launch_decode_d<uint16_t, 128>(G, a, rows, st) : launch_decode_d<uint16_t, 64>(G, a, rows, st);
    return d == 128 ? launch_decode_d<float, 128>(G, a, rows, st) : launch_decode_d<float, 64>(G, a, rows, st);
}

}  // namespace nosa
