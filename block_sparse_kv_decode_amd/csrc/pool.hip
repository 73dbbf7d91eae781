// pool.hip -- sub-block mean pooling of keys, and the per-token append path.
//
// "NOSA: Native and Offloadable Sparse Attention" ([P1] paperlayer.ai summary §3.1; [P4] gist.science
// technical summary, Method 1): block scoring is two-stage, and its first stage averages the keys
// of each sub-block.  The pooled keys are state kept beside the KV cache (built once for the
// prompt and again for every block that fills up), so this kernel is off the per-step path.
//
// One workgroup per (row, block): thread (j, c) sums the sbs tokens of sub-block j at dim c in
// float32, in token order, and scales by 1/sbs (a power of two, so the scaling is exact).
// Reads are coalesced along the head dim.
#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
    const int row = blockIdx.x / a.n_new;
    const int blk = a.first_block + (blockIdx.x - row * a.n_new);
    const size_t kbase = ((size_t)row * a.n_blocks_max + blk) * kBlockTokens * D;
    float *out = a.kp + ((size_t)row * a.n_blocks_max * a.spb + (size_t)blk * a.spb) * D;
    const float inv = 1.0f / (float)a.sbs;
    for (int idx = threadIdx.x; idx < a.spb * D; idx += blockDim.x) {
        const int j = idx / D, c = idx - j * D;
        float s = 0.0f;
        for (int t = 0; t < a.sbs; ++t) s += load_elem<T>(a.k, kbase + (size_t)(j * a.sbs + t) * D + c);
        out[(size_t)j * D + c] = s * inv;
    }
}

template <typename T, int D>
static hipError_t launch_pool_t(const PoolArgs &a, int rows, hipStream_t st) {
    const long long grid = (long long)rows * a.n_new;
    if (grid == 0) return hipSuccess;
    pool_kernel<T, D><<<dim3((unsigned)grid), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

// Decode append path: token positions[b] of every (b, g) row is written into the K and V stores
// (device memory, or pinned host memory through its device mapping), and its key is added to the
// row's running sum of the open sub-block; when the token closes the sub-block, the sum times
// 1/sbs becomes that sub-block's pooled key.  Sums start from 0 and add tokens in order, exactly
// as pool_kernel does, so the two give bit-identical pooled keys.  Rows whose position is out of
// range are skipped.
template <typename T, int D>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.Hkv;
    const int pos = a.positions[b];
    if (pos < 0 || pos >= a.n_blocks_max * kBlockTokens) return;
    const int blk = pos / kBlockTokens, t = pos - blk * kBlockTokens;
    const size_t dst = (((size_t)row * a.n_blocks_max + blk) * kBlockTokens + t) * D;
    const bool first = (pos % a.sbs) == 0, last = ((pos + 1) % a.sbs) == 0;
    const float inv = 1.0f / (float)a.sbs;
    float *kp = a.kp + ((size_t)row * a.n_blocks_max * a.spb + (size_t)(pos / a.sbs)) * D;
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        const T kv = ((const T *)a.k_new)[(size_t)row * D + c];
        const T vv = ((const T *)a.v_new)[(size_t)row * D + c];
        ((T *)a.k_store)[dst + c] = kv;
        ((T *)a.v_store)[dst + c] = vv;
        const float x = load_elem<T>(a.k_new, (size_t)row * D + c);
        const float s = (first ? 0.0f : a.acc[(size_t)row * D + c]) + x;
        a.acc[(size_t)row * D + c] = s;
        if (last) kp[c] = s * inv;
    }
}

template <typename T, int D>
static hipError_t launch_append_t(const AppendArgs &a, int rows, hipStream_t st) {
    append_kernel<T, D><<<dim3((unsigned)rows), dim3(128), 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_append(int dtype, int d, const AppendArgs &a, int rows, hipStream_t st) {
    if (dtype == 1) return d == 128 ? launch_append_t<uint16_t, 128>(a, rows, st) : launch_append_t<uint16_t, 64>(a, rows, st);
    return d == 128 ? launch_append_t<float, 128>(a, rows, st) : launch_append_t<float, 64>(a, rows, st);
}

hipError_t launch_pool(int dtype, int d, const PoolArgs &a, int rows, hipStream_t st) {
    if (dtype == 1) return d == 128 ? launch_pool_t<uint16_t, 128>(a, rows, st) : launch_pool_t<uint16_t, 64>(a, rows, st);
    return d == 128 ? launch_pool_t<float, 128>(a, rows, st) : launch_pool_t<float, 64>(a, rows, st);
}

}  // namespace nosa
