// pool.hip -- sub-block mean pooling of keys.
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

hipError_t launch_pool(int dtype, int d, const PoolArgs &a, int rows, hipStream_t st) {
    if (dtype == 1) return d == 128 ? launch_pool_t<uint16_t, 128>(a, rows, st) : launch_pool_t<uint16_t, 64>(a, rows, st);
    return d == 128 ? launch_pool_t<float, 128>(a, rows, st) : launch_pool_t<float, 64>(a, rows, st);
}

}  // namespace nosa
