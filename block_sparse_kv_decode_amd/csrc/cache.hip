// cache.hip -- GPU block-cache hit/miss check, replacement map, and host-to-GPU block gather.
//
// "NOSA: Native and Offloadable Sparse Attention", [P1] paperlayer.ai summary §4: a dedicated
// kernel takes the set difference between the previous and the new selection to build a
// replacement mapping; since cached blocks need not be contiguous on the GPU, only blocks that
// the current step does not use are swapped out; a transfer kernel moves fine-grained 16 KiB KV
// blocks from host memory through unified virtual addressing.  [P1] App. A: per step, selection,
// then transfer of the missed blocks, then attention.
//
// cache_map: one wave per row.  Hits are found from slot_of_block; misses are ranked in
//   ascending block id with a ballot prefix count; free slots (empty, or holding a block not
//   selected now) are ranked in ascending slot order from an LDS bitmap of hit slots; the i-th
//   miss takes the i-th free slot.  Deterministic, no global atomics.
// gather: a small persistent grid walks the flattened miss list; for each miss a workgroup copies
//   one K block and one V block from the device-mapped pinned host pool into the cache slot with
//   16-byte loads.
#include "cache_core.h"
#include "gather_core.h"
#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

// One wave per row (cache_map_row in cache_core.h).
__global__ __launch_bounds__(64) void cache_map_kernel(CacheArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    cache_map_row(a, blockIdx.x, threadIdx.x, dyn);
}

// Persistent gather (gather_blocks in gather_core.h), on its own.
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
    __shared__ int start[kGatherMaxRows + 1];   // start[row] = misses of rows before it
    __shared__ int wsum[kGatherThreads / 64];
    gather_blocks(a, blockIdx.x, gridDim.x, start, wsum);
}

// Transfer at any granularity: unit u of the source (src_unit[u] * unit_bytes bytes in) goes to
// unit dst_unit[u] of the destination.  The flattened (unit, 16-byte chunk) index space is walked
// with a grid stride, four chunks in flight per thread; unit_bytes is a power of two, so the unit
// and the chunk come from a shift and a mask.  With 16 KiB units this is the block gather's
// traffic pattern; with the 256 bytes of one token's key (or value) it is an element-wise gather.
constexpr int kUnitsThreads = 256;
constexpr int kUnitsWorkgroups = 32;

__global__ __launch_bounds__(kUnitsThreads) void gather_units_kernel(UnitsArgs a) {
    const long long total = a.n_units << a.chunk_shift;
    const long long stride = (long long)gridDim.x * kUnitsThreads;
    const long long cmask = (1ll << a.chunk_shift) - 1;
    for (long long i0 = (long long)blockIdx.x * kUnitsThreads + threadIdx.x; i0 < total; i0 += 4 * stride) {
        uint4 x[4];
        long long dsto[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const long long i = i0 + j * stride;
            dsto[j] = -1;
            if (i < total) {
                const long long u = i >> a.chunk_shift, c = i & cmask;
                const int su = a.src_unit[u], du = a.dst_unit[u];
                if (su >= 0 && su < a.n_src && du >= 0 && du < a.n_dst) {   // out-of-range units are skipped
                    dsto[j] = ((long long)du << a.chunk_shift) + c;
                    x[j] = ((const uint4 *)a.src)[((long long)su << a.chunk_shift) + c];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (dsto[j] >= 0) ((uint4 *)a.dst)[dsto[j]] = x[j];
    }
}

hipError_t launch_gather_units(const UnitsArgs &a, hipStream_t st) {
    if (a.n_units == 0) return hipSuccess;
    const long long chunks = a.n_units << a.chunk_shift;
    long long wgs = (chunks + kUnitsThreads * 4 - 1) / (kUnitsThreads * 4);
    if (wgs > kUnitsWorkgroups) wgs = kUnitsWorkgroups;
    gather_units_kernel<<<dim3((unsigned)wgs), dim3(kUnitsThreads), 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_cache_map(const CacheArgs &a, int rows, hipStream_t st) {
    const size_t dyn = cache_map_lds_bytes(a.C, a.k);
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)cache_map_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    cache_map_kernel<<<dim3((unsigned)rows), dim3(64), dyn, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t st) {
    gather_kernel<<<dim3((unsigned)kGatherWorkgroups), dim3(kGatherThreads), 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace nosa
