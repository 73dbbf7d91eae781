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
// gather: grid (row, miss index); a workgroup copies one K block and one V block from the
//   device-mapped pinned host pool into the cache slot with 16-byte loads, or exits at once when
//   its index is past the row's miss count.
#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

__global__ __launch_bounds__(64) void cache_map_kernel(CacheArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    const int k = a.k, C = a.C;
    const int cpad = (C + 15) & ~15;
    uint8_t *held = dyn;                        // [C] slot holds a hit
    int *miss_blk = (int *)(dyn + cpad);        // [k]
    int *miss_pos = miss_blk + k;               // [k]
    int *free_slot = miss_pos + k;              // [k]

    const int row = blockIdx.x, lane = threadIdx.x;
    const int32_t *sel = a.sel + (size_t)row * k;
    int32_t *sob = a.sob + (size_t)row * a.nbmax;
    int32_t *bos = a.bos + (size_t)row * C;
    int32_t *table = a.table + (size_t)row * k;

    for (int s = lane; s < C; s += 64) held[s] = 0;
    __syncthreads();

    int nmiss = 0;
    for (int base = 0; base < k; base += 64) {
        const int i = base + lane;
        const bool valid = i < k;
        const int blk = valid ? sel[i] : -1;
        const bool inr = valid && (unsigned)blk < (unsigned)a.nbmax;
        const int slot = inr ? sob[blk] : -1;
        const bool hit = inr && slot >= 0 && slot < C;
        if (hit) held[slot] = 1;
        if (valid) table[i] = hit ? slot : -1;
        const bool miss = inr && !hit;
        const uint64_t mm = __ballot(miss);
        if (miss) {
            const int r = nmiss + lanes_below(mm);
            miss_blk[r] = blk;
            miss_pos[r] = i;
        }
        nmiss += __popcll(mm);
    }
    __syncthreads();

    int nfree = 0;
    for (int base = 0; base < C && nfree < nmiss; base += 64) {
        const int s = base + lane;
        const bool f = s < C && !held[s];
        const uint64_t fm = __ballot(f);
        if (f) {
            const int r = nfree + lanes_below(fm);
            if (r < nmiss) free_slot[r] = s;
        }
        nfree += __popcll(fm);
    }
    __syncthreads();

    const int nuse = min(nmiss, nfree);
    for (int r = lane; r < nuse; r += 64) {
        const int s = free_slot[r], blk = miss_blk[r];
        const int old = bos[s];
        if ((unsigned)old < (unsigned)a.nbmax) sob[old] = -1;
        sob[blk] = s;
        bos[s] = blk;
        table[miss_pos[r]] = s;
        a.mlist[((size_t)row * k + r) * 2 + 0] = blk;
        a.mlist[((size_t)row * k + r) * 2 + 1] = s;
    }
    if (lane == 0) a.mcnt[row] = nuse;
}

constexpr int kGatherThreads = 256;

// Block bytes are 64 tokens x d x element size, always a multiple of 2 x 256 x 16 bytes, so every
// thread moves whole pairs of 16-byte chunks of K and of V (four loads in flight per thread).
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
    const int row = blockIdx.x / a.k, r = blockIdx.x - row * a.k;
    if (r >= a.mcnt[row]) return;
    const int blk = a.mlist[((size_t)row * a.k + r) * 2 + 0];
    const int slot = a.mlist[((size_t)row * a.k + r) * 2 + 1];
    if ((unsigned)blk >= (unsigned)a.nbmax || (unsigned)slot >= (unsigned)a.C) return;
    const size_t src = ((size_t)row * a.nbmax + blk) * (size_t)a.block_bytes;
    const size_t dst = ((size_t)row * a.C + slot) * (size_t)a.block_bytes;
    const uint4 *hk = (const uint4 *)(a.hk + src);
    const uint4 *hv = (const uint4 *)(a.hv + src);
    uint4 *ck = (uint4 *)(a.ck + dst);
    uint4 *cv = (uint4 *)(a.cv + dst);
    const int n16 = (int)(a.block_bytes / 16);
    for (int i = threadIdx.x; i < n16; i += 2 * kGatherThreads) {
        const uint4 k0 = hk[i], k1 = hk[i + kGatherThreads];
        const uint4 v0 = hv[i], v1 = hv[i + kGatherThreads];
        ck[i] = k0;
        ck[i + kGatherThreads] = k1;
        cv[i] = v0;
        cv[i + kGatherThreads] = v1;
    }
}

hipError_t launch_cache_map(const CacheArgs &a, int rows, hipStream_t st) {
    const size_t dyn = (size_t)((a.C + 15) & ~15) + 3 * sizeof(int) * (size_t)a.k;
    if (dyn > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)cache_map_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    cache_map_kernel<<<dim3((unsigned)rows), dim3(64), dyn, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, int rows, hipStream_t st) {
    gather_kernel<<<dim3((unsigned)(rows * a.k)), dim3(kGatherThreads), 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace nosa
