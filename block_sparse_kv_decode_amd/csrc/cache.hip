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
        if (valid && a.table_hit) a.table_hit[(size_t)row * k + i] = hit ? slot : -1;
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
#ifndef NOSA_GATHER_WORKGROUPS
#define NOSA_GATHER_WORKGROUPS 32
#endif
// A few workgroups, each with 16 KiB of host reads in flight, keep the link busy.  Many more
// (one per miss) would park megabytes of slow host reads in the memory queues, where they hold up
// the HBM traffic of the attention kernel that runs beside the gather.
constexpr int kGatherWorkgroups = NOSA_GATHER_WORKGROUPS;

// Persistent gather.  Every workgroup scans the per-row miss counts into LDS, then walks the
// flattened miss list (row-major, rank within the row) with stride gridDim.x, finding the row of
// item t by binary search in the scanned counts.  Block bytes are 64 tokens x d x element size,
// always a multiple of 2 x 256 x 16 bytes: each thread moves pairs of 16-byte chunks of K and of V
// (four loads in flight per thread).
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
    __shared__ int start[kGatherMaxRows + 1];   // start[row] = misses of rows before it
    __shared__ int wsum[kGatherThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int carry = 0;
    for (int base = 0; base < a.rows; base += kGatherThreads) {
        const int row = base + tid;
        const int c = row < a.rows ? min(max(a.mcnt[row], 0), a.k) : 0;
        int x = c;                                   // inclusive scan inside the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        int before = carry;
        for (int ww = 0; ww < w; ++ww) before += wsum[ww];
        if (row < a.rows) start[row] = before + x - c;
        int tot = 0;
        for (int ww = 0; ww < kGatherThreads / 64; ++ww) tot += wsum[ww];
        carry += tot;
        __syncthreads();
    }
    if (tid == 0) start[a.rows] = carry;
    __syncthreads();
    const int total = carry;
    const int n16 = (int)(a.block_bytes / 16);
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        int lo = 0, hi = a.rows - 1;                 // last row with start[row] <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (start[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const int row = lo, r = t - start[row];
        const int blk = a.mlist[((size_t)row * a.k + r) * 2 + 0];
        const int slot = a.mlist[((size_t)row * a.k + r) * 2 + 1];
        if ((unsigned)blk >= (unsigned)a.nbmax || (unsigned)slot >= (unsigned)a.C) continue;
        const size_t src = ((size_t)row * a.nbmax + blk) * (size_t)a.block_bytes;
        const size_t dst = ((size_t)row * a.C + slot) * (size_t)a.block_bytes;
        const uint4 *hk = (const uint4 *)(a.hk + src);
        const uint4 *hv = (const uint4 *)(a.hv + src);
        uint4 *ck = (uint4 *)(a.ck + dst);
        uint4 *cv = (uint4 *)(a.cv + dst);
        for (int i = tid; i < n16; i += 2 * kGatherThreads) {
            const uint4 k0 = hk[i], k1 = hk[i + kGatherThreads];
            const uint4 v0 = hv[i], v1 = hv[i + kGatherThreads];
            ck[i] = k0;
            ck[i + kGatherThreads] = k1;
            cv[i] = v0;
            cv[i + kGatherThreads] = v1;
        }
    }
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
    const size_t dyn = (size_t)((a.C + 15) & ~15) + 3 * sizeof(int) * (size_t)a.k;
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
