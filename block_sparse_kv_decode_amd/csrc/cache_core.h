// cache_core.h -- the GPU block-cache map of one row as a device function, run by one wave: shared
// by the map kernel and by the Gamma_q pick of the one-call offloaded step.
//
// "NOSA: Native and Offloadable Sparse Attention", [P1] paperlayer.ai summary §4: a dedicated
// kernel takes the set difference between the previous and the new selection to build a
// replacement mapping; since cached blocks need not be contiguous on the GPU, only blocks that the
// current step does not use are swapped out.
//
// Hits are found from slot_of_block; misses are ranked in ascending block id with a ballot prefix
// count; free slots (empty, or holding a block not selected now) are ranked in ascending slot order
// from an LDS bitmap of hit slots; the i-th miss takes the i-th free slot.  Deterministic, no global
// atomics.
#pragma once

#include <hip/hip_runtime.h>

#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

// LDS bytes of cache_map_row: a byte per slot, then three int lists of k entries.
__host__ __device__ inline size_t cache_map_lds_bytes(int C, int k) {
    return (size_t)((C + 15) & ~15) + 3 * sizeof(int) * (size_t)k;
}

__device__ __forceinline__ void map_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The map of row `row`, by the 64 lanes of one wave (lane = 0 .. 63); lds: cache_map_lds_bytes(C, k)
// bytes of this wave's own.  The row's selection a.sel must be visible to the wave.
__device__ __forceinline__ void cache_map_row(const CacheArgs &a, int row, int lane, unsigned char *lds) {
    const int k = a.k, C = a.C;
    const int cpad = (C + 15) & ~15;
    uint8_t *held = lds;                        // [C] slot holds a hit
    int *miss_blk = (int *)(lds + cpad);        // [k]
    int *miss_pos = miss_blk + k;               // [k]
    int *free_slot = miss_pos + k;              // [k]

    const int32_t *sel = a.sel + (size_t)row * k;
    int32_t *sob = a.sob + (size_t)row * a.nbmax;
    int32_t *bos = a.bos + (size_t)row * C;
    int32_t *table = a.table + (size_t)row * k;

    for (int s = lane; s < C; s += 64) held[s] = 0;
    map_wave_sync();

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
    map_wave_sync();

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
    map_wave_sync();

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

}  // namespace nosa
