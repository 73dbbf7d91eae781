// gather_core.h -- the host-to-GPU block gather as a device function, shared by the gather kernel
// and by the launch that attends the cache hits while the misses arrive.
//
// "NOSA: Native and Offloadable Sparse Attention", [P1] paperlayer.ai summary §4: a transfer
// kernel moves the missed 16 KiB KV blocks from host memory through unified virtual addressing.
#pragma once

#include <hip/hip_runtime.h>

#include "nosa_internal.h"

namespace nosa {

constexpr int kGatherThreads = 256;
#ifndef NOSA_GATHER_WORKGROUPS
#define NOSA_GATHER_WORKGROUPS 32
#endif
// A few workgroups, each with 16 KiB of host reads in flight, keep the link busy.  Many more
// (one per miss) would park megabytes of slow host reads in the memory queues, where they hold up
// the HBM traffic of the attention kernel that runs beside the gather.
constexpr int kGatherWorkgroups = NOSA_GATHER_WORKGROUPS;

// Persistent gather, run by workgroup wg of nwg.  Every workgroup scans the per-row miss counts into
// LDS (start: rows + 1 ints; wsum: kGatherThreads / 64 ints), then walks the flattened miss list
// (row-major, rank within the row) with stride nwg, finding the row of item t by binary search in
// the scanned counts.  Block bytes are 64 tokens x d x element size, always a multiple of
// 2 x 256 x 16 bytes: each thread moves pairs of 16-byte chunks of K and of V (four loads in flight
// per thread).  Needs kGatherThreads threads.
__device__ __forceinline__ void gather_blocks(const GatherArgs &a, int wg, int nwg, int *start, int *wsum) {
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
    for (int t = wg; t < total; t += nwg) {
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

}  // namespace nosa
