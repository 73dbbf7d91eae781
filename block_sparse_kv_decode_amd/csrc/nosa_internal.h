// nosa_internal.h -- launch descriptors shared by the host API (api.cpp) and the kernels.
// Not part of the public ABI (that is include/nosa.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace nosa {

constexpr int kBlockTokens = 64;     // tokens per KV block (the selection / transfer unit)
constexpr int kMaxBlocks = 16384;    // per-row block limit of the selection kernel's LDS

struct PoolArgs {
    const void *k;        // [R, nbmax, 64, d]
    float *kp;            // [R, nbmax * spb, d]
    int n_blocks_max;
    int first_block;
    int n_new;
    int spb;              // sub-blocks per block
    int sbs;              // tokens per sub-block
};

struct AppendArgs {
    const void *k_new, *v_new;   // [R, d] the new token's key / value
    const int32_t *positions;    // [B] index of the new token in each sequence
    void *k_store, *v_store;     // [R, nbmax, 64, d], device addresses
    float *acc;                  // [R, d] running sum of the open sub-block
    float *kp;                   // [R, nbmax * spb, d]
    int Hkv, n_blocks_max, spb, sbs;
};

struct SelectArgs {
    const void *q;        // [B, Hq, d]
    const float *kp;      // [R, nbmax * spb, d]
    const float *ev;      // [R, nbmax]
    int32_t *agn;         // [R, ke]
    int32_t *sel;         // [R, kq + ke]
    float *scores;        // [R, scores_stride] global block scores (parts > 1, or scores-only mode)
    int Hq, Hkv, G;
    int n_blocks, n_blocks_max, kq, ke, n_prev;
    int n_sink, n_window;  // blocks always in the query-agnostic subset (start / end of the context)
    int rows;             // batch x KV heads
    int parts;            // workgroups per row
    int blocks_per_part;
    int scores_only;      // 1: stop after writing block scores
    int no_pick;          // 1: multi-part plan without the Gamma_q kernel (the fused decode step ranks it)
    int scores_stride;
};

struct CacheArgs {
    const int32_t *sel;   // [R, k]
    int32_t *sob;         // [R, nbmax]
    int32_t *bos;         // [R, C]
    int32_t *table;       // [R, k]
    int32_t *mcnt;        // [R]
    int32_t *mlist;       // [R, k, 2]
    int32_t *table_hit;   // optional [R, k]: table with the misses as -1
    int k, C, nbmax;
};

struct GatherArgs {
    const unsigned char *hk, *hv;   // device-mapped pinned host pools [R, nbmax, block_bytes]
    unsigned char *ck, *cv;         // cache [R, C, block_bytes]
    const int32_t *mcnt;
    const int32_t *mlist;
    int rows, k, C, nbmax;
    long long block_bytes;
};
constexpr int kGatherMaxRows = 8192;   // rows (batch x KV heads) one cache update can serve

// Rows longer than this many blocks are scored by 1024-thread workgroups (the row's Gamma_e
// workgroup then ranks with four lanes per key); shorter rows by 256-thread workgroups, twice as
// many per CU.  Measured on MI355X: at 256 blocks per row the 256-thread plan selects in 15.6 us
// against 17.7 us; at 2048 blocks per row the 1024-thread plan takes 22.7 us against 28.0 us.
constexpr int kLongRowBlocks = 1024;

struct UnitsArgs {
    const unsigned char *src;       // device address (device memory or mapped pinned host memory)
    unsigned char *dst;
    const int32_t *src_unit, *dst_unit;
    long long n_units;
    long long n_src, n_dst;         // units in the source / destination buffers
    int chunk_shift;                // log2(unit_bytes / 16)
};

struct DecodeArgs {
    const void *q;        // [B, Hq, d]
    const void *k, *v;    // [R, store_blocks, 64, d]
    const int32_t *table; // row r's entries: table[(r * k_sel + j) * tab_stride], j < k_sel
    void *out;            // [B, Hq, d]
    float *part;          // [R, St, G, d + 2] split partials (max, sum, acc)
    const int32_t *count; // optional [R]: row r uses its first count[r] entries (NULL: all k_sel)
    int Hq, Hkv, k_sel, store_blocks;
    int tab_stride;       // int32 elements from one table entry to the next (1, or 2 for a miss list)
    int S;                // splits per row in this launch
    int nbs;              // blocks per split
    int St, s0;           // partial slots per row; first slot written by this launch
    int direct;           // 1: single split, write the output itself (no partials)
    float sl2;            // softmax scale * log2(e)
};

// Optional timing events recorded on the launch stream immediately before and after the attention
// kernel of a decode launcher (nullptr: none).  The profiling hook of the C ABI arms them.
struct KernelMarks {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Sets the calling thread's error message (nosa_last_error) and returns code.
int api_fail(int code, const char *fmt, ...);

// Each launcher returns hipSuccess or the error of the launch.
hipError_t launch_pool(int dtype, int d, const PoolArgs &a, int rows, hipStream_t st);
hipError_t launch_append(int dtype, int d, const AppendArgs &a, int rows, hipStream_t st);
// fused_threads: workgroup size (256 or 1024) of the one-workgroup-per-row plan (parts == 1);
// part_threads: workgroup size (256 or 1024) of the multi-part scoring kernel.
// The Gamma_q pick of rows scored in parts (pick_kernel), then each row's cache map (one wave).
hipError_t launch_pick_map(const SelectArgs &a, const CacheArgs &c, int rows, hipStream_t st);
hipError_t launch_select(int dtype, int d, int spb, const SelectArgs &a, int rows, int fused_threads, int part_threads,
                         hipStream_t st);
hipError_t launch_cache_map(const CacheArgs &a, int rows, hipStream_t st);
hipError_t launch_gather(const GatherArgs &a, hipStream_t st);
// bf16: the gather (kGatherWorkgroups workgroups) and decode_mfma_kernel's splits over a.table in one
// launch; no merge.
hipError_t launch_hit_gather(int d, int G, const DecodeArgs &a, const GatherArgs &g, int rows, hipStream_t st);
hipError_t launch_gather_units(const UnitsArgs &a, hipStream_t st);
hipError_t launch_decode(int dtype, int d, int G, const DecodeArgs &a, int rows, hipStream_t st, bool merge,
                         const KernelMarks &marks = KernelMarks());
// bf16 decode step after a no_pick selection launch: attention over Gamma_e (S_e splits per row) and
// over Gamma_q ranked in the same launch (S_q splits), then the merge of the S_e + S_q partials.
hipError_t launch_step_decode(int d, int G, const DecodeArgs &a, const SelectArgs &s, int rows, int S_e, int S_q,
                              hipStream_t st, const KernelMarks &marks = KernelMarks());
// bf16 decode step in one workgroup per row: scoring, selection and single-split attention.
hipError_t launch_row_step(int d, int G, int spb, const DecodeArgs &a, const SelectArgs &s, int rows,
                           hipStream_t st, const KernelMarks &marks = KernelMarks());
// Dynamic LDS of the one-workgroup-per-row step (the row's selection state plus its k-entry work
// list) within this bound, which leaves room for two workgroups per CU in the 160 KiB of LDS.
constexpr size_t kRowStepMaxLds = 56 * 1024;
bool row_step_fits(int n_blocks, int k);

}  // namespace nosa
