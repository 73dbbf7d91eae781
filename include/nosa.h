/*
 * nosa.h -- C ABI of the NOSA decode-step hot path on AMD Instinct MI355X (gfx950).
 *
 * The method is NOSA, "NOSA: Native and Offloadable Sparse Attention" (arXiv 2510.13602),
 * as described on
 *   [P1] the paperlayer.ai structured summary of the paper (sections as numbered there), and
 *   [P4] the gist.science explainer, part "Technical summary", Method sections 1 and 2.
 *
 * One decode step of one attention layer, per sequence b and KV head g (a "row"):
 *   1. score every visible KV block against the query        -> nosa_select    ([P1] §2.1, §3.1)
 *   2. pick k = kq + ke blocks: ke query-agnostic blocks under strict eviction, then the
 *      kq best query-aware blocks among the rest              -> nosa_select    ([P1] §2.1, App. A, App. E)
 *   3. (offloaded KV only) hit/miss check against the GPU block cache, replacement map and
 *      host-to-GPU copy of the missed blocks                  -> nosa_cache_update ([P1] §4, App. A)
 *   4. GQA attention over the tokens of the selected blocks  -> nosa_sparse_decode ([P1] App. A)
 *   1+2+4 in one call on GPU-resident KV                     -> nosa_decode_step
 *   3+4 fused for offloaded KV, with the copy of the missed blocks overlapped with attention over
 *      the blocks already cached                             -> nosa_offload_decode ([P1] §4, App. A)
 * Pooled keys (sub-block means) are state kept next to the KV cache -> nosa_pool_keys ([P1] §3.1),
 * extended token by token by the decode append path -> nosa_append_kv.
 *
 * Conventions for every entry point
 *   - All buffers are owned by the caller.  Device pointers point to GPU memory of the current
 *     HIP device.  Host pools are pinned (page-locked) host memory, passed to the per-step calls as
 *     the device address that nosa_host_map returned for them once: the per-step calls make no
 *     pointer query of their own, so they can be captured into a HIP graph in strict mode.  The
 *     library allocates no memory.
 *   - Calls only enqueue work on the given stream(s) and never synchronise the host.
 *   - Shapes, pointers and alignment are validated on the host before any HIP call; a rejected
 *     call returns a negative nosa_status, launches nothing and leaves every buffer untouched.
 *     nosa_last_error() returns a message for the last failure of the calling thread.
 *   - Layouts are dense, row-major, in the order written: [B, Hkv, ...] rows are indexed
 *     r = b * n_kv_heads + g, and query head h belongs to KV head h / (n_q_heads / n_kv_heads).
 *   - Element type of q, K, V and the output: NOSA_BF16 (bfloat16) or NOSA_F32.  Pooled keys,
 *     eviction scores and block scores are float32.  Accumulation is float32 everywhere.
 *   - Supported set: batch x n_kv_heads <= 65536; head_dim 64 or 128; block_size 64;
 *     sub_block_size 8, 16, 32 or 64; n_q_heads / n_kv_heads in {1, 2, 4, 8};
 *     1 <= kq + ke <= n_blocks <= n_blocks_max <= 16384; cache_slots >= kq + ke (for
 *     nosa_cache_update and nosa_offload_decode).  Anything else returns NOSA_EUNSUPPORTED or
 *     NOSA_EINVAL.
 *   - Workspace: nosa_workspace_bytes() bytes of device memory, 256-byte aligned, no initial
 *     contents required (it holds block scores and split-K partials between the kernels of one
 *     call).  Calls that share a workspace must be ordered (same stream, or synchronised);
 *     concurrent calls on one workspace race.
 */
#ifndef NOSA_H
#define NOSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NOSA_OK = 0,
    NOSA_EINVAL = -1,        /* malformed argument: null/misaligned pointer, inconsistent sizes */
    NOSA_EUNSUPPORTED = -2,  /* well-formed but outside the supported set listed above */
    NOSA_ECAPACITY = -3,     /* workspace or cache too small for the request */
    NOSA_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} nosa_status;

typedef enum { NOSA_F32 = 0, NOSA_BF16 = 1 } nosa_dtype;

/* Sizes of one decode step of one attention layer. */
typedef struct {
    int32_t batch;           /* B: sequences decoded together */
    int32_t n_q_heads;       /* Hq: query heads */
    int32_t n_kv_heads;      /* Hkv: KV heads (Hq % Hkv == 0; G = Hq / Hkv heads share one KV head) */
    int32_t head_dim;        /* d */
    int32_t block_size;      /* tokens per KV block: the unit of selection and transfer (64) */
    int32_t sub_block_size;  /* tokens per mean-pooled sub-block (divides block_size) */
    int32_t n_blocks;        /* blocks visible at this step (whole blocks of the context) */
    int32_t n_blocks_max;    /* blocks allocated per row in K/V stores, pooled keys, eviction scores */
    int32_t kq;              /* query-aware budget, blocks */
    int32_t ke;              /* query-agnostic budget, blocks */
    int32_t cache_slots;     /* C: GPU cache slots per row (nosa_cache_update only; else ignored) */
    int32_t dtype;           /* nosa_dtype of q, K, V, output */
    int32_t decode_splits;   /* split-K partitions per row in nosa_sparse_decode; 0 = automatic */
    int32_t select_parts;    /* workgroups that score one row in nosa_select; 0 = automatic */
    int32_t sink_blocks;     /* first blocks always in the query-agnostic subset (0 = none) */
    int32_t window_blocks;   /* most recent visible blocks always in it (0 = none) */
} nosa_shape;

/* Message for the last failed call on this thread ("" if none).  Never NULL. */
const char *nosa_last_error(void);

/* Library build identifier (compile target and version string). */
const char *nosa_version(void);

/*
 * Device address of a caller buffer, resolved once so that the per-step calls need no pointer
 * query ([P1] §4: the transfer kernel reads host memory through unified virtual addressing).
 *   ptr            : device memory (returned as is) or pinned host memory (its device mapping)
 *   device_address : out; NULL on failure
 * Errors: NOSA_EINVAL for NULL arguments, pageable host memory or an unknown pointer.  Call it
 * outside graph capture (it queries the HIP runtime); the address stays valid while the buffer
 * stays allocated.
 */
int nosa_host_map(const void *ptr, void **device_address);

/*
 * Profiling hook.  Arms two HIP events for the next nosa_decode_step or nosa_sparse_decode call on
 * the calling host thread: that call records `start` on its stream immediately before launching its
 * dominant kernel (the attention launch; the whole step when it is one launch) and `stop`
 * immediately after it, before any merge kernel.  The call consumes the pair whatever its outcome;
 * both NULL disarms.  With events created by the caller (e.g. with hipEventDisableSystemFence, so
 * that they do not flush caches), hipEventElapsedTime then gives that kernel's duration on the
 * stream it ran on.  Errors: NOSA_EINVAL if exactly one of the two is NULL.
 */
int nosa_profile_next_kernel(hipEvent_t start, hipEvent_t stop);

/* Name of the kernel that the last call consuming an armed pair bracketed with it (e.g.
 * "step_decode_kernel"), or "" if that call launched nothing.  Per host thread; never NULL. */
const char *nosa_profile_last_kernel(void);

/* Device workspace bytes needed by nosa_select / nosa_block_scores / nosa_sparse_decode /
 * nosa_offload_decode for this shape (the same workspace serves all four; it is larger when
 * cache_slots >= kq + ke, for the offload path).  Returns 0 if the shape is invalid (see
 * nosa_last_error). */
size_t nosa_workspace_bytes(const nosa_shape *shape);

/*
 * Sub-block mean pooling of keys ([P1] §3.1 and [P4] Method 1: the first pooling stage averages
 * the keys of each sub-block).
 *   k        : device, [B, Hkv, n_blocks_max, block_size, d], dtype   (16-byte aligned)
 *   pooled_k : device, [B, Hkv, n_blocks_max * spb, d] float32, spb = block_size / sub_block_size
 * For blocks first_block .. first_block + n_new - 1 (all rows):
 *   pooled_k[r][j][c] = (sum of k over the sub_block_size tokens of sub-block j) / sub_block_size,
 * summed in float32 in token order.  Other entries are untouched.  Requires
 * 0 <= first_block, first_block + n_new <= n_blocks_max, n_new >= 0.
 */
int nosa_pool_keys(const nosa_shape *shape, const void *k, int32_t first_block, int32_t n_new,
                   float *pooled_k, hipStream_t stream);

/*
 * Decode append path: one new token per sequence joins the KV stores and the pooled keys
 * ([P1] §3.1: pooled sub-block keys; [P4] Method 1: strict eviction applies to blocks as they
 * arrive).  For every row r = (b, g), with p = positions[b] (the token's index in sequence b):
 *   k_store[r][p / block_size][p % block_size] = k_new[r], and the same for v;
 *   pool_acc[r] = (p % sub_block_size == 0 ? 0 : pool_acc[r]) + k_new[r]   (float32);
 *   when (p + 1) % sub_block_size == 0: pooled_k[r][p / sub_block_size] = pool_acc[r] / sub_block_size.
 * The sums run in token order from 0, as in nosa_pool_keys, so both give bit-identical pooled keys.
 * A block whose last token is appended becomes visible to nosa_select at the next step (pass the
 * previous n_blocks as n_blocks_prev, so it competes for the query-agnostic subset as an arrival).
 *   k_new, v_new : device, [B, Hkv, d], dtype
 *   positions    : device, [B] int32; rows whose position lies outside [0, n_blocks_max * block_size)
 *                  are skipped
 *   k_store, v_store : [B, Hkv, n_blocks_max, block_size, d], dtype; device memory, or the device
 *                  address (nosa_host_map) of pinned host memory: the offloaded host pool
 *   pool_acc     : device, [B, Hkv, d] float32, running sums of the open sub-blocks (state kept by
 *                  the caller between calls; no initial contents needed)
 *   pooled_k     : device, as in nosa_pool_keys
 */
int nosa_append_kv(const nosa_shape *shape, const void *k_new, const void *v_new, const int32_t *positions,
                   void *k_store, void *v_store, float *pool_acc, float *pooled_k, hipStream_t stream);

/*
 * Query-aware block scores only (the scoring half of nosa_select, exposed for inspection;
 * [P1] §2.1 and §3.1: query-key similarity on mean-pooled sub-blocks, max-pooled per block).
 * For row r = (b, g) and visible block i < n_blocks:
 *   u[j]        = sum over the G query heads h of group g of  q[b][h] . pooled_k[r][j]
 *   scores[r][i] = max of u[j] over the block's sub-blocks j = i*spb .. i*spb + spb - 1
 * (computed as (sum_h q[b][h]) . pooled_k[r][j] in float32; the two agree up to rounding).
 *   q       : device, [B, Hq, d], dtype                 pooled_k : as in nosa_pool_keys
 *   scores  : device, [B, Hkv, n_blocks_max] float32, entries >= n_blocks untouched
 *   ws      : device workspace (see above)
 */
int nosa_block_scores(const nosa_shape *shape, const void *q, const float *pooled_k, float *scores,
                      void *ws, hipStream_t stream);

/*
 * Block selection for one decode step ([P1] §2.1, §3.1, App. A, App. E; [P4] Method 1).
 * Per row, with the block scores s of nosa_block_scores and the fixed per-block eviction scores e:
 *   Query-agnostic subset Gamma_e (ke blocks).  The sink_blocks first blocks and the window_blocks
 *   last visible blocks always belong to it ([P1] B.2.2: the paper's query-agnostic blocks include an
 *   attention sink and a sliding window); the other ke - sink - window members are the blocks with
 *   the highest e among the candidates:
 *     n_blocks_prev == 0 : all visible blocks outside sink and window (first step).
 *     n_blocks_prev  > 0 : the previous score-ranked members (from agn_state on entry) and the
 *                          blocks that left the window, or became visible past it, since then
 *                          ([n_blocks_prev - window, n_blocks - window)).  A block once left out
 *                          of Gamma_e never re-enters it (strict eviction), so consecutive
 *                          selections share at least ke - (blocks that became visible) blocks.
 *   Query-aware subset Gamma_q: the kq visible blocks outside Gamma_e with the highest s.
 *   Ties on e or s go to the lower block id.  The selection is Gamma_e U Gamma_q, k = kq + ke
 *   distinct blocks, written in ascending block id.  Requires sink + window <= ke,
 *   n_blocks >= sink + window, and n_blocks_prev == 0 or n_blocks_prev >= sink + window.
 *   q           : device, [B, Hq, d], dtype
 *   pooled_k    : device, [B, Hkv, n_blocks_max * spb, d] float32 (nosa_pool_keys)
 *   evict       : device, [B, Hkv, n_blocks_max] float32, first n_blocks used; finite values
 *   n_blocks_prev : 0, or the n_blocks of the previous step for this agn_state (<= n_blocks)
 *   agn_state   : device, [B, Hkv, ke] int32, in (when n_blocks_prev > 0) / out: Gamma_e ascending.
 *                 Entries outside [0, n_blocks_prev) on entry are ignored.
 *   selected    : device, [B, Hkv, kq + ke] int32, out: block ids ascending
 *   ws          : device workspace
 * Non-finite q, pooled keys or eviction scores are outside the contract.
 */
int nosa_select(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, void *ws,
                hipStream_t stream);

/*
 * Cache hit/miss check, replacement map and host-to-GPU block transfer for offloaded KV
 * ([P1] §4: set difference of old and new selections into a replacement map, only blocks unused
 * at this step are swapped out, fine-grained block transfers from host memory; [P1] App. A).
 * Per row, against a cache of C = cache_slots slots:
 *   hits   = selected blocks already resident (slot_of_block[blk] >= 0);
 *   misses = the other selected blocks, in ascending block id;
 *   free   = slots that are empty or hold a block not selected now, in ascending slot index;
 *   the i-th miss takes the i-th free slot (its previous block, if any, becomes non-resident).
 *   selected      : device, [B, Hkv, k] int32 ascending (nosa_select output)
 *   slot_of_block : device, [B, Hkv, n_blocks_max] int32, in/out, -1 = not resident
 *   block_of_slot : device, [B, Hkv, C] int32, in/out, -1 = empty (both maps start all -1)
 *   block_table   : device, [B, Hkv, k] int32, out: the slot holding selected[i]
 *   miss_cnt      : device, [B, Hkv] int32, out
 *   miss_list     : device, [B, Hkv, k, 2] int32, out: (block, slot) of the first miss_cnt misses
 *   host_k/host_v : the device addresses (nosa_host_map) of the pinned host pool,
 *                   [B, Hkv, n_blocks_max, block_size, d], dtype, read by the gather kernel
 *   cache_k/cache_v : device, [B, Hkv, C, block_size, d], dtype; missed blocks are copied in
 *   compute       : stream of the map update; copy : stream of the block transfer (may equal
 *                   compute or be NULL = compute).  On return, work later enqueued on `compute`
 *                   is ordered after the transfer.  A distinct copy stream is ordered through two
 *                   HIP events that the library creates once per host thread and device.
 * Selected ids outside [0, n_blocks_max) are skipped.  Maps that are not mutual inverses are
 * outside the contract.
 */
int nosa_cache_update(const nosa_shape *shape, const int32_t *selected, int32_t *slot_of_block,
                      int32_t *block_of_slot, int32_t *block_table, int32_t *miss_cnt,
                      int32_t *miss_list, const void *host_k, const void *host_v, void *cache_k,
                      void *cache_v, hipStream_t compute, hipStream_t copy);

/*
 * GQA sparse attention of one decode query per head over the selected blocks ([P1] App. A;
 * the pages give no formula: standard scaled dot-product attention restricted to the tokens of
 * the selected blocks).  For query head h of sequence b, KV head g = h / G, row r = (b, g):
 *   T      = the block_size tokens of each store block block_table[r][0 .. k-1]
 *   z_t    = softmax_scale * q[b][h] . k_store[r][blk][t]
 *   out[b][h] = sum_t softmax(z)_t * v_store[r][blk][t]
 * computed as split-K flash decoding (online softmax, float32 accumulation).
 *   q        : device, [B, Hq, d], dtype
 *   k_store, v_store : device, [B, Hkv, store_blocks, block_size, d], dtype -- the resident KV
 *              (store_blocks = n_blocks_max, table = selected) or the GPU cache
 *              (store_blocks = cache_slots, table = block_table of nosa_cache_update)
 *   block_table : device, [B, Hkv, k] int32 with k = kq + ke; entries outside [0, store_blocks)
 *              are skipped; a row with no entry inside the store gets an output of 0 (attention
 *              over an empty set of tokens is undefined; 0 is the value that carries nothing)
 *   out      : device, [B, Hq, d], dtype
 *   ws       : device workspace
 */
int nosa_sparse_decode(const nosa_shape *shape, const void *q, const void *k_store,
                       const void *v_store, int32_t store_blocks, const int32_t *block_table,
                       float softmax_scale, void *out, void *ws, hipStream_t stream);

/*
 * One whole decode step on GPU-resident KV: nosa_select followed by nosa_sparse_decode over the
 * selection ([P1] App. A: select, then attend; §2.1 and §3.1 for the selection).  Arguments as for
 * the two calls (table = selected), except that store_blocks must be at least n_blocks (every
 * selected id names a block of the store; NOSA_EINVAL otherwise).  agn_state, selected and out come
 * out as from the two calls:
 * selected and agn_state exactly, out up to float32 summation order.  When the selection would
 * score a row in several workgroups and rank Gamma_q in a kernel of its own (rows of more than
 * 64 KiB of pooled keys and fewer than 256 rows; bf16; kq, ke > 0; n_blocks <= 512, or
 * n_blocks <= 2048 with kq and ke at most 64), the ranking
 * moves into the attention launch instead: the splits over Gamma_e start at once, and each split
 * over Gamma_q ranks the row's Gamma_q itself, so the ranking hides under attention.  When one
 * 256-thread workgroup would both score-and-select a row and attend it in a single split (256 rows
 * or more and a budget that gives one split per row; bf16), the whole step is one launch: each
 * workgroup scores, selects and attends its own row.  Otherwise the step is the two calls.  The
 * workspace is that of nosa_workspace_bytes.
 */
int nosa_decode_step(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                     int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, const void *k_store,
                     const void *v_store, int32_t store_blocks, float softmax_scale, void *out, void *ws,
                     hipStream_t stream);

/*
 * nosa_decode_step for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments and results are those of
 * nosa_decode_step without `ws`: the step's workspace (block scores and split partials) is instead
 * a fixed array of NOSA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from the
 * library's load until the process ends.  The call allocates nothing.  Its first call on a device
 * (with that device current) looks the array's device address up once (hipGetSymbolAddress); make
 * that first call outside graph capture.  The array needs no initial contents and keeps whatever
 * the last call left.  Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different host threads without ordering) race and give undefined
 * results; order them, or use nosa_decode_step with a workspace per stream.
 * Errors: those of nosa_decode_step, and NOSA_ECAPACITY when nosa_workspace_bytes(shape) exceeds
 * NOSA_NOALLOC_SCRATCH_BYTES (checked on the host before any HIP call).
 */
#define NOSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int nosa_decode_step_noalloc(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                             int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, const void *k_store,
                             const void *v_store, int32_t store_blocks, float softmax_scale, void *out,
                             hipStream_t stream);

/*
 * Transfer at a chosen granularity ([P1] §3.2: block-wise against element-wise communication;
 * [P1] §4: the transfer kernel reads pinned host memory through unified virtual addressing).
 * For u < n_units: bytes [src_unit[u] * unit_bytes, +unit_bytes) of src are copied to
 * [dst_unit[u] * unit_bytes, +unit_bytes) of dst.  With unit_bytes = one KV block per head
 * (16 KiB at 64 tokens x d 128 x bf16) this is the block gather of nosa_cache_update; with the
 * bytes of one token's key or value it is an element-wise gather.
 *   src, src_units : device address (nosa_host_map) of pinned host memory, or device memory,
 *               holding src_units units
 *   dst, dst_units : device memory (or the device address of pinned host memory), dst_units units
 *   unit_bytes: power of two in [16, 1 MiB]
 *   src_unit, dst_unit : device, [n_units] int32 unit indices; a pair with either index outside
 *               its buffer is skipped; dst_unit entries must be distinct (else which copy lands is
 *               undefined)
 * n_units == 0 is a no-op.  Errors: NOSA_EINVAL for a bad size or a NULL or misaligned pointer.
 */
int nosa_gather_units(const void *src, int64_t src_units, void *dst, int64_t dst_units, int64_t unit_bytes,
                      const int32_t *src_unit, const int32_t *dst_unit, int64_t n_units, hipStream_t stream);

/*
 * Offloaded decode step after selection: nosa_cache_update, then nosa_sparse_decode over the GPU
 * cache, with the host-to-GPU copy of the missed blocks overlapped with attention over the hit
 * blocks ([P1] §4: cached blocks are used in place and only missed blocks are moved; App. A: the
 * step is selection, transfer, attention).  With `copy` a distinct stream: on `compute` the map
 * kernel, then attention over the hits; on `copy` the gather of the misses; `compute` then waits
 * for the gather, attends the missed blocks and merges the two parts with the online-softmax rule.
 * With copy NULL or equal to compute everything runs on compute, in order: for bf16 the map kernel,
 * then one launch in which a few workgroups gather the misses while the others attend the hits (no
 * cross-stream event between them, the faster form), then the missed blocks and the merge; for
 * fp32 the map, the gather, the hits, the misses and the merge.
 * All arguments are those of nosa_cache_update and nosa_sparse_decode (store_blocks =
 * cache_slots, table = block_table).  slot_of_block, block_of_slot, block_table, miss_cnt,
 * miss_list and the cache contents come out exactly as from nosa_cache_update; `out` equals the
 * nosa_sparse_decode result up to float32 summation order (the split partials are grouped by
 * hit / miss).  The workspace must come from nosa_workspace_bytes of a shape with
 * cache_slots >= kq + ke.  Errors as for the two calls.
 */
int nosa_offload_decode(const nosa_shape *shape, const void *q, const int32_t *selected,
                        int32_t *slot_of_block, int32_t *block_of_slot, int32_t *block_table,
                        int32_t *miss_cnt, int32_t *miss_list, const void *host_k, const void *host_v,
                        void *cache_k, void *cache_v, float softmax_scale, void *out, void *ws,
                        hipStream_t compute, hipStream_t copy);

/*
 * One offloaded decode step in one call: nosa_select, then nosa_offload_decode ([P1] App. A: per
 * step, selection, transfer of the missed blocks, attention; §4: the replacement map from the set
 * difference of the selections).  Arguments: those of nosa_select (q, pooled_k, evict,
 * n_blocks_prev, agn_state, selected) and of nosa_offload_decode (the rest), with the same layouts
 * and ownership; ws from nosa_workspace_bytes of a shape with cache_slots >= kq + ke.  Outputs
 * equal those of the two calls made in order: agn_state, selected, the slot maps, block table,
 * miss list and cache contents bit for bit, `out` up to float32 summation order.  When the rows are
 * scored in parts (the selection's Gamma_q pick is a kernel of its own), each row's cache map runs
 * at the end of its pick instead of in a launch of its own.  Streams as for nosa_offload_decode.
 * Every argument is validated on the host before any launch; errors as for the two calls.
 */
int nosa_offload_step(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                      int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, int32_t *slot_of_block,
                      int32_t *block_of_slot, int32_t *block_table, int32_t *miss_cnt, int32_t *miss_list,
                      const void *host_k, const void *host_v, void *cache_k, void *cache_v, float softmax_scale,
                      void *out, void *ws, hipStream_t compute, hipStream_t copy);

#ifdef __cplusplus
}
#endif

#endif /* NOSA_H */
