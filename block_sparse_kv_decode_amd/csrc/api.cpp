// api.cpp -- the C ABI of include/nosa.h: host-side validation, workspace layout, launch plans.
//
// Every entry point validates its arguments on the host before it makes any HIP call, so the
// error paths run (and are tested) on machines without a GPU.
#include "nosa.h"

#include <float.h>
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "nosa_internal.h"

using namespace nosa;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return NOSA_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(NOSA_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Rows (batch x KV heads) per call: keeps every grid (rows x splits or parts) within 2^31 workgroups.
constexpr int kMaxRows = 1 << 16;
// Work distribution targets: enough workgroups to give every one of the 256 CUs two of them.
constexpr int kCUs = 256;
constexpr int kTargetWorkgroups = 2 * kCUs;
constexpr int kMinBlocksPerPart = 8;
// A split shorter than this many blocks spends more time filling its load pipeline and merging
// than it saves (measured on MI355X: 4-block splits lose to 8-block splits at 128K context).
constexpr int kMinBlocksPerSplit = 8;
// In the fused decode step the splits over Gamma_q start only after their ranking, and 4-block
// splits fill the chip sooner (measured on MI355X at bs4/128K: 36.4 against 38.6 us per step).
constexpr int kMinBlocksPerFusedSplit = 4;

// Rows the fused decode step takes: their Gamma_q ranking in a 256-thread workgroup must hide under
// the Gamma_e splits' streaming.  Up to 512 blocks the LDS ranking does; up to 2048 blocks (8 per
// thread) with both subsets of at most 64 blocks, the ranking from registers does.
constexpr int kStepMaxBlocks = 512;
constexpr int kStepRegMaxBlocks = 2048;
bool step_rows_fit(const nosa_shape *s) {
    return s->n_blocks <= kStepMaxBlocks || (s->n_blocks <= kStepRegMaxBlocks && s->kq <= 64 && s->ke <= 64);
}

int check_shape(const nosa_shape *s) {
    if (!s) return fail(NOSA_EINVAL, "shape is NULL");
    if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
        return fail(NOSA_EINVAL, "batch, n_q_heads and n_kv_heads must be >= 1");
    if ((long long)s->batch * s->n_kv_heads > kMaxRows)
        return fail(NOSA_EUNSUPPORTED, "batch x n_kv_heads = %lld exceeds %d", (long long)s->batch * s->n_kv_heads,
                    kMaxRows);
    if (s->n_q_heads % s->n_kv_heads != 0)
        return fail(NOSA_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", s->n_q_heads, s->n_kv_heads);
    const int G = s->n_q_heads / s->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(NOSA_EUNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(NOSA_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", s->head_dim);
    if (s->block_size != kBlockTokens)
        return fail(NOSA_EUNSUPPORTED, "block_size must be 64 (got %d)", s->block_size);
    if (s->sub_block_size != 8 && s->sub_block_size != 16 && s->sub_block_size != 32 && s->sub_block_size != 64)
        return fail(NOSA_EUNSUPPORTED, "sub_block_size must be 8, 16, 32 or 64 (got %d)", s->sub_block_size);
    if (s->dtype != NOSA_F32 && s->dtype != NOSA_BF16)
        return fail(NOSA_EUNSUPPORTED, "dtype must be NOSA_F32 or NOSA_BF16 (got %d)", s->dtype);
    if (s->kq < 0 || s->ke < 0 || (long long)s->kq + s->ke < 1)
        return fail(NOSA_EINVAL, "budget kq=%d ke=%d: both >= 0 and kq + ke >= 1", s->kq, s->ke);
    if (s->n_blocks_max < 1 || s->n_blocks_max > kMaxBlocks)
        return s->n_blocks_max < 1 ? fail(NOSA_EINVAL, "n_blocks_max must be >= 1")
                                   : fail(NOSA_EUNSUPPORTED, "n_blocks_max %d exceeds %d", s->n_blocks_max, kMaxBlocks);
    if (s->n_blocks < 1 || s->n_blocks > s->n_blocks_max)
        return fail(NOSA_EINVAL, "n_blocks %d must lie in [1, n_blocks_max=%d]", s->n_blocks, s->n_blocks_max);
    if ((long long)s->kq + s->ke > s->n_blocks)
        return fail(NOSA_EINVAL, "budget kq + ke = %lld exceeds the %d visible blocks", (long long)s->kq + s->ke,
                    s->n_blocks);
    if (s->decode_splits < 0 || s->select_parts < 0)
        return fail(NOSA_EINVAL, "decode_splits and select_parts must be >= 0");
    if (s->sink_blocks < 0 || s->window_blocks < 0 || (long long)s->sink_blocks + s->window_blocks > s->ke)
        return fail(NOSA_EINVAL, "sink_blocks (%d) and window_blocks (%d) must be >= 0 and fit in ke (%d)",
                    s->sink_blocks, s->window_blocks, s->ke);
    if (s->n_blocks < s->sink_blocks + s->window_blocks)
        return fail(NOSA_EINVAL, "n_blocks %d is below sink_blocks + window_blocks", s->n_blocks);
    return NOSA_OK;
}

int rows_of(const nosa_shape *s) { return s->batch * s->n_kv_heads; }
int group_of(const nosa_shape *s) { return s->n_q_heads / s->n_kv_heads; }
int spb_of(const nosa_shape *s) { return s->block_size / s->sub_block_size; }
size_t elem_bytes(const nosa_shape *s) { return s->dtype == NOSA_BF16 ? 2 : 4; }

struct SplitPlan {
    int S;     // splits per row
    int nbs;   // blocks per split
};

SplitPlan decode_plan(const nosa_shape *s, int min_blocks = kMinBlocksPerSplit) {
    const int R = rows_of(s), k = s->kq + s->ke;
    int S = s->decode_splits > 0 ? s->decode_splits : (kTargetWorkgroups + R - 1) / R;
    if (s->decode_splits <= 0 && S > k / min_blocks) S = k / min_blocks;
    if (S < 1) S = 1;
    if (S > k) S = k;
    const int nbs = (k + S - 1) / S;
    S = (k + nbs - 1) / nbs;   // no empty split
    return {S, nbs};
}

struct PartPlan {
    int P;              // workgroups scoring one row
    int bpp;            // blocks per part
    int threads;        // workgroup size of the one-workgroup-per-row plan (P == 1)
    int part_threads;   // workgroup size of the multi-part scoring kernel
};

// Select plan.  Enough rows to fill the chip: one 256-thread workgroup scores and selects a row.
// Fewer rows: short rows are still handled by one (1024-thread) workgroup each; longer rows are
// scored by several workgroups and selected by a second kernel, which keeps every CU streaming
// pooled keys (one workgroup per row would leave most CUs idle; measured on MI355X at 16K context:
// 20 us fused on 128 CUs vs 8 us scoring on all of them).
constexpr size_t kFusedRowBytes = 64 * 1024;

PartPlan select_plan(const nosa_shape *s) {
    const int R = rows_of(s), n = s->n_blocks;
    const int threads = R >= kTargetWorkgroups / 2 ? 256 : 1024;
    const int part_threads = n > kLongRowBlocks ? 512 : 256;
    int P;
    if (s->select_parts > 0) {
        P = s->select_parts;
    } else {
        const size_t row_bytes = (size_t)n * spb_of(s) * s->head_dim * sizeof(float);
        if (threads == 256 || row_bytes <= kFusedRowBytes) {
            P = 1;
        } else if (part_threads == 512) {
            // Long rows: 512-thread parts, two per CU, so that the parts and the row's Gamma_e
            // workgroup fill the 512 workgroup slots at once.  (Measured on MI355X at 2048 blocks
            // per row and 32 rows, one-call step: 15 parts of 512 threads 35.2 us per step, against
            // 36.2 us for 7 parts of 1024 threads, one per CU; with 1024-thread parts, 8 parts,
            // whose last workgroups waited for a free CU, had been slower than 7.)
            P = kTargetWorkgroups / R - 1;
            const int cap = n / kMinBlocksPerPart > 0 ? n / kMinBlocksPerPart : 1;
            if (P > cap) P = cap;
        } else {
            P = (kTargetWorkgroups + R - 1) / R;
            const int cap = n / kMinBlocksPerPart > 0 ? n / kMinBlocksPerPart : 1;
            if (P > cap) P = cap;
        }
    }
    if (P < 1) P = 1;
    if (P > n) P = n;
    const int bpp = (n + P - 1) / P;
    P = (n + bpp - 1) / bpp;
    return {P, bpp, threads, part_threads};
}

struct WsLayout {
    size_t scores, part, tab_hit, total;
};

WsLayout ws_layout(const nosa_shape *s) {
    const size_t R = (size_t)rows_of(s);
    const SplitPlan dp = decode_plan(s), dpf = decode_plan(s, kMinBlocksPerFusedSplit);
    WsLayout L;
    size_t off = 0;
    L.scores = off;
    off = round_up(off + R * (size_t)s->n_blocks_max * sizeof(float), kAlign);
    // With a cache configured, nosa_offload_decode fills 2 S partial slots per row (hits, then
    // misses) and keeps the hit-only table beside them.
    const bool offload = s->cache_slots >= s->kq + s->ke;
    // The fused decode step uses up to S + 1 of its own plan (Gamma_e and Gamma_q splits are rounded
    // up apart).
    size_t slots = (size_t)(dp.S > dpf.S ? dp.S : dpf.S) + 1;
    if (offload && (size_t)(2 * dp.S) > slots) slots = 2 * (size_t)dp.S;
    L.part = off;
    off = round_up(off + R * slots * group_of(s) * (size_t)(s->head_dim + 2) * sizeof(float), kAlign);
    L.tab_hit = off;
    if (offload) off = round_up(off + R * (size_t)(s->kq + s->ke) * sizeof(int32_t), kAlign);
    L.total = off;
    return L;
}

#define REQUIRE_PTR(p, al)                                                                          \
    do {                                                                                            \
        if (!(p)) return fail(NOSA_EINVAL, "%s is NULL", #p);                                       \
        if (!aligned((p), (al))) return fail(NOSA_EINVAL, "%s is not %d-byte aligned", #p, (int)(al)); \
    } while (0)

// Two events per (host thread, device) order the copy stream after the map update and the compute
// stream after the transfer.  Per thread, so that calls made from different host threads never wait
// on each other's events; created on first use and kept for the life of the thread.
struct DeviceEvents {
    hipEvent_t mapped = nullptr, copied = nullptr;
};
constexpr int kMaxDevices = 64;
thread_local DeviceEvents g_events[kMaxDevices];

int get_events(DeviceEvents **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(NOSA_EUNSUPPORTED, "device index %d too large", dev);
    DeviceEvents &d = g_events[dev];
    if (!d.mapped) {
        if ((e = hipEventCreateWithFlags(&d.mapped, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
        if ((e = hipEventCreateWithFlags(&d.copied, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    *out = &d;
    return NOSA_OK;
}

// One-shot pair of timing events per host thread: armed by nosa_profile_next_kernel, recorded
// around the dominant kernel of the next decode call on this thread, then disarmed.
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
thread_local const char *g_prof_kernel = "";

struct ProfileMarks {
    hipEvent_t start = nullptr, stop = nullptr;
    ProfileMarks() {
        start = g_prof_start;
        stop = g_prof_stop;
        g_prof_start = g_prof_stop = nullptr;
        if (start) g_prof_kernel = "";
    }
    // names the kernel the marks bracket (when armed)
    void timed(const char *kernel) const {
        if (start) g_prof_kernel = kernel;
    }
};

}  // namespace

namespace nosa {
int api_fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}
}  // namespace nosa

extern "C" {

const char *nosa_last_error(void) { return g_err; }

const char *nosa_version(void) { return "nosa-mi355x 0.2 (gfx950)"; }

int nosa_host_map(const void *ptr, void **device_address) {
    if (!device_address) return fail(NOSA_EINVAL, "device_address is NULL");
    *device_address = nullptr;
    if (!ptr) return fail(NOSA_EINVAL, "ptr is NULL");
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NOSA_EINVAL, "ptr is neither device memory nor pinned host memory (%s)", hipGetErrorString(e));
    }
    if (attr.type == hipMemoryTypeHost) {
        void *d = nullptr;
        e = hipHostGetDevicePointer(&d, const_cast<void *>(ptr), 0);
        if (e != hipSuccess || !d) {
            (void)hipGetLastError();
            return fail(NOSA_EINVAL, "pinned host memory without a device mapping (%s)", hipGetErrorString(e));
        }
        *device_address = d;
        return ok();
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged || attr.type == hipMemoryTypeUnified) {
        *device_address = const_cast<void *>(ptr);
        return ok();
    }
    return fail(NOSA_EINVAL, "ptr is neither device memory nor pinned host memory");
}

const char *nosa_profile_last_kernel(void) { return g_prof_kernel; }

int nosa_profile_next_kernel(hipEvent_t start, hipEvent_t stop) {
    if ((start == nullptr) != (stop == nullptr)) return fail(NOSA_EINVAL, "start and stop must both be set or both NULL");
    g_prof_start = start;
    g_prof_stop = stop;
    return ok();
}

size_t nosa_workspace_bytes(const nosa_shape *shape) {
    if (check_shape(shape) != NOSA_OK) return 0;
    ok();
    return ws_layout(shape).total;
}

int nosa_pool_keys(const nosa_shape *shape, const void *k, int32_t first_block, int32_t n_new, float *pooled_k,
                   hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    REQUIRE_PTR(k, 16);
    REQUIRE_PTR(pooled_k, 16);
    if (first_block < 0 || n_new < 0 || (long long)first_block + n_new > shape->n_blocks_max)
        return fail(NOSA_EINVAL, "blocks [%d, %d) outside [0, n_blocks_max=%d)", first_block,
                    first_block + n_new, shape->n_blocks_max);
    if (n_new == 0) return ok();
    PoolArgs a;
    a.k = k;
    a.kp = pooled_k;
    a.n_blocks_max = shape->n_blocks_max;
    a.first_block = first_block;
    a.n_new = n_new;
    a.spb = spb_of(shape);
    a.sbs = shape->sub_block_size;
    hipError_t e = launch_pool(shape->dtype, shape->head_dim, a, rows_of(shape), stream);
    return e == hipSuccess ? ok() : hip_fail(e, "pool_keys launch");
}

int nosa_append_kv(const nosa_shape *shape, const void *k_new, const void *v_new, const int32_t *positions,
                   void *k_store, void *v_store, float *pool_acc, float *pooled_k, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    REQUIRE_PTR(k_new, 16);
    REQUIRE_PTR(v_new, 16);
    REQUIRE_PTR(positions, 4);
    REQUIRE_PTR(k_store, 16);
    REQUIRE_PTR(v_store, 16);
    REQUIRE_PTR(pool_acc, 16);
    REQUIRE_PTR(pooled_k, 16);
    AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.positions = positions;
    a.k_store = k_store;
    a.v_store = v_store;
    a.acc = pool_acc;
    a.kp = pooled_k;
    a.Hkv = shape->n_kv_heads;
    a.n_blocks_max = shape->n_blocks_max;
    a.spb = spb_of(shape);
    a.sbs = shape->sub_block_size;
    hipError_t e = launch_append(shape->dtype, shape->head_dim, a, rows_of(shape), stream);
    return e == hipSuccess ? ok() : hip_fail(e, "append_kv launch");
}

int nosa_gather_units(const void *src, int64_t src_units, void *dst, int64_t dst_units, int64_t unit_bytes,
                      const int32_t *src_unit, const int32_t *dst_unit, int64_t n_units, hipStream_t stream) {
    if (unit_bytes < 16 || unit_bytes > (1 << 20) || (unit_bytes & (unit_bytes - 1)) != 0)
        return fail(NOSA_EINVAL, "unit_bytes must be a power of two in [16, 1 MiB] (got %lld)", (long long)unit_bytes);
    if (n_units < 0) return fail(NOSA_EINVAL, "n_units must be >= 0 (got %lld)", (long long)n_units);
    if (src_units < 0 || dst_units < 0) return fail(NOSA_EINVAL, "buffer sizes must be >= 0");
    if (n_units == 0) return ok();
    REQUIRE_PTR(src, 16);
    REQUIRE_PTR(dst, 16);
    REQUIRE_PTR(src_unit, 4);
    REQUIRE_PTR(dst_unit, 4);
    UnitsArgs a;
    a.src = (const unsigned char *)src;
    a.dst = (unsigned char *)dst;
    a.src_unit = src_unit;
    a.dst_unit = dst_unit;
    a.n_units = n_units;
    a.n_src = src_units;
    a.n_dst = dst_units;
    int sh = 0;
    while ((16ll << sh) < unit_bytes) ++sh;
    a.chunk_shift = sh;
    hipError_t e = launch_gather_units(a, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "gather_units launch");
}

// The selection launch(es).  no_pick: the multi-part plan stops after scoring and Gamma_e (the
// fused decode step ranks Gamma_q); *used receives the launch descriptor when not NULL; with
// describe_only nothing is launched (the one-workgroup-per-row step runs the selection itself).
static int run_scores(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                      int32_t n_prev, int32_t *agn_state, int32_t *selected, float *scores_out, void *ws,
                      hipStream_t stream, bool no_pick = false, SelectArgs *used = nullptr,
                      bool describe_only = false) {
    const bool scores_only = scores_out != nullptr;
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(pooled_k, 16);
    REQUIRE_PTR(ws, kAlign);
    if (scores_only) {
        REQUIRE_PTR(scores_out, 4);
    } else {
        REQUIRE_PTR(evict, 4);
        REQUIRE_PTR(selected, 4);
        if (shape->ke > 0) REQUIRE_PTR(agn_state, 4);
        if (n_prev < 0 || n_prev > shape->n_blocks)
            return fail(NOSA_EINVAL, "n_blocks_prev %d must lie in [0, n_blocks=%d]", n_prev, shape->n_blocks);
        if (n_prev > 0 && n_prev < shape->sink_blocks + shape->window_blocks)
            return fail(NOSA_EINVAL, "n_blocks_prev %d is below sink_blocks + window_blocks", n_prev);
    }
    const WsLayout L = ws_layout(shape);
    const PartPlan pp = select_plan(shape);
    SelectArgs a;
    a.q = q;
    a.kp = pooled_k;
    a.ev = evict;
    a.agn = agn_state;
    a.sel = selected;
    a.scores = scores_only ? scores_out : (float *)((char *)ws + L.scores);
    a.Hq = shape->n_q_heads;
    a.Hkv = shape->n_kv_heads;
    a.G = group_of(shape);
    a.n_blocks = shape->n_blocks;
    a.n_blocks_max = shape->n_blocks_max;
    a.kq = shape->kq;
    a.ke = shape->ke;
    a.n_prev = n_prev;
    a.n_sink = shape->sink_blocks;
    a.n_window = shape->window_blocks;
    a.rows = rows_of(shape);
    a.parts = pp.P;
    a.blocks_per_part = pp.bpp;
    a.scores_only = scores_only ? 1 : 0;
    a.no_pick = no_pick ? 1 : 0;
    a.scores_stride = shape->n_blocks_max;
    if (used) *used = a;
    if (describe_only) return NOSA_OK;
    hipError_t e = launch_select(shape->dtype, shape->head_dim, spb_of(shape), a, rows_of(shape), pp.threads,
                                  pp.part_threads, stream);
    return e == hipSuccess ? ok() : hip_fail(e, scores_only ? "block_scores launch" : "select launch");
}

int nosa_block_scores(const nosa_shape *shape, const void *q, const float *pooled_k, float *scores, void *ws,
                      hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!scores) return fail(NOSA_EINVAL, "scores is NULL");
    return run_scores(shape, q, pooled_k, nullptr, 0, nullptr, nullptr, scores, ws, stream);
}

int nosa_select(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, void *ws, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    return run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws, stream);
}

// Validation and launches shared by nosa_cache_update and nosa_offload_decode.  With a distinct
// copy stream the gather runs there, after the map (event), and *copied is set to an event that
// marks its end; the caller makes the compute stream wait on it.
// Validation of the cache step's arguments, and the map's and the gather's kernel arguments.
static int cache_plan(const nosa_shape *shape, const int32_t *selected, int32_t *slot_of_block,
                      int32_t *block_of_slot, int32_t *block_table, int32_t *miss_cnt, int32_t *miss_list,
                      const void *host_k, const void *host_v, void *cache_k, void *cache_v, int32_t *table_hit,
                      CacheArgs *c, GatherArgs *g) {
    const int k = shape->kq + shape->ke;
    if (shape->cache_slots < k)
        return fail(NOSA_ECAPACITY, "cache_slots %d is below the budget kq + ke = %d", shape->cache_slots, k);
    if (shape->cache_slots > kMaxBlocks)
        return fail(NOSA_EUNSUPPORTED, "cache_slots %d exceeds %d", shape->cache_slots, kMaxBlocks);
    if (rows_of(shape) > kGatherMaxRows)
        return fail(NOSA_EUNSUPPORTED, "batch x n_kv_heads = %d exceeds %d for the cache", rows_of(shape),
                    kGatherMaxRows);
    REQUIRE_PTR(selected, 4);
    REQUIRE_PTR(slot_of_block, 4);
    REQUIRE_PTR(block_of_slot, 4);
    REQUIRE_PTR(block_table, 4);
    REQUIRE_PTR(miss_cnt, 4);
    REQUIRE_PTR(miss_list, 4);
    REQUIRE_PTR(host_k, 16);
    REQUIRE_PTR(host_v, 16);
    REQUIRE_PTR(cache_k, 16);
    REQUIRE_PTR(cache_v, 16);
    c->sel = selected;
    c->sob = slot_of_block;
    c->bos = block_of_slot;
    c->table = block_table;
    c->mcnt = miss_cnt;
    c->mlist = miss_list;
    c->table_hit = table_hit;
    c->k = k;
    c->C = shape->cache_slots;
    c->nbmax = shape->n_blocks_max;
    g->hk = (const unsigned char *)host_k;
    g->hv = (const unsigned char *)host_v;
    g->ck = (unsigned char *)cache_k;
    g->cv = (unsigned char *)cache_v;
    g->mcnt = miss_cnt;
    g->mlist = miss_list;
    g->rows = rows_of(shape);
    g->k = k;
    g->C = shape->cache_slots;
    g->nbmax = shape->n_blocks_max;
    g->block_bytes = (long long)shape->block_size * shape->head_dim * (long long)elem_bytes(shape);
    return NOSA_OK;
}

// The launches shared by nosa_cache_update, nosa_offload_decode and nosa_offload_step: the map
// (unless map_done: the caller has run it), then the gather.  With a distinct copy stream the
// gather runs there, after the map (event), and *copied is set to an event that marks its end; the
// caller makes the compute stream wait on it.  With defer the caller launches the gather itself.
static int cache_step(const nosa_shape *shape, const CacheArgs &c, const GatherArgs &g, bool map_done,
                      hipStream_t compute, hipStream_t copy, hipEvent_t *copied, GatherArgs *defer = nullptr) {
    *copied = nullptr;
    hipError_t e;
    if (!map_done && (e = launch_cache_map(c, rows_of(shape), compute)) != hipSuccess)
        return hip_fail(e, "cache_map launch");
    if (defer) {   // the caller launches the gather
        *defer = g;
        return NOSA_OK;
    }
    if (copy == nullptr || copy == compute) {
        e = launch_gather(g, compute);
        return e == hipSuccess ? NOSA_OK : hip_fail(e, "gather launch");
    }
    DeviceEvents *ev = nullptr;
    int rc;
    if ((rc = get_events(&ev)) != NOSA_OK) return rc;
    if ((e = hipEventRecord(ev->mapped, compute)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(copy, ev->mapped, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    if ((e = launch_gather(g, copy)) != hipSuccess) return hip_fail(e, "gather launch");
    if ((e = hipEventRecord(ev->copied, copy)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    *copied = ev->copied;
    return NOSA_OK;
}

static int check_decode_args(const void *q, const void *k_store, const void *v_store, int32_t store_blocks,
                             float softmax_scale, const void *out, const void *ws) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(k_store, 16);
    REQUIRE_PTR(v_store, 16);
    REQUIRE_PTR(out, 16);
    REQUIRE_PTR(ws, kAlign);
    if (store_blocks < 1) return fail(NOSA_EINVAL, "store_blocks must be >= 1 (got %d)", store_blocks);
    if (!(softmax_scale > 0.0f) || !(softmax_scale <= FLT_MAX))   // also rejects NaN and +inf
        return fail(NOSA_EINVAL, "softmax_scale must be a positive finite number");
    return NOSA_OK;
}

static DecodeArgs decode_args(const nosa_shape *shape, const void *q, const void *k_store, const void *v_store,
                              int32_t store_blocks, float softmax_scale, void *out, void *ws) {
    const WsLayout L = ws_layout(shape);
    const SplitPlan sp = decode_plan(shape);
    DecodeArgs a;
    a.q = q;
    a.k = k_store;
    a.v = v_store;
    a.table = nullptr;
    a.out = out;
    a.part = (float *)((char *)ws + L.part);
    a.count = nullptr;
    a.Hq = shape->n_q_heads;
    a.Hkv = shape->n_kv_heads;
    a.k_sel = shape->kq + shape->ke;
    a.store_blocks = store_blocks;
    a.tab_stride = 1;
    a.S = sp.S;
    a.nbs = sp.nbs;
    a.St = sp.S;
    a.s0 = 0;
    a.direct = sp.S == 1;
    a.sl2 = softmax_scale * 1.4426950408889634f;
    return a;
}

int nosa_cache_update(const nosa_shape *shape, const int32_t *selected, int32_t *slot_of_block,
                      int32_t *block_of_slot, int32_t *block_table, int32_t *miss_cnt, int32_t *miss_list,
                      const void *host_k, const void *host_v, void *cache_k, void *cache_v, hipStream_t compute,
                      hipStream_t copy) {
    int rc = check_shape(shape);
    if (rc) return rc;
    CacheArgs c;
    GatherArgs g;
    if ((rc = cache_plan(shape, selected, slot_of_block, block_of_slot, block_table, miss_cnt, miss_list, host_k,
                         host_v, cache_k, cache_v, nullptr, &c, &g)) != NOSA_OK)
        return rc;
    hipEvent_t copied = nullptr;
    if ((rc = cache_step(shape, c, g, false, compute, copy, &copied)) != NOSA_OK) return rc;
    if (copied) {
        hipError_t e = hipStreamWaitEvent(compute, copied, 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }
    return ok();
}

// The offloaded decode after the selection: the map (unless map_done), the gather and the attention
// over the hits, then the misses and one merge.  Arguments validated by the caller.
static int offload_decode_run(const nosa_shape *shape, const void *q, const CacheArgs &c, const GatherArgs &g,
                              bool map_done, const int32_t *miss_list, const int32_t *miss_cnt, void *cache_k,
                              void *cache_v, const int32_t *tab_hit, float softmax_scale, void *out, void *ws,
                              hipStream_t compute, hipStream_t copy) {
    hipEvent_t copied = nullptr;
    // bf16 without a distinct copy stream: the gather and the attention over the hits share one
    // launch on the compute stream, so no cross-stream event separates them (measured on MI355X at
    // bs16/16K with 4.4% misses per step: 0.259 against 0.283 ms per step with the gather on a copy
    // stream)
    const bool one_launch = shape->dtype == NOSA_BF16 && (copy == nullptr || copy == compute);
    GatherArgs gd;
    int rc = cache_step(shape, c, g, map_done, compute, copy, &copied, one_launch ? &gd : nullptr);
    if (rc) return rc;
    // hits: attended while the misses are in transit (partial slots [0, S))
    DecodeArgs a = decode_args(shape, q, cache_k, cache_v, shape->cache_slots, softmax_scale, out, ws);
    a.table = tab_hit;
    a.St = 2 * a.S;
    a.direct = 0;
    const int G = group_of(shape), R = rows_of(shape);
    hipError_t e = one_launch ? launch_hit_gather(shape->head_dim, G, a, gd, R, compute)
                              : launch_decode(shape->dtype, shape->head_dim, G, a, R, compute, false);
    if (e != hipSuccess) return hip_fail(e, "offload_decode hit launch");
    if (copied && (e = hipStreamWaitEvent(compute, copied, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    // misses: their cache slots straight from the miss list (slots [S, 2S)), then one merge
    a.table = miss_list + 1;
    a.tab_stride = 2;
    a.count = miss_cnt;
    a.s0 = a.S;
    e = launch_decode(shape->dtype, shape->head_dim, G, a, R, compute, true);
    return e == hipSuccess ? ok() : hip_fail(e, "offload_decode miss launch");
}

int nosa_offload_decode(const nosa_shape *shape, const void *q, const int32_t *selected, int32_t *slot_of_block,
                        int32_t *block_of_slot, int32_t *block_table, int32_t *miss_cnt, int32_t *miss_list,
                        const void *host_k, const void *host_v, void *cache_k, void *cache_v, float softmax_scale,
                        void *out, void *ws, hipStream_t compute, hipStream_t copy) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_decode_args(q, cache_k, cache_v, shape->cache_slots, softmax_scale, out, ws)) != NOSA_OK) return rc;
    const WsLayout L = ws_layout(shape);
    int32_t *tab_hit = (int32_t *)((char *)ws + L.tab_hit);
    CacheArgs c;
    GatherArgs g;
    if ((rc = cache_plan(shape, selected, slot_of_block, block_of_slot, block_table, miss_cnt, miss_list, host_k,
                         host_v, cache_k, cache_v, tab_hit, &c, &g)) != NOSA_OK)
        return rc;
    return offload_decode_run(shape, q, c, g, false, miss_list, miss_cnt, cache_k, cache_v, tab_hit, softmax_scale,
                              out, ws, compute, copy);
}

int nosa_offload_step(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                      int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, int32_t *slot_of_block,
                      int32_t *block_of_slot, int32_t *block_table, int32_t *miss_cnt, int32_t *miss_list,
                      const void *host_k, const void *host_v, void *cache_k, void *cache_v, float softmax_scale,
                      void *out, void *ws, hipStream_t compute, hipStream_t copy) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_decode_args(q, cache_k, cache_v, shape->cache_slots, softmax_scale, out, ws)) != NOSA_OK) return rc;
    const WsLayout L = ws_layout(shape);
    int32_t *tab_hit = (int32_t *)((char *)ws + L.tab_hit);
    CacheArgs c;
    GatherArgs g;
    if ((rc = cache_plan(shape, selected, slot_of_block, block_of_slot, block_table, miss_cnt, miss_list, host_k,
                         host_v, cache_k, cache_v, tab_hit, &c, &g)) != NOSA_OK)
        return rc;
    SelectArgs sa;
    // validation of the selection's arguments, before anything is launched
    if ((rc = run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws, compute, false,
                         &sa, true)) != NOSA_OK)
        return rc;
    // Rows scored in parts take their Gamma_q pick in a kernel of its own: the rows' cache maps
    // run at its end instead of in a launch of their own.
    const bool fold_map = select_plan(shape).P > 1;
    if (fold_map) {
        if ((rc = run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws, compute,
                             true, &sa)) != NOSA_OK)
            return rc;
        hipError_t e = launch_pick_map(sa, c, rows_of(shape), compute);
        if (e != hipSuccess) return hip_fail(e, "pick_map launch");
    } else if ((rc = run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws,
                                compute)) != NOSA_OK) {
        return rc;
    }
    return offload_decode_run(shape, q, c, g, fold_map, miss_list, miss_cnt, cache_k, cache_v, tab_hit,
                              softmax_scale, out, ws, compute, copy);
}

int nosa_decode_step(const nosa_shape *shape, const void *q, const float *pooled_k, const float *evict,
                     int32_t n_blocks_prev, int32_t *agn_state, int32_t *selected, const void *k_store,
                     const void *v_store, int32_t store_blocks, float softmax_scale, void *out, void *ws,
                     hipStream_t stream) {
    const ProfileMarks pm;   // consumed by this call, whatever its outcome
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_decode_args(q, k_store, v_store, store_blocks, softmax_scale, out, ws)) != NOSA_OK) return rc;
    if (store_blocks < shape->n_blocks)
        return fail(NOSA_EINVAL, "store_blocks %d is below n_blocks %d: the selection would name blocks outside the "
                    "store", store_blocks, shape->n_blocks);
    const KernelMarks km{pm.start, pm.stop};
    const PartPlan pp = select_plan(shape);
    const SplitPlan dp = decode_plan(shape);
    // The pick moves into the attention launch when the selection would otherwise need its own
    // Gamma_q kernel (multi-part plan), for bf16 rows with both subsets non-empty.
    const bool fused = shape->dtype == NOSA_BF16 && pp.P > 1 && shape->kq > 0 && shape->ke > 0 && step_rows_fit(shape);
    // One workgroup per row does it all when it would both score-and-select the row and attend it
    // in a single split anyway.
    const bool row_fused = shape->dtype == NOSA_BF16 && pp.P == 1 && pp.threads == 256 && dp.S == 1 &&
                           row_step_fits(shape->n_blocks, shape->kq + shape->ke);
    if (row_fused) {
        SelectArgs sa;
        if ((rc = run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws, stream,
                             false, &sa, true)))
            return rc;
        DecodeArgs a = decode_args(shape, q, k_store, v_store, store_blocks, softmax_scale, out, ws);
        a.table = selected;
        pm.timed("row_step_kernel");
        hipError_t e = launch_row_step(shape->head_dim, group_of(shape), spb_of(shape), a, sa, rows_of(shape),
                                       stream, km);
        return e == hipSuccess ? ok() : hip_fail(e, "decode_step launch");
    }
    if (!fused) {
        if ((rc = run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws, stream)))
            return rc;
        DecodeArgs a = decode_args(shape, q, k_store, v_store, store_blocks, softmax_scale, out, ws);
        a.table = selected;
        pm.timed(shape->dtype == NOSA_BF16 ? "decode_mfma_kernel" : "decode_valu_kernel");
        hipError_t e =
            launch_decode(shape->dtype, shape->head_dim, group_of(shape), a, rows_of(shape), stream, true, km);
        return e == hipSuccess ? ok() : hip_fail(e, "decode_step attention launch");
    }
    SelectArgs sa;
    if ((rc = run_scores(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, nullptr, ws, stream, true,
                         &sa)))
        return rc;
    DecodeArgs a = decode_args(shape, q, k_store, v_store, store_blocks, softmax_scale, out, ws);
    const SplitPlan fp = decode_plan(shape, kMinBlocksPerFusedSplit);
    const int S_e = (shape->ke + fp.nbs - 1) / fp.nbs, S_q = (shape->kq + fp.nbs - 1) / fp.nbs;
    a.nbs = fp.nbs;
    a.table = nullptr;
    a.S = S_e + S_q;
    a.St = S_e + S_q;
    a.s0 = 0;
    a.direct = 0;
    pm.timed("step_decode_kernel");
    hipError_t e = launch_step_decode(shape->head_dim, group_of(shape), a, sa, rows_of(shape), S_e, S_q, stream, km);
    return e == hipSuccess ? ok() : hip_fail(e, "decode_step launch");
}

int nosa_sparse_decode(const nosa_shape *shape, const void *q, const void *k_store, const void *v_store,
                       int32_t store_blocks, const int32_t *block_table, float softmax_scale, void *out, void *ws,
                       hipStream_t stream) {
    const ProfileMarks pm;   // consumed by this call, whatever its outcome
    int rc = check_shape(shape);
    if (rc) return rc;
    REQUIRE_PTR(block_table, 4);
    if ((rc = check_decode_args(q, k_store, v_store, store_blocks, softmax_scale, out, ws)) != NOSA_OK) return rc;
    DecodeArgs a = decode_args(shape, q, k_store, v_store, store_blocks, softmax_scale, out, ws);
    a.table = block_table;
    pm.timed(shape->dtype == NOSA_BF16 ? "decode_mfma_kernel" : "decode_valu_kernel");
    hipError_t e = launch_decode(shape->dtype, shape->head_dim, group_of(shape), a, rows_of(shape), stream, true,
                                 KernelMarks{pm.start, pm.stop});
    return e == hipSuccess ? ok() : hip_fail(e, "sparse_decode launch");
}

}  // extern "C"
