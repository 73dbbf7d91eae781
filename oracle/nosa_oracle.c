/*
 * nosa_oracle.c -- plain CPU reference of the NOSA decode-step hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The HIP product
 * path never uses it, and it shares no code, header or constant with that path.
 *
 * Source of the method: "NOSA: Native and Offloadable Sparse Attention"
 * (arXiv 2510.13602), as summarised on
 *   [P1] the paperlayer.ai structured summary (sections numbered as on that page), and
 *   [P4] the gist.science explainer, part "Technical summary", Method sections 1 and 2.
 * The pages print no equations; every formula below is the plainest reading of
 * their prose, and each function names the passage it follows.
 *
 * Arithmetic: one accumulator type, acc_t, for every value the method computes.
 * The default build is float32, the precision the oracle's contract names: inputs
 * (fp32, or bf16 bit patterns widened exactly) are used as fp32, and every sum
 * runs sequentially in fp32, in index order.  Compiled with -DORACLE_F64 the same
 * source accumulates in double instead (fp64 inputs then pass through unrounded);
 * the tests hold the two builds against each other to bound the fp32 build's
 * rounding.  No blocking, fusion or reordering.  Rows (batch x KV head) are
 * independent and are spread over OpenMP threads; each row is computed serially,
 * so results do not depend on the thread count.
 *
 * Error convention: functions return 0 on success and a negative number on an
 * input they cannot process (the Python wrapper raises on it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_F64
typedef double acc_t;
#define ACC_EXP exp
#define ACC_BITS 64
#else
typedef float acc_t;
#define ACC_EXP expf
#define ACC_BITS 32
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

/* Bits of the accumulator type the oracle was compiled with (32 or 64). */
int oracle_acc_bits(void)
{
    return ACC_BITS;
}

/* One input element as acc_t: bf16 and fp32 exactly; an fp64 input is rounded in the fp32 build. */
static acc_t elem(const void *p, int dtype, size_t i)
{
    if (dtype == OR_F32)
        return (acc_t)((const float *)p)[i];
    if (dtype == OR_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (acc_t)f;
    }
    return (acc_t)((const double *)p)[i];
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Sub-block mean pooling of keys  ([P1] §3.1; [P4] Method 1, block-wise implementation):
 * the first of the two pooling stages averages the keys of each sub-block.
 *
 *   K  : [rows][n_tokens][d]            (n_tokens = whole blocks)
 *   Kp : [rows][n_tokens / sbs][d]      acc_t
 *   Kp[r][j][c] = (1/sbs) * sum_{t = j*sbs}^{j*sbs+sbs-1} K[r][t][c]
 */
int oracle_pool_keys(int64_t rows, int64_t n_tokens, int d, int sbs,
                     const void *K, int kdtype, acc_t *Kp)
{
    if (rows < 0 || n_tokens < 0 || d <= 0 || sbs <= 0 || n_tokens % sbs != 0)
        return -1;
    const int64_t nsub = n_tokens / sbs;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < nsub; j++) {
            for (int c = 0; c < d; c++) {
                acc_t sum = 0;
                for (int t = 0; t < sbs; t++)
                    sum += elem(K, kdtype, ((size_t)r * n_tokens + (size_t)(j * sbs + t)) * d + c);
                Kp[((size_t)r * nsub + j) * d + c] = sum / (acc_t)sbs;
            }
        }
    }
    return 0;
}

/*
 * Query-aware block scores  ([P1] §2.1 query-key similarity scoring; [P1] §3.1 and
 * [P4] Method 1: mean pooling over sub-blocks, then max pooling to the block).
 *
 * Reading for grouped-query attention (the pages are silent): every query head of
 * a KV-head group scores the group's pooled keys, and the group's sub-block score is
 * the sum of its heads' dot products; the block score is the maximum over the
 * block's sub-blocks.  No scale and no softmax (a positive scale keeps the ranks).
 *
 *   q  : [B][Hq][d]       Kp : [B*Hkv][kp_stride][d] (acc_t, from oracle_pool_keys)
 *   s  : [B*Hkv][n_blocks] acc_t
 *   u[j]  = sum_{h = g*G}^{g*G+G-1} ( sum_c q[b][h][c] * Kp[b,g][j][c] )
 *   s[i]  = max_{j = i*spb}^{i*spb+spb-1} u[j]
 */
int oracle_block_scores(int B, int Hq, int Hkv, int d, int n_blocks, int spb,
                        const void *q, int qdtype, const acc_t *Kp, int64_t kp_stride,
                        acc_t *s)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || n_blocks < 0 || spb <= 0 ||
        kp_stride < (int64_t)n_blocks * spb)
        return -1;
    const int G = Hq / Hkv;
    const int64_t R = (int64_t)B * Hkv;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        const int b = (int)(r / Hkv), g = (int)(r % Hkv);
        for (int i = 0; i < n_blocks; i++) {
            acc_t best = 0;
            for (int jj = 0; jj < spb; jj++) {
                const int64_t j = (int64_t)i * spb + jj;
                acc_t u = 0;
                for (int h = g * G; h < g * G + G; h++) {
                    acc_t dot = 0;
                    for (int c = 0; c < d; c++)
                        dot += elem(q, qdtype, ((size_t)b * Hq + h) * d + c) *
                               Kp[((size_t)r * kp_stride + j) * d + c];
                    u += dot;
                }
                if (jj == 0 || u > best)
                    best = u;
            }
            s[(size_t)r * n_blocks + i] = best;
        }
    }
    return 0;
}

/*
 * Top-kk of the candidates by (key descending, block id ascending), found the plain
 * way: kk rounds, each taking the best candidate not yet chosen.  Scanning ids in
 * ascending order with a strict comparison keeps the lower id on equal keys.
 * Returns 0, or -1 if fewer than kk candidates exist.
 */
static int topk_plain(int n, const acc_t *key, const uint8_t *cand, int kk, uint8_t *chosen)
{
    for (int round = 0; round < kk; round++) {
        int best = -1;
        for (int i = 0; i < n; i++) {
            if (!cand[i] || chosen[i])
                continue;
            if (best < 0 || key[i] > key[best])
                best = i;
        }
        if (best < 0)
            return -1;
        chosen[best] = 1;
    }
    return 0;
}

/*
 * Block selection for one decode step.
 *
 * Query-agnostic subset Gamma_e ([P1] §2.1 and §1; [P4] Method 1, dual selection with
 * strict eviction): ke blocks.  Optionally ([P1] B.2.2: the query-agnostic blocks of the
 * paper's setting include one attention-sink block and a sliding window of recent blocks)
 * the first n_sink blocks and the last n_window visible blocks always belong to Gamma_e;
 * the other ke - n_sink - n_window members are ranked by the fixed eviction score e under
 * strict eviction: a block that is not in Gamma_e at some step never enters it again.
 *   - n_prev == 0 (first step): candidates are all visible blocks outside sink and window.
 *   - otherwise: candidates are the previous score-ranked members (blocks of Gamma_e(t-1)
 *     that were neither sink nor window then, i.e. below n_prev - n_window) and the blocks
 *     that left the window (or became visible past it) since the previous step,
 *     [n_prev - n_window, n_blocks - n_window).  Every other block was left out at an
 *     earlier step and stays out.
 * Query-aware subset Gamma_q ([P1] §2.1 and App. A; [P4] Method 1): the kq blocks with the
 * highest block score s among the visible blocks outside Gamma_e, so Gamma_e and Gamma_q
 * are disjoint and the selection holds exactly k = kq + ke blocks (reading: Gamma_e is
 * formed first, then Gamma_q from its complement).
 * Ties on e or s go to the lower block id.
 *
 *   s         : [R][n_blocks] acc_t         e : [R][e_stride] float32 (first n_blocks used)
 *   agn_state : [R][ke] int32  in: Gamma_e(t-1) (ignored when n_prev == 0); out: Gamma_e(t), ascending
 *   selected  : [R][kq+ke] int32 out: Gamma_e(t) U Gamma_q(t), ascending
 *   is_agn    : [R][kq+ke] uint8 out (may be NULL): 1 where selected[i] came from Gamma_e
 * Requires n_sink + n_window <= ke, n_blocks >= n_sink + n_window, and n_prev == 0 or
 * n_prev >= n_sink + n_window.
 */
int oracle_select_sw(int64_t R, int n_blocks, int kq, int ke, int n_sink, int n_window, int n_prev,
                     const acc_t *s, const float *e, int64_t e_stride,
                     int32_t *agn_state, int32_t *selected, uint8_t *is_agn)
{
    const int k = kq + ke;
    if (R < 0 || n_blocks <= 0 || kq < 0 || ke < 0 || k <= 0 || k > n_blocks || n_prev < 0 ||
        n_prev > n_blocks || e_stride < n_blocks || n_sink < 0 || n_window < 0 ||
        n_sink + n_window > ke || n_blocks < n_sink + n_window ||
        (n_prev > 0 && n_prev < n_sink + n_window))
        return -1;
    const int n_dyn = ke - n_sink - n_window;
    int status = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : status)
    for (int64_t r = 0; r < R; r++) {
        uint8_t *prevE = calloc((size_t)n_blocks, 1);
        uint8_t *candE = calloc((size_t)n_blocks, 1);
        uint8_t *inE = calloc((size_t)n_blocks, 1);
        uint8_t *candQ = calloc((size_t)n_blocks, 1);
        uint8_t *inQ = calloc((size_t)n_blocks, 1);
        acc_t *ekey = malloc(sizeof(acc_t) * (size_t)n_blocks);
        int bad = (!prevE || !candE || !inE || !candQ || !inQ || !ekey);
        if (!bad) {
            for (int i = 0; i < n_blocks; i++)
                ekey[i] = (acc_t)e[(size_t)r * e_stride + i];   /* exact: fp32 values */
            if (n_prev > 0) {
                for (int j = 0; j < ke; j++) {
                    int id = agn_state[(size_t)r * ke + j];
                    if (id < 0 || id >= n_prev)
                        bad = 1;
                    else
                        prevE[id] = 1;
                }
            }
            for (int i = 0; i < n_blocks; i++) {
                const int fixed = (i < n_sink) || (i >= n_blocks - n_window);
                if (fixed) {
                    inE[i] = 1;
                    continue;
                }
                if (n_prev == 0)
                    candE[i] = 1;
                else if (i < n_prev - n_window)
                    candE[i] = prevE[i];
                else
                    candE[i] = 1;   /* left the window, or visible past it, since the last step */
            }
        }
        if (!bad && topk_plain(n_blocks, ekey, candE, n_dyn, inE) != 0)
            bad = 1;
        if (!bad) {
            for (int i = 0; i < n_blocks; i++)
                candQ[i] = !inE[i];
            if (topk_plain(n_blocks, s + (size_t)r * n_blocks, candQ, kq, inQ) != 0)
                bad = 1;
        }
        if (!bad) {
            int ne = 0, ns = 0;
            for (int i = 0; i < n_blocks; i++) {
                if (inE[i])
                    agn_state[(size_t)r * ke + ne++] = i;
                if (inE[i] || inQ[i]) {
                    if (is_agn)
                        is_agn[(size_t)r * k + ns] = inE[i];
                    selected[(size_t)r * k + ns++] = i;
                }
            }
        }
        free(prevE);
        free(candE);
        free(inE);
        free(candQ);
        free(inQ);
        free(ekey);
        if (bad)
            status = -2;
    }
    return status;
}

/* The selection without sink and window blocks: every query-agnostic member is score-ranked. */
int oracle_select(int64_t R, int n_blocks, int kq, int ke, int n_prev,
                  const acc_t *s, const float *e, int64_t e_stride,
                  int32_t *agn_state, int32_t *selected, uint8_t *is_agn)
{
    return oracle_select_sw(R, n_blocks, kq, ke, 0, 0, n_prev, s, e, e_stride, agn_state, selected, is_agn);
}

/*
 * One cache step against a GPU block cache of C slots per row ([P1] §4: a set difference
 * between the previous and the new selection gives a replacement mapping, and only
 * blocks not used at the current step are swapped out; [P1] App. A: selection, then
 * transfer of cache-missed blocks, then attention).
 *
 * Reading of the replacement mapping (the pages give no listing): hits are selected
 * blocks already resident; misses are the other selected blocks, in ascending id; free
 * slots are the slots that are empty or hold a block outside the new selection, in
 * ascending slot index; the i-th miss goes to the i-th free slot.
 *
 *   selected      : [R][k]      ascending block ids
 *   slot_of_block : [R][nbmax]  in/out, -1 = not resident
 *   block_of_slot : [R][C]      in/out, -1 = empty
 *   table         : [R][k]      out: slot holding selected[i]
 *   miss_cnt      : [R]         out
 *   miss_list     : [R][k][2]   out: (block, slot) for the first miss_cnt entries
 */
int oracle_cache_step(int64_t R, int k, int C, int nbmax, const int32_t *selected,
                      int32_t *slot_of_block, int32_t *block_of_slot, int32_t *table,
                      int32_t *miss_cnt, int32_t *miss_list)
{
    if (R < 0 || k <= 0 || C < k || nbmax <= 0)
        return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : status)
    for (int64_t r = 0; r < R; r++) {
        const int32_t *sel = selected + (size_t)r * k;
        int32_t *sob = slot_of_block + (size_t)r * nbmax;
        int32_t *bos = block_of_slot + (size_t)r * C;
        uint8_t *in_sel = calloc((size_t)nbmax, 1);
        int *misses = malloc(sizeof(int) * (size_t)k);
        int *free_slots = malloc(sizeof(int) * (size_t)C);
        int bad = (!in_sel || !misses || !free_slots);
        int nmiss = 0, nfree = 0;
        for (int i = 0; !bad && i < k; i++) {
            if (sel[i] < 0 || sel[i] >= nbmax)
                bad = 1;
            else
                in_sel[sel[i]] = 1;
        }
        for (int i = 0; !bad && i < k; i++) {
            const int slot = sob[sel[i]];
            if (slot >= 0)
                table[(size_t)r * k + i] = slot;   /* hit */
            else
                misses[nmiss++] = i;               /* miss, ascending id */
        }
        for (int slot = 0; !bad && slot < C; slot++) {
            const int ob = bos[slot];
            if (ob < 0 || !in_sel[ob])
                free_slots[nfree++] = slot;
        }
        if (!bad && nfree < nmiss)
            bad = 1;
        for (int m = 0; !bad && m < nmiss; m++) {
            const int i = misses[m], blk = sel[i], slot = free_slots[m];
            const int ob = bos[slot];
            if (ob >= 0)
                sob[ob] = -1;
            sob[blk] = slot;
            bos[slot] = blk;
            table[(size_t)r * k + i] = slot;
            miss_list[((size_t)r * k + m) * 2 + 0] = blk;
            miss_list[((size_t)r * k + m) * 2 + 1] = slot;
        }
        if (!bad)
            miss_cnt[r] = nmiss;
        free(in_sel);
        free(misses);
        free(free_slots);
        if (bad)
            status = -2;
    }
    return status;
}

/*
 * Host-to-GPU transfer of the missed blocks ([P1] §4: fine-grained block transfers from
 * host memory): every (block, slot) pair of the miss list copies the block's bytes from
 * the host pool into the cache slot.
 *
 *   host  : [R][nbmax][block_bytes]   cache : [R][C][block_bytes]
 */
int oracle_gather(int64_t R, int k, int C, int nbmax, int64_t block_bytes,
                  const int32_t *miss_cnt, const int32_t *miss_list,
                  const uint8_t *host, uint8_t *cache)
{
    if (R < 0 || k <= 0 || C <= 0 || nbmax <= 0 || block_bytes <= 0)
        return -1;
    int status = 0;
    for (int64_t r = 0; r < R; r++) {
        for (int m = 0; m < miss_cnt[r]; m++) {
            const int blk = miss_list[((size_t)r * k + m) * 2 + 0];
            const int slot = miss_list[((size_t)r * k + m) * 2 + 1];
            if (blk < 0 || blk >= nbmax || slot < 0 || slot >= C) {
                status = -2;
                continue;
            }
            memcpy(cache + ((size_t)r * C + slot) * block_bytes,
                   host + ((size_t)r * nbmax + blk) * block_bytes, (size_t)block_bytes);
        }
    }
    return status;
}

/*
 * Attention of one decode query over the selected blocks only ([P1] App. A: attention with
 * the KV cache after selection; the pages give no formula, so the standard scaled
 * dot-product attention is read, restricted to the tokens of the selected blocks).
 * Gather form: the tokens of the blocks named by `table`, in table order.
 *
 *   q     : [B][Hq][d]                      query head h reads KV head g = h / (Hq/Hkv)
 *   Ks,Vs : [B*Hkv][store_blocks][bs][d]    table : [B*Hkv][k] indices into the store
 *   out   : [B][Hq][d] acc_t
 *   z_t = scale * q.K_t ;  w_t = exp(z_t - max z) ;  out = sum_t w_t V_t / sum_t w_t
 */
int oracle_attention(int B, int Hq, int Hkv, int d, int bs, int k, int store_blocks,
                     const void *q, int qdtype, const void *Ks, const void *Vs, int kvdtype,
                     const int32_t *table, double scale, acc_t *out)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || bs <= 0 || k <= 0 ||
        store_blocks <= 0)
        return -1;
    const int G = Hq / Hkv;
    const int T = k * bs;
    const acc_t sc = (acc_t)scale;
    int status = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : status)
    for (int64_t bh = 0; bh < (int64_t)B * Hq; bh++) {
        const int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / G;
        const int64_t r = (int64_t)b * Hkv + g;
        acc_t *z = malloc(sizeof(acc_t) * (size_t)T);
        if (!z) {
            status = -2;
            continue;
        }
        int bad = 0;
        for (int i = 0; i < k && !bad; i++) {
            const int blk = table[(size_t)r * k + i];
            if (blk < 0 || blk >= store_blocks) {
                bad = 1;
                break;
            }
            for (int t = 0; t < bs; t++) {
                const size_t kv = (((size_t)r * store_blocks + blk) * bs + t) * d;
                acc_t dot = 0;
                for (int c = 0; c < d; c++)
                    dot += elem(q, qdtype, (size_t)bh * d + c) * elem(Ks, kvdtype, kv + c);
                z[i * bs + t] = sc * dot;
            }
        }
        if (!bad) {
            acc_t m = z[0];
            for (int t = 1; t < T; t++)
                if (z[t] > m)
                    m = z[t];
            acc_t l = 0;
            for (int t = 0; t < T; t++) {
                z[t] = ACC_EXP(z[t] - m);
                l += z[t];
            }
            for (int c = 0; c < d; c++) {
                acc_t acc = 0;
                for (int i = 0; i < k; i++) {
                    const int blk = table[(size_t)r * k + i];
                    for (int t = 0; t < bs; t++)
                        acc += z[i * bs + t] *
                               elem(Vs, kvdtype, (((size_t)r * store_blocks + blk) * bs + t) * d + c);
                }
                out[(size_t)bh * d + c] = acc / l;
            }
        } else {
            status = -2;
        }
        free(z);
    }
    return status;
}

/*
 * Second form of the same attention: dense softmax over every token of the first
 * n_blocks blocks, with the logits of tokens outside the selected blocks set to -inf
 * (block mask [B*Hkv][n_blocks], nonzero = selected).  Same reading as oracle_attention.
 */
int oracle_attention_masked(int B, int Hq, int Hkv, int d, int bs, int n_blocks, int store_blocks,
                            const void *q, int qdtype, const void *Ks, const void *Vs, int kvdtype,
                            const uint8_t *mask, double scale, acc_t *out)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || bs <= 0 || n_blocks <= 0 ||
        store_blocks < n_blocks)
        return -1;
    const int G = Hq / Hkv;
    const int N = n_blocks * bs;
    const acc_t sc = (acc_t)scale;
    int status = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : status)
    for (int64_t bh = 0; bh < (int64_t)B * Hq; bh++) {
        const int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / G;
        const int64_t r = (int64_t)b * Hkv + g;
        acc_t *z = malloc(sizeof(acc_t) * (size_t)N);
        if (!z) {
            status = -2;
            continue;
        }
        for (int t = 0; t < N; t++) {
            if (!mask[(size_t)r * n_blocks + t / bs]) {
                z[t] = -INFINITY;
                continue;
            }
            const size_t kv = ((size_t)r * store_blocks * bs + t) * d;
            acc_t dot = 0;
            for (int c = 0; c < d; c++)
                dot += elem(q, qdtype, (size_t)bh * d + c) * elem(Ks, kvdtype, kv + c);
            z[t] = sc * dot;
        }
        acc_t m = -INFINITY;
        for (int t = 0; t < N; t++)
            if (z[t] > m)
                m = z[t];
        if (m == -INFINITY) {
            status = -2;   /* empty mask */
            free(z);
            continue;
        }
        acc_t l = 0;
        for (int t = 0; t < N; t++) {
            z[t] = ACC_EXP(z[t] - m);   /* exp(-inf) = 0 outside the selection */
            l += z[t];
        }
        for (int c = 0; c < d; c++) {
            acc_t acc = 0;
            for (int t = 0; t < N; t++)
                acc += z[t] * elem(Vs, kvdtype, ((size_t)r * store_blocks * bs + t) * d + c);
            out[(size_t)bh * d + c] = acc / l;
        }
        free(z);
    }
    return status;
}

/*
 * Locality between adjacent steps ([P1] §2.2): the share of the blocks selected at step t
 * that were also selected at step t-1.  With equal-size selections of k blocks,
 * gamma[r] = |prev_r intersect cur_r| / k.
 */
int oracle_locality(int64_t R, int k, int nbmax, const int32_t *prev, const int32_t *cur,
                    double *gamma)
{
    if (R < 0 || k <= 0 || nbmax <= 0)
        return -1;
    int status = 0;
#pragma omp parallel for schedule(static) reduction(min : status)
    for (int64_t r = 0; r < R; r++) {
        uint8_t *was = calloc((size_t)nbmax, 1);
        if (!was) {
            status = -2;
            continue;
        }
        int bad = 0, both = 0;
        for (int i = 0; i < k; i++) {
            const int id = prev[(size_t)r * k + i];
            if (id < 0 || id >= nbmax)
                bad = 1;
            else
                was[id] = 1;
        }
        for (int i = 0; i < k && !bad; i++) {
            const int id = cur[(size_t)r * k + i];
            if (id < 0 || id >= nbmax)
                bad = 1;
            else
                both += was[id];
        }
        gamma[r] = bad ? NAN : (double)both / (double)k;
        free(was);
        if (bad)
            status = -2;
    }
    return status;
}
