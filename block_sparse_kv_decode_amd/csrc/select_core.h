// select_core.h -- the selection machinery shared by the selection kernels and the fused decode
// steps: exact top-k on 64-bit keys, the query-agnostic subset under strict eviction, the
// query-aware subset, the compaction of the outputs, and the pooled-key scoring of a row range.  The method and the algorithms are
// described at the top of select.hip.
#pragma once

#include "nosa_device.h"
#include "nosa_internal.h"

namespace nosa {

namespace {

constexpr int kUnroll = 4;           // groups of eight sub-blocks per wave kept in flight
constexpr int kRankMaxBlocks = 512;  // rows up to this length use the one-pass rank selection
constexpr int kCandMax = 512;        // candidates kept after the chunk-maximum bound
constexpr int kEvPre = 4;            // eviction scores prefetched per thread
constexpr int kScorePer = 4;         // block scores per thread loaded together by a Gamma_q ranking
constexpr int kEvLdsMax = 4096;      // rows up to this length keep their eviction scores in LDS
constexpr int kKeyScratch = 256 + kCandMax;   // uint64 LDS entries of the top-k scratch

// Workgroup barrier for LDS: waits for this wave's LDS accesses only, so global loads a caller
// left in flight (prefetched K/V blocks) stay in flight.  The selection helpers read global
// memory only as input and write it only as output, so LDS is all their barriers must order.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NT>
struct SelectShared {
    uint32_t hist[256];
    int scan[NT / 64];
    int bcast[4];
};

// Inclusive sum over the NT threads of the workgroup, in thread order (all threads call it).
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int *ws) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) ws[w] = v;
    wg_barrier();
    if (NW > 1 && w == 0) {
        int t = lane < NW ? ws[lane] : 0;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const int u = __shfl_up(t, o, 64);
            if (lane >= o) t += u;
        }
        if (lane < NW) ws[lane] = t;   // inclusive prefix of the wave totals
    }
    wg_barrier();
    const int add = w > 0 ? ws[w - 1] : 0;
    wg_barrier();
    return v + add;
}

__device__ __forceinline__ uint64_t composite_key(uint32_t k, int id) {
    return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// Radix select over 32-bit keys: marks the kk best candidates; equal keys go to the lowest ids.
template <int NT, class KeyF, class CandF>
__device__ void topk_radix(int n, int kk, KeyF key, CandF cand, uint8_t *mark, SelectShared<NT> &sh) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int need = kk;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) sh.hist[tid] = 0u;
        if (tid == 0) { sh.bcast[0] = 0; sh.bcast[1] = 0; }
        wg_barrier();
        for (int i = tid; i < n; i += NT) {
            if (cand(i)) {
                const uint32_t kv = key(i);
                if ((kv & pmask) == prefix) atomicAdd(&sh.hist[(kv >> shift) & 255u], 1u);
            }
        }
        wg_barrier();
        const int cnt = tid < 256 ? (int)sh.hist[255 - tid] : 0;
        const int ge = block_incl_scan<NT>(cnt, sh.scan);   // candidates with digit >= 255 - tid
        const int gt = ge - cnt;
        if (tid < 256 && gt < need && need <= ge) { sh.bcast[0] = 255 - tid; sh.bcast[1] = gt; }
        wg_barrier();
        prefix |= (uint32_t)sh.bcast[0] << shift;
        pmask |= 0xFFu << shift;
        need -= sh.bcast[1];
        wg_barrier();
    }
    // prefix is the kk-th largest key; take every larger key and the `need` lowest ids equal to it.
    const uint32_t T = prefix;
    const int per = (n + NT - 1) / NT;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int eq = 0;
    for (int i = lo; i < hi; ++i)
        if (cand(i) && key(i) == T) ++eq;
    int rank = block_incl_scan<NT>(eq, sh.scan) - eq;
    for (int i = lo; i < hi; ++i) {
        if (!cand(i)) continue;
        const uint32_t kv = key(i);
        if (kv > T) {
            mark[i] = 1;
        } else if (kv == T) {
            if (rank < need) mark[i] = 1;
            ++rank;
        }
    }
    wg_barrier();
}

// Marks the kk largest of the m unique keys buf[0..m) (zeros are empty slots): several lanes of a
// wave count, for one key, the keys above it and add their counts with lane swaps, so a row of m
// keys costs m * m / NT comparisons per thread.  mark_id(i, key, rank) is called for each winner.
template <int NT, class MarkF>
__device__ __forceinline__ void rank_mark(const uint64_t *buf, int m, int kk, MarkF mark_id) {
    int tpc = 1;                                     // lanes per key: power of two, <= 64
    while (tpc < 64 && tpc * 2 * m <= NT) tpc *= 2;
    if (tpc == 1) {
        // One lane per key: every lane walks the same keys, so the walk is uniform and sixteen
        // keys come from one LDS address with immediate offsets (broadcast reads).
        for (int i = threadIdx.x; i < m; i += NT) {
            const uint64_t ki = buf[i];
            int cnt = 0;
            int j = 0;
            for (; j + 16 <= m; j += 16) {
                uint64_t b[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) b[u] = buf[j + u];
#pragma unroll
                for (int u = 0; u < 16; ++u) cnt += b[u] > ki ? 1 : 0;
            }
            for (; j < m; ++j) cnt += buf[j] > ki ? 1 : 0;
            if (ki != 0ull && cnt < kk) mark_id(i, ki, cnt);
        }
        return;
    }
    const int r = threadIdx.x & (tpc - 1);
    for (int i = threadIdx.x / tpc; i < m; i += NT / tpc) {
        const uint64_t ki = buf[i];
        int cnt = 0;
        int j = r;
        for (; j + 7 * tpc < m; j += 8 * tpc) {   // eight independent LDS reads in flight
            const uint64_t b0 = buf[j], b1 = buf[j + tpc], b2 = buf[j + 2 * tpc], b3 = buf[j + 3 * tpc];
            const uint64_t b4 = buf[j + 4 * tpc], b5 = buf[j + 5 * tpc], b6 = buf[j + 6 * tpc], b7 = buf[j + 7 * tpc];
            cnt += (b0 > ki) + (b1 > ki) + (b2 > ki) + (b3 > ki) + (b4 > ki) + (b5 > ki) + (b6 > ki) + (b7 > ki);
        }
        for (; j < m; j += tpc) cnt += buf[j] > ki ? 1 : 0;
        for (int o = 1; o < tpc; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
        if (r == 0 && ki != 0ull && cnt < kk) mark_id(i, ki, cnt);
    }
}

// Marks the kk best candidates (key descending, id ascending) in mark[0..n).  Keys are made
// unique by appending the inverted block id (composite_key), so the kk-th best is well defined.
//   n <= 512 : every candidate is ranked against all others (rank_mark).
//   n  > 512 : the row is cut into at most 256 chunks; the kk-th best chunk maximum is a lower bound
//              T0 of the kk-th best key overall (the kk best maxima are distinct keys >= T0), and
//              at most kk chunks hold keys >= T0, so at most kk * chunk candidates survive; they
//              are gathered (in any order: the ranking needs none) and ranked.  Chunks are as long
//              as kCandMax / kk allows, so that few maxima are ranked.  When more than kCandMax
//              survive, a radix select takes over.
// keybuf: LDS scratch of 256 + kCandMax uint64.
template <int NT, class KeyF, class CandF>
__device__ void topk_mark(int n, int kk, KeyF key, CandF cand, uint8_t *mark, uint64_t *keybuf, SelectShared<NT> &sh) {
    if (kk <= 0) return;
    const int tid = threadIdx.x;
    if (n <= kRankMaxBlocks) {
        for (int i = tid; i < n; i += NT) keybuf[i] = cand(i) ? composite_key(key(i), i) : 0ull;
        wg_barrier();
        rank_mark<NT>(keybuf, n, kk, [&](int i, uint64_t, int) { mark[i] = 1; });
        wg_barrier();
        return;
    }
    constexpr int kMaxChunks = 256;
    constexpr int TPCH = NT / kMaxChunks;           // threads per chunk (adjacent lanes)
    uint64_t *tmax = keybuf;                        // [nch] chunk maxima
    uint64_t *cbuf = keybuf + kMaxChunks;           // [kCandMax] surviving candidates
    int csize = kCandMax / kk;                      // at most kk * csize keys survive
    if (csize < (n + kMaxChunks - 1) / kMaxChunks) csize = (n + kMaxChunks - 1) / kMaxChunks;
    const int nch = (n + csize - 1) / csize;        // <= 256
    {
        const int ch = tid / TPCH, part = tid - ch * TPCH;
        const int lo = min(n, ch * csize), hi = min(n, lo + csize);
        uint64_t best = 0ull;
        for (int i = lo + part; i < hi; i += TPCH)
            if (cand(i)) {
                const uint64_t c = composite_key(key(i), i);
                best = c > best ? c : best;
            }
        for (int o = 1; o < TPCH; o <<= 1) {
            const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, 64) << 32) |
                                   (uint32_t)__shfl_xor((int)(uint32_t)best, o, 64);
            best = other > best ? other : best;
        }
        if (part == 0 && ch < nch) tmax[ch] = best;
        if (tid == 0) cbuf[0] = 1ull;   // T0 when fewer than kk chunks hold a candidate: keep all
    }
    wg_barrier();
    // threshold T0: the kk-th best chunk maximum (the maximum ranked kk - 1)
    rank_mark<NT>(tmax, nch, kk, [&](int, uint64_t ki, int rank) {
        if (rank == kk - 1) cbuf[0] = ki;
    });
    wg_barrier();
    const uint64_t T0 = cbuf[0];
    if (tid == 0) sh.bcast[3] = 0;
    wg_barrier();
    const int per = (n + NT - 1) / NT;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int cnt = 0;
    for (int i = lo; i < hi; ++i)
        if (cand(i) && composite_key(key(i), i) >= T0) ++cnt;
    const int pos0 = cnt ? atomicAdd(&sh.bcast[3], cnt) : 0;   // a slot range of cbuf per thread
    wg_barrier();
    const int total = sh.bcast[3];
    if (total <= kCandMax) {
        int pos = pos0;
        for (int i = lo; i < hi; ++i)
            if (cand(i)) {
                const uint64_t c = composite_key(key(i), i);
                if (c >= T0) cbuf[pos++] = c;
            }
        wg_barrier();
        rank_mark<NT>(cbuf, total, kk, [&](int, uint64_t c, int) { mark[0xFFFFFFFFu - (uint32_t)c] = 1; });
        wg_barrier();
        return;
    }
    topk_radix<NT>(n, kk, key, cand, mark, sh);
}

// Writes, in ascending id, the ids i < n with inE[i] to agn[0..ke) and those with inE[i] | inQ[i]
// to sel[0..k), padding with -1: one scan over packed (agnostic, selected) counts.
template <int NT>
__device__ void compact_outputs(int n, const uint8_t *inE, const uint8_t *inQ, int32_t *agn, int ke, int32_t *sel,
                                int k, SelectShared<NT> &sh) {
    const int tid = threadIdx.x;
    const int per = (n + NT - 1) / NT;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int cnt = 0;   // low 16 bits: selected; high 16 bits: agnostic
    for (int i = lo; i < hi; ++i) cnt += ((inE[i] | inQ[i]) != 0 ? 1 : 0) + (inE[i] != 0 ? 0x10000 : 0);
    const int incl = block_incl_scan<NT>(cnt, sh.scan);
    int ps = (incl - cnt) & 0xFFFF, pe = (incl - cnt) >> 16;
    for (int i = lo; i < hi; ++i) {
        if (inE[i]) {
            if (agn && pe < ke) agn[pe] = i;
            ++pe;
        }
        if (inE[i] | inQ[i]) {
            if (sel && ps < k) sel[ps] = i;
            ++ps;
        }
    }
    if (tid == NT - 1) sh.bcast[2] = incl;
    wg_barrier();
    const int ns = sh.bcast[2] & 0xFFFF, ne = sh.bcast[2] >> 16;
    if (sel)
        for (int p = ns + tid; p < k; p += NT) sel[p] = -1;
    if (agn)
        for (int p = ne + tid; p < ke; p += NT) agn[p] = -1;
}

// ---- Gamma_q of a row held in registers ------------------------------------------------------
// For rows of at most kRegPickMax * NT (= 2048) blocks and both subsets of at most 64 blocks.
// Thread t owns the kpt consecutive blocks [t * kpt, t * kpt + kpt), kpt the smallest power of two
// with kpt * NT >= n, and builds their keys in registers straight from the scores in global memory:
// same keys, candidates and tie order as topk_mark, and the same chunk-maximum bound, with chunks of
// up to four threads (at most 64 of them).  The steps work on whole waves with lane ballots rather
// than on per-key counts, and take two workgroup barriers (three with more than 64 survivors):
//   - each wave marks Gamma_e in an LDS bitmap of its own and reads its threads' bits;
//   - after the chunk maxima are in LDS, every wave finds their kq-th best, T0, by a most-significant-
//     bit-first search on ballots (one maximum per lane);
//   - survivors (keys >= T0) are placed with ballots and one LDS atomic per wave;
//   - after the survivors are in LDS, wave 0 takes their kq-th best the same way (one survivor per
//     lane), so the winners are the survivors at or above it, and orders ids through an LDS bitmap
//     of the row with prefix popcounts: Gamma_q ascending into qlist and, when sel is given, the
//     ascending union with Gamma_e into sel.
// The loads are issued unconditionally (indices clamped into the row), Gamma_e ids first, so that
// waiting for the ids waits for nothing else.
constexpr int kRegPickMax = 8;

template <int NT>
__host__ __device__ inline bool reg_pick_fits(int n, int kq, int ke) {
    return n >= 1 && n <= kRegPickMax * NT && n <= 2048 && kq >= 1 && kq <= 64 && ke <= 64;
}

__device__ __forceinline__ uint64_t dpp_max64(uint64_t v, int ctrl_is_xor2) {
    const int lo = (int)(uint32_t)v, hi = (int)(v >> 32);
    const int olo = ctrl_is_xor2 ? __builtin_amdgcn_update_dpp(0, lo, kDppQuadXor2, 0xF, 0xF, false)
                                 : __builtin_amdgcn_update_dpp(0, lo, kDppQuadXor1, 0xF, 0xF, false);
    const int ohi = ctrl_is_xor2 ? __builtin_amdgcn_update_dpp(0, hi, kDppQuadXor2, 0xF, 0xF, false)
                                 : __builtin_amdgcn_update_dpp(0, hi, kDppQuadXor1, 0xF, 0xF, false);
    const uint64_t o = ((uint64_t)(uint32_t)ohi << 32) | (uint32_t)olo;
    return o > v ? o : v;
}

// The kk-th largest of the non-zero keys held one per lane (0 when fewer than kk lanes hold one):
// the kk-th largest high word by a bit-by-bit search on ballots, then, among the lanes with that high
// word, the low word that completes the count.  Keys are unique, so the result is one lane's key.
__device__ __forceinline__ uint64_t wave_kth_largest(uint64_t key, int kk) {
    const bool live = key != 0ull;
    if (kk < 1 || __popcll(__ballot(live)) < kk) return 0ull;
    const uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
    uint32_t vh = 0u;
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = vh | (1u << b);
        if (__popcll(__ballot(live && hi >= c)) >= kk) vh = c;
    }
    const int need = kk - __popcll(__ballot(live && hi > vh));   // >= 1
    const bool eq = live && hi == vh;
    const uint64_t eqm = __ballot(eq);
    uint32_t vl;
    if (__popcll(eqm) == 1) {
        vl = (uint32_t)__builtin_amdgcn_readlane((int)lo, __builtin_ctzll(eqm));
    } else {
        vl = 0u;
        for (int b = 31; b >= 0; --b) {
            const uint32_t c = vl | (1u << b);
            if (__popcll(__ballot(eq && lo >= c)) >= need) vl = c;
        }
    }
    return ((uint64_t)vh << 32) | vl;
}

// Inclusive sum over the 64 lanes of the wave: row shifts, then row broadcasts.
__device__ __forceinline__ int wave_incl_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// Ascending ranks of ids below 2048 held by the lanes of one wave (a lane may hold two: a, b),
// among all ids the wave holds: a 64-word LDS bitmap (word w = ids 32w .. 32w + 31), its prefix
// popcounts, and one lookup per id.  words: 128 LDS words of the calling wave.  Returns -1 for an
// id not held.
__device__ __forceinline__ int2 wave_id_ranks(uint32_t *words, int a, bool ha, int b, bool hb) {
    const int lane = threadIdx.x & 63;
    words[lane] = 0u;
    wave_lds_sync();
    if (ha) atomicOr(&words[a >> 5], 1u << (a & 31));
    if (hb) atomicOr(&words[b >> 5], 1u << (b & 31));
    wave_lds_sync();
    const int c = __popc(words[lane]);
    words[64 + lane] = wave_incl_sum(c) - c;
    wave_lds_sync();
    int2 r = make_int2(-1, -1);
    if (ha) r.x = (int)words[64 + (a >> 5)] + __popc(words[a >> 5] & ((1u << (a & 31)) - 1u));
    if (hb) r.y = (int)words[64 + (b >> 5)] + __popc(words[b >> 5] & ((1u << (b & 31)) - 1u));
    return r;
}

// gscore: the row's n block scores; agn: Gamma_e, ke ids ascending (then -1); keybuf: LDS,
// kKeyScratch entries; qlist: LDS, kq entries; sel: the row's k = kq + ke selection entries in
// global memory, or nullptr.  Returns false, with nothing written to qlist or sel, when more than
// kCandMax blocks pass the bound (workgroup-uniform); the caller then takes the LDS path.  The
// caller synchronises the workgroup before reading qlist.
template <int NT>
__device__ __forceinline__ bool pick_query_regs(const float *gscore, int n, const int32_t *agn, int ke, int kq,
                                                uint64_t *keybuf, int32_t *qlist, int32_t *sel, SelectShared<NT> &sh) {
    static_assert(NT % 64 == 0 && NT <= 256, "per-wave bitmaps must fit in keybuf[64, 192)");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int kpt = n <= NT ? 1 : n <= 2 * NT ? 2 : n <= 4 * NT ? 4 : 8;
    const int base = tid * kpt;
    const int eid = lane < ke ? agn[lane] : -1;
    float sv[kRegPickMax];
#pragma unroll
    for (int j = 0; j < kRegPickMax; ++j) sv[j] = gscore[min(base + min(j, kpt - 1), n - 1)];
    uint64_t *tmax = keybuf;                                  // [<= 64] chunk maxima
    uint32_t *words = (uint32_t *)(keybuf + 64) + wv * 64;    // [64] this wave's Gamma_e bitmap
    int32_t *win = (int32_t *)(keybuf + 192);                 // [64] winner ids by rank (many survivors)
    uint64_t *cbuf = keybuf + 256;                            // [kCandMax] survivors
    if (tid == 0) sh.bcast[3] = 0;
    // this thread's Gamma_e members (kpt divides 32: its blocks share one bitmap word)
    const bool has_e = eid >= 0 && eid < n;
    words[lane] = 0u;
    wave_lds_sync();
    if (has_e) atomicOr(&words[eid >> 5], 1u << (eid & 31));
    wave_lds_sync();
    const uint32_t mine = (words[base >> 5] >> (base & 31)) & ((1u << kpt) - 1u);
    uint64_t key[kRegPickMax];
    uint64_t best = 0ull;
#pragma unroll
    for (int j = 0; j < kRegPickMax; ++j) {
        const int i = base + j;
        const bool c = j < kpt && i < n && !((mine >> j) & 1u);
        key[j] = c ? composite_key(order_key(sv[j]), i) : 0ull;
        best = key[j] > best ? key[j] : best;
    }
    int ct = 1;                            // threads per chunk (within a quad): at most 64 chunks
    while (ct < 4 && n > 64 * kpt * ct) ct *= 2;
    if (ct >= 2) best = dpp_max64(best, 0);
    if (ct >= 4) best = dpp_max64(best, 1);
    const int nch = (n + kpt * ct - 1) / (kpt * ct);
    if ((tid & (ct - 1)) == 0 && tid / ct < nch) tmax[tid / ct] = best;
    wg_barrier();
    // T0: the kq-th best chunk maximum (1, keeping every candidate, when fewer than kq chunks hold one)
    uint64_t T0 = wave_kth_largest(lane < nch ? tmax[lane] : 0ull, kq);
    if (T0 == 0ull) T0 = 1ull;
    uint32_t keep = 0u;
#pragma unroll
    for (int j = 0; j < kRegPickMax; ++j) keep |= (key[j] != 0ull && key[j] >= T0) ? (1u << j) : 0u;
    // survivor slots: ballots per key index, one LDS atomic per wave
    uint64_t bal[kRegPickMax];
    int wtot = 0;
#pragma unroll
    for (int j = 0; j < kRegPickMax; ++j) {
        bal[j] = __ballot((keep >> j) & 1u);
        wtot += __popcll(bal[j]);
    }
    int pos = 0;
    if (wtot) {
        int got = 0;
        if (lane == 0) got = atomicAdd(&sh.bcast[3], wtot);
        pos = __builtin_amdgcn_readfirstlane(__shfl(got, 0, 64));
    }
#pragma unroll
    for (int j = 0; j < kRegPickMax; ++j) {
        if ((keep >> j) & 1u) {
            const int p = pos + lanes_below(bal[j]);
            if (p < kCandMax) cbuf[p] = key[j];
        }
        pos += __popcll(bal[j]);
    }
    wg_barrier();
    const int total = sh.bcast[3];
    if (total > kCandMax) return false;
    int qid = -1;                          // wave 0: this lane's winner id, or -1
    if (total > 64) {
        if (tid < 64) win[lane] = -1;
        wg_barrier();
        rank_mark<NT>(cbuf, total, kq, [&](int, uint64_t c, int rank) { win[rank] = (int)(0xFFFFFFFFu - (uint32_t)c); });
        wg_barrier();
        if (tid < 64 && lane < kq) qid = win[lane];
    } else if (tid < 64) {
        const uint64_t c = lane < total ? cbuf[lane] : 0ull;
        uint64_t kth = total > kq ? wave_kth_largest(c, kq) : 1ull;
        if (c != 0ull && c >= kth) qid = (int)(0xFFFFFFFFu - (uint32_t)c);
    }
    if (tid < 64) {
        uint32_t *lw = (uint32_t *)(keybuf + 64);   // [128] words for the id ranks (wave 0's bitmaps are done)
        const bool hq = qid >= 0;
        const int nq = __popcll(__ballot(hq)), ne = __popcll(__ballot(has_e));
        const int qr = wave_id_ranks(lw, qid, hq, 0, false).x;
        if (hq) qlist[qr] = qid;
        for (int p = nq + lane; p < kq; p += 64) qlist[p] = -1;
        if (sel) {
            const int k = kq + ke;
            const int2 ur = wave_id_ranks(lw, qid, hq, eid, has_e);
            if (hq) sel[ur.x] = qid;
            if (has_e) sel[ur.y] = eid;
            for (int p = nq + ne + lane; p < k; p += 64) sel[p] = -1;
        }
    }
    return true;
}

// LDS layout of the selection phase for a row of n blocks.
struct RowLds {
    uint64_t *keys;     // [kKeyScratch] top-k scratch
    float *sc;          // [n] block scores
    float *ev;          // [n] eviction scores, or nullptr (then read from global)
    uint8_t *inE;       // [n]
    uint8_t *inQ;       // [n]
};

template <int NT>
__host__ __device__ inline bool ev_in_lds(int n) { return n <= kEvLdsMax; }

template <int NT>
__host__ __device__ inline size_t row_lds_bytes(int n) {
    const size_t n16 = (size_t)((n + 15) & ~15);
    return 8 * (size_t)kKeyScratch + 4 * n16 + (ev_in_lds<NT>(n) ? 4 * n16 : 0) + 2 * n16;
}

template <int NT>
__device__ inline RowLds carve(unsigned char *dyn, int n) {
    const int n16 = (n + 15) & ~15;
    RowLds L;
    unsigned char *p = dyn;
    L.keys = (uint64_t *)p;
    p += 8 * kKeyScratch;
    L.sc = (float *)p;
    p += 4 * n16;
    L.ev = nullptr;
    if (ev_in_lds<NT>(n)) {
        L.ev = (float *)p;
        p += 4 * n16;
    }
    L.inE = p;
    L.inQ = p + n16;
    return L;
}

// Loads up to kEvPre * NT eviction scores of the row into registers (issued early; stored to
// LDS by ev_store once they are needed, together with the rest of a row of up to kEvLdsMax
// blocks).  Longer rows read their eviction scores from global memory during the top-k.
template <int NT>
__device__ __forceinline__ void ev_load(const SelectArgs &a, int row, float (&e)[kEvPre]) {
    const float *evr = a.ev + (size_t)row * a.n_blocks_max;
#pragma unroll
    for (int r = 0; r < kEvPre; ++r) {
        const int i = threadIdx.x + r * NT;
        e[r] = i < a.n_blocks ? evr[i] : 0.0f;
    }
}

template <int NT>
__device__ __forceinline__ void ev_store(const SelectArgs &a, int row, const RowLds &L, int n,
                                         const float (&e)[kEvPre]) {
    if (!L.ev) return;
#pragma unroll
    for (int r = 0; r < kEvPre; ++r) {
        const int i = threadIdx.x + r * NT;
        if (i < n) L.ev[i] = e[r];
    }
    // the rest of a long row (beyond the prefetch): independent loads, several in flight
    const float *evr = a.ev + (size_t)row * a.n_blocks_max;
#pragma unroll 4
    for (int i = threadIdx.x + kEvPre * NT; i < n; i += NT) L.ev[i] = evr[i];
}

// Copies a row's n block scores from global memory to L.sc and clears L.inE and L.inQ: up to
// kScorePer scores per thread are loaded together before any is stored (one round trip).
template <int NT>
__device__ __forceinline__ void scores_to_lds(const float *gscore, int n, const RowLds &L) {
    const int tid = threadIdx.x;
    float sv[kScorePer];
#pragma unroll
    for (int r = 0; r < kScorePer; ++r) {
        const int i = tid + r * NT;
        sv[r] = i < n ? gscore[i] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kScorePer; ++r) {
        const int i = tid + r * NT;
        if (i < n) {
            L.sc[i] = sv[r];
            L.inE[i] = 0;
            L.inQ[i] = 0;
        }
    }
    for (int i = tid + kScorePer * NT; i < n; i += NT) {
        L.sc[i] = gscore[i];
        L.inE[i] = 0;
        L.inQ[i] = 0;
    }
}

// Entry idx of the row's agn_state (the previous Gamma_e), or -1 on a fresh step or past ke.  The
// selection kernels load it together with the eviction scores, so the previous members cost no
// round trip of their own later.
__device__ __forceinline__ int prev_agn(const SelectArgs &a, int row, int idx) {
    return (a.n_prev > 0 && idx < a.ke) ? a.agn[(size_t)row * a.ke + idx] : -1;
}

// Gamma_e of one row into L.inE (all threads of the workgroup): the sink and window blocks plus
// the score-ranked members under strict eviction.  id0 = prev_agn(a, row, threadIdx.x); entries
// past the first NT of the previous Gamma_e are read here.  Uses L.inQ as scratch and leaves it
// cleared.
template <int NT>
__device__ void select_agnostic(const SelectArgs &a, int row, const RowLds &L, SelectShared<NT> &sh, int id0) {
    const int tid = threadIdx.x;
    const int n = a.n_blocks;
    for (int i = tid; i < n; i += NT) {
        L.inE[i] = 0;
        L.inQ[i] = 0;
    }
    wg_barrier();
    const int n_prev = a.n_prev;
    const bool fresh = (n_prev == 0);
    const int w_lo = n - a.n_window;              // first window block
    const int left = n_prev - a.n_window;         // blocks below this were ranked (or out) last step
    if (!fresh) {   // previous Gamma_e (inQ reused as scratch)
        if (id0 >= 0 && id0 < n_prev) L.inQ[id0] = 1;
        for (int j = tid + NT; j < a.ke; j += NT) {
            const int id = a.agn[(size_t)row * a.ke + j];
            if (id >= 0 && id < n_prev) L.inQ[id] = 1;
        }
    }
    for (int i = tid; i < n; i += NT)
        if (i < a.n_sink || i >= w_lo) L.inE[i] = 1;
    wg_barrier();
    const float *evg = a.ev + (size_t)row * a.n_blocks_max;
    const float *evl = L.ev;
    const uint8_t *prevE = L.inQ;
    const int n_sink = a.n_sink;
    topk_mark<NT>(
        n, a.ke - a.n_sink - a.n_window, [&](int i) { return order_key(evl ? evl[i] : evg[i]); },
        [&](int i) { return i >= n_sink && i < w_lo && (fresh || i >= left || prevE[i]); }, L.inE, L.keys, sh);
    for (int i = tid; i < n; i += NT) L.inQ[i] = 0;
    wg_barrier();
}

// Gamma_q of one row from the block scores in L.sc and Gamma_e in L.inE, then the outputs in
// ascending block id: the selection, and agn_state when write_agn is set.
template <int NT>
__device__ void select_query(const SelectArgs &a, int row, const RowLds &L, SelectShared<NT> &sh, bool write_agn) {
    const int n = a.n_blocks;
    const uint8_t *inE = L.inE;
    const float *sc = L.sc;
    topk_mark<NT>(
        n, a.kq, [&](int i) { return order_key(sc[i]); }, [&](int i) { return !inE[i]; }, L.inQ, L.keys, sh);
    const int k = a.kq + a.ke;
    compact_outputs<NT>(n, L.inE, L.inQ, (write_agn && a.ke > 0) ? a.agn + (size_t)row * a.ke : nullptr, a.ke,
                        a.sel + (size_t)row * k, k, sh);
}


// Rows of at most 64 blocks: lane i of every wave holds block i.
constexpr int kWaveRowMax = 64;

// Rank of lane i's key among the 64 lanes' keys (the number of larger keys), counted by all
// NT / 64 waves of the workgroup: wave w compares against lanes [w * 64 / NW, (w + 1) * 64 / NW)
// with lane reads and the partial counts are added through part[NW][64] in LDS.  Every thread
// calls it with its wave's copy of the keys.
template <int NT>
__device__ __forceinline__ int group_rank64(uint64_t key, int *part) {
    constexpr int NW = NT / 64, JW = 64 / NW;
    const int i = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < JW; ++u) {
        const int j = w * JW + u;
        const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, j) << 32) |
                            (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, j);
        cnt += kj > key ? 1 : 0;
    }
    if (NW == 1) return cnt;
    part[w * 64 + i] = cnt;
    wg_barrier();
    int r = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) r += part[v * 64 + i];
    wg_barrier();   // part is written again by the next call
    return r;
}

// The whole selection of a row of n <= 64 blocks, with lane i of every wave on block i: Gamma_e
// (sink and window blocks, plus the best blocks by eviction score among the same candidates as
// select_agnostic), then Gamma_q (the best block scores outside Gamma_e), both by exact rank of
// the same unique keys topk_mark uses, so the result is identical.  Wave 0 writes agn_state and
// the selection like select_query and, when wl is given, Gamma_e then Gamma_q (each ascending,
// padded with -1 to ke and kq entries) to wl[0..k).  Reads L.sc and L.ev and uses L.keys as
// scratch; called by all NT threads after the barrier that follows the scoring.
// prev_id = prev_agn(a, row, lane).
template <int NT>
__device__ void select_row64(const SelectArgs &a, int row, const RowLds &L, int32_t *wl, int prev_id) {
    const int i = threadIdx.x & 63;
    const int n = a.n_blocks, ke = a.ke, kq = a.kq, k = kq + ke;
    const bool in_row = i < n;
    int *part = (int *)L.keys;
    // previous Gamma_e as a lane mask (strict eviction): ids < n_prev only
    const int n_prev = a.n_prev;
    const bool fresh = (n_prev == 0);
    uint64_t prev = 0ull;
    if (!fresh && ke > 0) {
        const int id = prev_id;
        const uint64_t has = __ballot(id >= 0 && id < n_prev);
        for (uint64_t m = has; m; m &= m - 1) {
            const int j = __builtin_ctzll(m);
            prev |= 1ull << __builtin_amdgcn_readlane(id, j);
        }
    }
    const int w_lo = n - a.n_window, left = n_prev - a.n_window;
    const bool forced = in_row && (i < a.n_sink || i >= w_lo);
    const bool cand_e = in_row && i >= a.n_sink && i < w_lo && (fresh || i >= left || ((prev >> i) & 1ull));
    const float evi = in_row ? (L.ev ? L.ev[i] : a.ev[(size_t)row * a.n_blocks_max + i]) : 0.0f;
    const int kk_e = ke - a.n_sink - a.n_window;
    const int re = group_rank64<NT>(cand_e ? composite_key(order_key(evi), i) : 0ull, part);
    const bool inE = forced || (cand_e && re < kk_e);
    const bool cand_q = in_row && !inE;
    const int rq = group_rank64<NT>(cand_q ? composite_key(order_key(L.sc[i]), i) : 0ull, part);
    const bool inQ = cand_q && rq < kq;
    if (threadIdx.x >= 64) return;
    // outputs in ascending block id
    const uint64_t mE = __ballot(inE), mQ = __ballot(inQ), mS = mE | mQ;
    const int pe = lanes_below(mE), pq = lanes_below(mQ), ps = lanes_below(mS);
    const int ne = __popcll(mE), nq = __popcll(mQ), ns = __popcll(mS);
    int32_t *agn = a.agn + (size_t)row * ke;
    int32_t *sel = a.sel + (size_t)row * k;
    if (inE && pe < ke) {
        agn[pe] = i;
        if (wl) wl[pe] = i;
    }
    if (inQ && pq < kq && wl) wl[ke + pq] = i;
    if ((inE || inQ) && ps < k) sel[ps] = i;
    for (int p = ne + i; p < ke; p += 64) {
        agn[p] = -1;
        if (wl) wl[p] = -1;
    }
    if (wl)
        for (int p = nq + i; p < kq; p += 64) wl[ke + p] = -1;
    for (int p = ns + i; p < k; p += 64) sel[p] = -1;
}

// qs slice of this lane: float4 chunks c8 + 8 i of sum_h q[b][g*G + h].  For bf16 the heads are
// read four at a time, the loads of a batch all issued before any is summed (heads past G re-read
// the last head and are weighted 0), so G <= 4 costs one memory round trip rather than one per head.
template <typename T, int D>
__device__ __forceinline__ void group_query(const SelectArgs &a, int b, int g, int c8, float4 (&qv)[D / 32]) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) qv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (sizeof(T) == 2) {
        constexpr int kBatch = 4;
        for (int h0 = 0; h0 < a.G; h0 += kBatch) {
            uint2 u[kBatch][D / 32];
#pragma unroll
            for (int hh = 0; hh < kBatch; ++hh) {
                const size_t base = (size_t)(b * a.Hq + g * a.G + min(h0 + hh, a.G - 1)) * D;
#pragma unroll
                for (int i = 0; i < D / 32; ++i)
                    u[hh][i] = *(const uint2 *)((const uint16_t *)a.q + base + (c8 + 8 * i) * 4);
            }
#pragma unroll
            for (int hh = 0; hh < kBatch; ++hh) {
                const float wt = h0 + hh < a.G ? 1.0f : 0.0f;   // no branch between loads and sums
#pragma unroll
                for (int i = 0; i < D / 32; ++i) {
                    qv[i].x = fmaf(wt, bf16_lo(u[hh][i].x), qv[i].x);
                    qv[i].y = fmaf(wt, bf16_hi(u[hh][i].x), qv[i].y);
                    qv[i].z = fmaf(wt, bf16_lo(u[hh][i].y), qv[i].z);
                    qv[i].w = fmaf(wt, bf16_hi(u[hh][i].y), qv[i].w);
                }
            }
        }
        return;
    }
    for (int h = 0; h < a.G; ++h) {
        const size_t base = (size_t)(b * a.Hq + g * a.G + h) * D;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const float4 f = *(const float4 *)((const float *)a.q + base + (size_t)(c8 + 8 * i) * 4);
            qv[i].x += f.x;
            qv[i].y += f.y;
            qv[i].z += f.z;
            qv[i].w += f.w;
        }
    }
}

// Scores blocks [blk_lo, blk_hi) of one row; writes them to LDS (sc) or global (gscore).
template <typename T, int D, int SPB, int NT>
__device__ __forceinline__ void score_range(const SelectArgs &a, int row, int blk_lo, int blk_hi, float *sc,
                                            float *gscore) {
    constexpr int CPLS = D / 32;   // 16-byte chunks per lane of one fp32 sub-block row
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = row / a.Hkv, g = row - b * a.Hkv;
    const int r8 = lane >> 3, c8 = lane & 7;
    const int sb_lo = blk_lo * SPB, sb_hi = blk_hi * SPB;
    const int ngroups = (sb_hi - sb_lo + 7) >> 3;   // groups of 8 sub-blocks
    const float *kprow = a.kp + (size_t)row * a.n_blocks_max * SPB * D;
    float4 qv[CPLS];
    // With 256 threads the group query is read after the first pass's pooled keys are requested, so
    // its round trip overlaps theirs; 1024-thread workgroups (128 VGPRs) cannot hold both in flight.
    bool have_q = NT > 256;
    if (have_q) group_query<T, D>(a, b, g, c8, qv);
    for (int g0 = w; g0 < ngroups; g0 += NW * kUnroll) {
        float4 x[kUnroll][CPLS];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = sb_lo + (g0 + NW * u) * 8 + r8;
            const bool v = (g0 + NW * u < ngroups) && (j < sb_hi);
#pragma unroll
            for (int i = 0; i < CPLS; ++i)
                x[u][i] = v ? *(const float4 *)(kprow + (size_t)j * D + (c8 + 8 * i) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (!have_q) {
            group_query<T, D>(a, b, g, c8, qv);
            have_q = true;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = sb_lo + (g0 + NW * u) * 8 + r8;
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < CPLS; ++i) {
                s = fmaf(x[u][i].x, qv[i].x, s);
                s = fmaf(x[u][i].y, qv[i].y, s);
                s = fmaf(x[u][i].z, qv[i].z, s);
                s = fmaf(x[u][i].w, qv[i].w, s);
            }
            s += dpp<kDppQuadXor1>(s);
            s += dpp<kDppQuadXor2>(s);
            s += dpp<kDppRowHalfMirror>(s);     // every lane of the 8-lane group holds u[j]
            if (SPB >= 2) s = fmaxf(s, dpp<kDppRowMirror>(s));
            if (SPB >= 4) s = fmaxf(s, xor_lane(s, 16));
            if (SPB >= 8) s = fmaxf(s, xor_lane(s, 32));
            const bool v = (g0 + NW * u < ngroups) && (j < sb_hi);
            if (v && (lane % (8 * SPB)) == 0) {
                const int blk = j / SPB;
                if (sc) sc[blk] = s;
                else gscore[blk] = s;
            }
        }
    }
}

}  // namespace

}  // namespace nosa
