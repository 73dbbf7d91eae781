"""Pins of the CPU oracle to facts outside itself (closed forms, hand-worked cases,
library routines, invariants the pages fix).  No GPU needed.

The method is the one of "NOSA: Native and Offloadable Sparse Attention"
(paperlayer.ai summary [P1], gist.science technical summary [P4]).
"""

import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from nosa_inputs import f32_to_bf16_bits, bf16_bits_to_f32, generate, small_workload

# Unit roundoff of the oracle build under test (2^-24 for the default float32 build, 2^-53 for the
# float64 one).  Closed forms below are exact in either build; comparisons with library routines
# that compute in float64 allow the rounding of sequential sums of the lengths involved.
EPS = O.rounding_eps()


def _tol(n_terms: float, scale: float = 1.0) -> float:
    """Bound on the error of a sequential sum of n_terms terms of magnitude ~scale (plus slack)."""
    return 4.0 * n_terms * EPS * scale


# --------------------------------------------------------------------------------------
# Sub-block mean pooling  ([P1] §3.1, [P4] Method 1: mean pooling inside sub-blocks)
# --------------------------------------------------------------------------------------

def test_pool_ramp_closed_form():
    # K[r, t, c] = t + 1000 c + 1e4 r  ->  mean over tokens [j*sbs, j*sbs+sbs) is
    # sbs*j + (sbs-1)/2 + 1000 c + 1e4 r, exactly (every partial sum is an integer below 2^24, so
    # float32 sums are exact too).  Catches a wrong token window, a wrong divisor and a wrong
    # row offset.
    B, H, nb, bs, d = 2, 3, 5, 64, 4
    t = np.arange(nb * bs, dtype=np.float64).reshape(nb, bs)
    K = np.empty((B, H, nb, bs, d))
    for b in range(B):
        for h in range(H):
            for c in range(d):
                K[b, h, :, :, c] = t + 1000.0 * c + 1e4 * (b * H + h)
    for sbs in (8, 16, 32, 64):
        kp = O.pool_keys(K, sbs)
        j = np.arange(nb * bs // sbs, dtype=np.float64)
        for b in range(B):
            for h in range(H):
                for c in range(d):
                    want = sbs * j + (sbs - 1) / 2.0 + 1000.0 * c + 1e4 * (b * H + h)
                    assert np.array_equal(kp[b, h, :, c], want)


def test_pool_constant_subblocks_and_unit_subblock():
    rng = np.random.default_rng(0)
    B, H, nb, bs, d, sbs = 1, 2, 4, 64, 16, 32
    const = rng.standard_normal((B, H, nb * bs // sbs, 1, d)).astype(np.float32)
    K = np.broadcast_to(const, (B, H, nb * bs // sbs, sbs, d)).reshape(B, H, nb, bs, d)
    bits = f32_to_bf16_bits(np.ascontiguousarray(K))
    kp = O.pool_keys(bits, sbs)
    assert np.array_equal(kp, bf16_bits_to_f32(f32_to_bf16_bits(const[:, :, :, 0, :])).astype(np.float64))
    # sub-block of one token: pooling is the identity
    K1 = rng.standard_normal((B, H, nb, bs, d)).astype(np.float32)
    kp1 = O.pool_keys(K1, 1)
    assert np.array_equal(kp1, K1.reshape(B, H, nb * bs, d).astype(np.float64))


# --------------------------------------------------------------------------------------
# Block scores  ([P1] §2.1 query-key similarity; [P1] §3.1 mean then max pooling)
# --------------------------------------------------------------------------------------

def test_scores_parallel_keys_closed_form():
    # Every pooled key of group g is alpha_j * e_g (a multiple of a basis vector), and the
    # group's heads carry 1, 2, ... on coordinate g, so the group's head-summed dot is
    # alpha_j * G(G+1)/2 whatever the other coordinates hold.  A wrong head-to-group
    # mapping, a missing head sum or a wrong max window changes the result.
    rng = np.random.default_rng(1)
    B, Hkv, G, d, nb, spb = 2, 3, 4, 8, 6, 2
    Hq = Hkv * G
    q = rng.integers(-5, 6, size=(B, Hq, d)).astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            q[b, h, h // G] = (h % G) + 1
    alpha = rng.integers(-50, 51, size=(B, Hkv, nb * spb)).astype(np.float64)
    kp = np.zeros((B, Hkv, nb * spb, d))
    for g in range(Hkv):
        kp[:, g, :, g] = alpha[:, g, :]
    s = O.block_scores(q, kp, nb, spb)
    beta = G * (G + 1) / 2
    want = (alpha.reshape(B, Hkv, nb, spb) * beta).max(axis=-1)
    assert np.array_equal(s, want)


def test_scores_match_torch_pooling_route():
    # Independent route through library primitives: torch avg_pool1d for the sub-block
    # means, a batched matmul for all head-key dots, a sum over the group and max_pool1d.
    w = small_workload(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, n_blocks=9, kq=2, ke=2, seed=5)
    x = generate(w)
    qf = torch.from_numpy(bf16_bits_to_f32(x["q"]).astype(np.float64))
    kf = torch.from_numpy(bf16_bits_to_f32(x["k"]).astype(np.float64))
    B, Hkv, nb, bs, d = kf.shape
    G = w.n_q_heads // Hkv
    for sbs in (16, 32, 64):
        kp_o = O.pool_keys(x["k"], sbs)
        s_o = O.block_scores(x["q"], kp_o, nb, bs // sbs)
        tok = kf.reshape(B * Hkv, nb * bs, d).transpose(1, 2)                      # [R, d, T]
        pooled = torch.nn.functional.avg_pool1d(tok, sbs, sbs).transpose(1, 2)     # [R, nsub, d]
        qg = qf.reshape(B * Hkv, G, d)                                             # heads of each group
        dots = torch.matmul(qg, pooled.transpose(1, 2).contiguous())               # [R, G, nsub]
        u = dots.sum(dim=1, keepdim=True)                                          # [R, 1, nsub]
        s_t = torch.nn.functional.max_pool1d(u, bs // sbs, bs // sbs).reshape(B, Hkv, nb)
        np.testing.assert_allclose(kp_o.reshape(B * Hkv, -1, d), pooled.numpy(), rtol=0, atol=_tol(sbs, 4.0))
        np.testing.assert_allclose(s_o, s_t.numpy(), rtol=0, atol=_tol(G * d, 4.0) + 1e-9)


def test_scores_planted_block_wins():
    # A block whose keys carry a large offset along the summed group query must score highest.
    w = small_workload(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, n_blocks=20, seed=7,
                       block_offset_sigma=0.0, dtype="f32")
    x = generate(w)
    q = x["q"].astype(np.float64)
    qsum = q[0].sum(axis=0)
    k = x["k"].astype(np.float64)
    k[0, 0, 13] += 3.0 * qsum / np.linalg.norm(qsum)
    kp = O.pool_keys(k, 32)
    s = O.block_scores(q, kp, 20, 2)
    assert int(np.argmax(s[0, 0])) == 13
    sel, st, isa = O.select(s, np.zeros((1, 1, 20), np.float32), kq=1, ke=0)
    assert sel.tolist() == [[[13]]]


# --------------------------------------------------------------------------------------
# Selection  ([P1] §2.1, §3.1, App. A, App. E; [P4] Method 1: dual selection, strict
# eviction, locality guarantee)
# --------------------------------------------------------------------------------------

def _lexsort_topk(score, cand, kk):
    ids = np.nonzero(cand)[0]
    order = np.lexsort((ids, -score[ids]))     # score descending, then id ascending
    return set(ids[order[:kk]].tolist())


def test_select_matches_lexsort_topk():
    rng = np.random.default_rng(2)
    B, H, n = 3, 4, 73
    for kq, ke in ((5, 7), (0, 9), (11, 0), (36, 37)):
        s = rng.standard_normal((B, H, n)).astype(np.float32)   # the values every build compares
        s[0, 0, 10:20] = 0.5      # a run of exact ties
        e = rng.random((B, H, n), dtype=np.float32)
        e[1, 1, 30:40] = np.float32(0.25)
        sel, st, isa = O.select(s, e, kq, ke)
        for b in range(B):
            for h in range(H):
                ge = _lexsort_topk(e[b, h].astype(np.float64), np.ones(n, bool), ke)
                comp = np.ones(n, bool)
                comp[list(ge)] = False
                gq = _lexsort_topk(s[b, h], comp, kq)
                assert st[b, h].tolist() == sorted(ge)
                assert sel[b, h].tolist() == sorted(ge | gq)
                assert [i for i, a in zip(sel[b, h], isa[b, h]) if a] == sorted(ge)


def test_select_permutation_eviction_closed_form():
    # e = a permutation of 0..n-1: the top-ke by e are exactly the blocks with e >= n - ke.
    rng = np.random.default_rng(3)
    n, ke = 50, 12
    e = rng.permutation(n).astype(np.float32).reshape(1, 1, n)
    s = rng.standard_normal((1, 1, n))
    sel, st, _ = O.select(s, e, kq=0, ke=ke)
    assert st[0, 0].tolist() == sorted(np.nonzero(e[0, 0] >= n - ke)[0].tolist())
    assert sel[0, 0].tolist() == st[0, 0].tolist()   # kq = 0: selection ignores the query


def test_select_ties_take_lowest_ids_and_full_budget():
    n, kq, ke = 16, 3, 2
    s = np.zeros((1, 1, n))
    e = np.zeros((1, 1, n), np.float32)
    sel, st, _ = O.select(s, e, kq, ke)
    assert st[0, 0].tolist() == [0, 1]
    assert sel[0, 0].tolist() == [0, 1, 2, 3, 4]
    sel, st, _ = O.select(np.ones((1, 1, n)), np.ones((1, 1, n), np.float32), 10, 6)
    assert sel[0, 0].tolist() == list(range(16))     # k = n: every block


def test_select_invariants_random():
    rng = np.random.default_rng(4)
    B, H, n, kq, ke = 2, 3, 200, 32, 32
    s = rng.standard_normal((B, H, n)).astype(np.float32)
    e = rng.random((B, H, n), dtype=np.float32)
    sel, st, isa = O.select(s, e, kq, ke)
    for b in range(B):
        for h in range(H):
            S = set(sel[b, h].tolist())
            E = set(st[b, h].tolist())
            Q = S - E
            assert len(S) == kq + ke and len(E) == ke and E <= S and len(Q) == kq
            rest = [i for i in range(n) if i not in S]
            assert min(s[b, h, list(Q)]) >= max(s[b, h, rest])
            assert min(e[b, h, list(E)]) >= max(e[b, h, [i for i in range(n) if i not in E]])
            assert np.all(np.diff(sel[b, h]) > 0)


def test_multistep_hand_worked_example():
    # ke = 2, kq = 1.  e is fixed per block; blocks 6 and 7 arrive at steps 1 and 2.
    e = np.array([[[0.9, 0.1, 0.5, 0.7, 0.2, 0.3, 0.8, 0.05]]], np.float32)
    # step 0: 6 visible blocks. Gamma_e = top-2 by e = {0 (0.9), 3 (0.7)}.
    s0 = np.array([[[5.0, 4.0, 9.0, 1.0, 2.0, 3.0]]])
    sel, st, _ = O.select(s0, e, kq=1, ke=2, n_prev=0)
    assert st.tolist() == [[[0, 3]]]
    assert sel.tolist() == [[[0, 2, 3]]]          # Gamma_q = best of {1,2,4,5} by s = {2}
    # step 1: block 6 arrives with e = 0.8 -> candidates {0, 3, 6} -> Gamma_e = {0, 6};
    # block 3 leaves Gamma_e for good, but the query-aware part may still recall it.
    s1 = np.array([[[1.0, 1.0, 1.0, 100.0, 1.0, 1.0, 1.0]]])
    sel, st, _ = O.select(s1, e, kq=1, ke=2, n_prev=6, agn_state=st)
    assert st.tolist() == [[[0, 6]]]
    assert sel.tolist() == [[[0, 3, 6]]]
    # step 2: block 7 arrives with e = 0.05 -> candidates {0, 6, 7} -> Gamma_e unchanged;
    # block 3 (e = 0.7 > 0.05) is not re-admitted: strict eviction.
    s2 = np.array([[[0.0, 7.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]]])
    sel, st, _ = O.select(s2, e, kq=1, ke=2, n_prev=7, agn_state=st)
    assert st.tolist() == [[[0, 6]]]
    assert sel.tolist() == [[[0, 1, 6]]]


def test_multistep_strict_eviction_and_locality_guarantee():
    # Random scores every step, arrivals now and then: Gamma_e(t) is a subset of
    # Gamma_e(t-1) plus the arrivals, a block that left never returns, and adjacent
    # selections overlap in at least ke - a(t) blocks (a(t) = admitted arrivals), i.e. in
    # at least ke blocks on steps without arrivals ([P1] App. E, [P4] locality guarantee).
    rng = np.random.default_rng(6)
    B, H, kq, ke, n0, nmax, steps = 2, 2, 6, 10, 40, 60, 40
    e = rng.random((B, H, nmax), dtype=np.float32)
    n = n0
    st = None
    prev_sel = prev_st = None
    dead = [[set() for _ in range(H)] for _ in range(B)]
    for t in range(steps):
        n_prev = 0 if t == 0 else n
        if t > 0 and rng.random() < 0.5 and n < nmax:
            n += 1
        s = rng.standard_normal((B, H, n))
        sel, st, _ = O.select(s, e, kq, ke, n_prev=n_prev, agn_state=st)
        if t > 0:
            gam = O.locality(prev_sel, sel, nmax)
            for b in range(B):
                for h in range(H):
                    E0, E1 = set(prev_st[b, h].tolist()), set(st[b, h].tolist())
                    arrivals = set(range(n_prev, n))
                    assert E1 <= E0 | arrivals
                    assert not (E1 & dead[b][h])
                    dead[b][h] |= E0 - E1
                    admitted = len(E1 & arrivals)
                    overlap = len(set(prev_sel[b, h].tolist()) & set(sel[b, h].tolist()))
                    assert overlap >= ke - admitted
                    assert gam[b, h] >= (ke - admitted) / (kq + ke)
                    if admitted == 0:
                        assert gam[b, h] >= ke / (kq + ke)
        prev_sel, prev_st = sel, st.copy()


# --------------------------------------------------------------------------------------
# Cache step  ([P1] §4 set difference / replacement mapping; [P1] App. A)
# --------------------------------------------------------------------------------------

def test_cache_hand_worked_sequence():
    k, C, nb = 2, 3, 5
    sob = np.full((1, nb), -1, np.int32)
    bos = np.full((1, C), -1, np.int32)
    # step 0: {1, 3}: both miss; free slots 0, 1, 2 -> 1->0, 3->1
    tab, mc, ml = O.cache_step(np.array([[1, 3]], np.int32), sob, bos)
    assert tab.tolist() == [[0, 1]] and mc.tolist() == [2]
    assert ml[0, :2].tolist() == [[1, 0], [3, 1]]
    assert bos.tolist() == [[1, 3, -1]] and sob.tolist() == [[-1, 0, -1, 1, -1]]
    # step 1: {0, 3}: 3 hits slot 1; free = slot 0 (holds 1, unused now), slot 2 -> 0->0
    tab, mc, ml = O.cache_step(np.array([[0, 3]], np.int32), sob, bos)
    assert tab.tolist() == [[0, 1]] and mc.tolist() == [1] and ml[0, 0].tolist() == [0, 0]
    assert bos.tolist() == [[0, 3, -1]] and sob.tolist() == [[0, -1, -1, 1, -1]]
    # step 2: {2, 4}: both miss; free slots 0, 1, 2 -> 2->0, 4->1
    tab, mc, ml = O.cache_step(np.array([[2, 4]], np.int32), sob, bos)
    assert tab.tolist() == [[0, 1]] and mc.tolist() == [2]
    assert bos.tolist() == [[2, 4, -1]] and sob.tolist() == [[-1, -1, 0, -1, 1]]
    # step 3: {2, 3}: 2 hits slot 0; free = slot 1 (holds 4), slot 2 -> 3->1
    tab, mc, ml = O.cache_step(np.array([[2, 3]], np.int32), sob, bos)
    assert tab.tolist() == [[0, 1]] and mc.tolist() == [1] and ml[0, 0].tolist() == [3, 1]
    assert bos.tolist() == [[2, 3, -1]] and sob.tolist() == [[-1, -1, 0, 1, -1]]


@pytest.mark.parametrize("extra_slots", [0, 5])
def test_cache_invariants_random(extra_slots):
    rng = np.random.default_rng(8)
    R, nb, k = 6, 40, 12
    C = k + extra_slots
    sob = np.full((R, nb), -1, np.int32)
    bos = np.full((R, C), -1, np.int32)
    host = rng.integers(0, 255, size=(1, R, nb, 4, 8), dtype=np.uint8)
    cache = np.zeros((1, R, C, 4, 8), np.uint8)
    prev = None
    for t in range(30):
        sel = np.sort(np.stack([rng.choice(nb, k, replace=False) for _ in range(R)]), axis=1).astype(np.int32)
        resident_before = [set(int(b) for b in bos[r] if b >= 0) for r in range(R)]
        tab, mc, ml = O.cache_step(sel, sob, bos)
        O.gather(mc.reshape(1, R), ml.reshape(1, R, k, 2), host, cache)
        for r in range(R):
            S = set(sel[r].tolist())
            assert mc[r] == len(S - resident_before[r])
            for s_, b in enumerate(bos[r]):
                if b >= 0:
                    assert sob[r, b] == s_
                    assert np.array_equal(cache[0, r, s_], host[0, r, b])     # slot holds its block's bytes
            for b in range(nb):
                if sob[r, b] >= 0:
                    assert bos[r, sob[r, b]] == b
            assert all(bos[r, tab[r, i]] == sel[r, i] for i in range(k))
            # only blocks unused at this step were swapped out
            assert S <= set(int(b) for b in bos[r] if b >= 0)
            if extra_slots == 0 and prev is not None:
                # with as many slots as the budget, the cache after step t-1 holds exactly
                # Gamma(t-1), so hits(t) = k * gamma(t)
                gam = len(S & set(prev[r].tolist())) / k
                assert k - mc[r] == round(k * gam)
        prev = sel


# --------------------------------------------------------------------------------------
# Attention over the selected blocks  ([P1] App. A; standard scaled dot-product attention)
# --------------------------------------------------------------------------------------

def test_attention_two_token_closed_form():
    # d = 1, one block of two tokens, scale 1: logits 0 and ln 3 -> weights 1/4, 3/4.
    q = np.array([[[1.0]]])
    K = np.array([[[[[0.0], [math.log(3.0)]]]]])
    V = np.array([[[[[1.0], [5.0]]]]])
    out = O.attention(q, K, V, np.array([[[0]]], np.int32), scale=1.0)
    assert abs(out[0, 0, 0] - (0.25 * 1.0 + 0.75 * 5.0)) < _tol(2, 5.0)


def test_attention_dense_case_matches_torch_sdpa():
    # Selecting every block reduces sparse attention to dense decode attention.
    w = small_workload(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, n_blocks=6, seed=9)
    x = generate(w)
    B, Hkv, nb, bs, d = x["k"].shape
    table = np.tile(np.arange(nb, dtype=np.int32), (B, Hkv, 1))
    out = O.attention(x["q"], x["k"], x["v"], table)
    qf = torch.from_numpy(bf16_bits_to_f32(x["q"]).astype(np.float64)).unsqueeze(2)      # [B,Hq,1,d]
    G = w.n_q_heads // Hkv
    kf = torch.from_numpy(bf16_bits_to_f32(x["k"]).astype(np.float64)).reshape(B, Hkv, nb * bs, d)
    vf = torch.from_numpy(bf16_bits_to_f32(x["v"]).astype(np.float64)).reshape(B, Hkv, nb * bs, d)
    kf = kf.repeat_interleave(G, dim=1)
    vf = vf.repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf).squeeze(2).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=_tol(nb * bs, 4.0) + 1e-12)


def test_attention_gather_and_masked_forms_agree_and_invariances():
    w = small_workload(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=23, kq=4, ke=5, seed=10)
    x = generate(w)
    rng = np.random.default_rng(10)
    B, Hkv, nb = 2, 2, 23
    sel = np.sort(np.stack([rng.choice(nb, 9, replace=False) for _ in range(B * Hkv)]), 1)
    sel = sel.reshape(B, Hkv, 9).astype(np.int32)
    mask = np.zeros((B, Hkv, nb), np.uint8)
    for b in range(B):
        for g in range(Hkv):
            mask[b, g, sel[b, g]] = 1
    o1 = O.attention(x["q"], x["k"], x["v"], sel)
    o2 = O.attention_masked(x["q"], x["k"], x["v"], mask)
    T = 9 * 64
    np.testing.assert_allclose(o1, o2, rtol=0, atol=_tol(T, 4.0) + 1e-13)
    perm = sel[:, :, rng.permutation(9)]
    o3 = O.attention(x["q"], x["k"], x["v"], np.ascontiguousarray(perm))
    np.testing.assert_allclose(o1, o3, rtol=0, atol=_tol(T, 4.0) + 1e-13)
    # constant V gives that constant back
    vc = np.full_like(x["v"], f32_to_bf16_bits(np.array([1.5], np.float32))[0])
    o4 = O.attention(x["q"], x["k"], vc, sel)
    np.testing.assert_allclose(o4, 1.5, rtol=0, atol=_tol(T, 1.5) + 1e-13)


def test_attention_dominant_token_returns_its_value():
    w = small_workload(batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, n_blocks=4, seed=12, dtype="f32",
                       block_offset_sigma=0.0)
    x = generate(w)
    k = x["k"].astype(np.float64)
    q = x["q"].astype(np.float64)
    # token (block 2, position 17) aligned with both heads, far above every other logit
    k[0, 0, 2, 17] = 40.0 * (q[0, 0] + q[0, 1])
    out = O.attention(q, k, x["v"].astype(np.float64), np.array([[[0, 1, 2, 3]]], np.int32))
    np.testing.assert_allclose(out[0], np.stack([x["v"][0, 0, 2, 17]] * 2).astype(np.float64), atol=_tol(256, 4.0))


def test_locality_hand_example():
    g = O.locality(np.array([[0, 2, 5, 7]], np.int32), np.array([[2, 3, 5, 9]], np.int32), 10)
    assert g.tolist() == [0.5]


def test_c1_regression_record():
    # The oracle still reproduces its recorded C1 result (tests/golden/make_golden.py).
    import json
    import os
    from nosa_inputs import WORKLOADS
    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "c1_oracle.json")))
    w = WORKLOADS["C1"]
    x = generate(w)
    r = O.decode_step(x["q"], O.pool_keys(x["k"], 32), x["evict"], x["k"], x["v"], w.n_blocks, w.kq, w.ke, 2)
    assert r["selected"].reshape(-1).tolist() == rec["selected"]
    assert r["agn_state"].reshape(-1).tolist() == rec["agn_state"]
    # the record holds the float64 build's values; the float32 build stays within its rounding
    np.testing.assert_allclose(r["scores"].reshape(-1), rec["block_scores"], rtol=0, atol=_tol(2 * 64, 8.0) + 1e-12)
    np.testing.assert_allclose(r["out"].reshape(-1), rec["out"], rtol=0, atol=_tol(8 * 64, 4.0) + 1e-12)


# --------------------------------------------------------------------------------------
# Sink and sliding-window blocks inside the query-agnostic budget ([P1] B.2.2: the paper's
# query-agnostic blocks include one attention-sink block and a window of recent blocks)
# --------------------------------------------------------------------------------------

def test_sink_window_hand_worked_example():
    # ke = 4 = 1 sink + 2 window + 1 score-ranked block; kq = 1.
    e = np.array([[[0.9, 0.1, 0.5, 0.7, 0.2, 0.3, 0.8, 0.05, 0.6, 0.95]]], np.float32)
    kw = dict(kq=1, ke=4, n_sink=1, n_window=2)
    # step 0, 8 blocks: fixed {0} + window {6, 7}; ranked candidates {1..5} -> 3 (e 0.7)
    sel, st, _ = O.select(np.arange(1.0, 9.0).reshape(1, 1, 8), e, **kw)
    assert st.tolist() == [[[0, 3, 6, 7]]]
    assert sel.tolist() == [[[0, 3, 5, 6, 7]]]        # query-aware: best of {1,2,4,5} = 5
    # step 1, block 8 arrives: window {7, 8}; block 6 left the window and competes with the
    # ranked member 3: e 0.8 > 0.7 -> 6 stays, 3 leaves Gamma_e for good (but may be recalled)
    s1 = np.zeros((1, 1, 9))
    s1[0, 0, 3] = 100.0
    sel, st, _ = O.select(s1, e, n_prev=8, agn_state=st, **kw)
    assert st.tolist() == [[[0, 6, 7, 8]]]
    assert sel.tolist() == [[[0, 3, 6, 7, 8]]]
    # step 2, block 9 arrives: block 7 (e 0.05) leaves the window and loses to 6
    sel, st, _ = O.select(np.zeros((1, 1, 10)), e, n_prev=9, agn_state=st, **kw)
    assert st.tolist() == [[[0, 6, 8, 9]]]
    # no score-ranked slot: Gamma_e is exactly sink + window
    sel, st, _ = O.select(np.zeros((1, 1, 10)), e, kq=2, ke=3, n_sink=1, n_window=2)
    assert st.tolist() == [[[0, 8, 9]]]


def test_sink_window_multistep_invariants():
    rng = np.random.default_rng(13)
    B, H, kq, ke, ns, nw, n0, nmax, steps = 2, 2, 5, 12, 1, 4, 30, 60, 40
    e = rng.random((B, H, nmax), dtype=np.float32)
    n, st, prev_sel, prev_st = n0, None, None, None
    left_for_good = [[set() for _ in range(H)] for _ in range(B)]
    for t in range(steps):
        n_prev = 0 if t == 0 else n
        if t > 0 and rng.random() < 0.6 and n < nmax:
            n += int(rng.integers(1, 3))
            n = min(n, nmax)
        s = rng.standard_normal((B, H, n))
        sel, st, _ = O.select(s, e, kq, ke, n_prev=n_prev, agn_state=st, n_sink=ns, n_window=nw)
        for b in range(B):
            for h in range(H):
                E = set(st[b, h].tolist())
                assert set(range(ns)) <= E and set(range(n - nw, n)) <= E
                assert len(E) == ke and len(set(sel[b, h].tolist())) == kq + ke
                assert not (E & left_for_good[b][h])
                if prev_st is not None:
                    E0 = set(prev_st[b, h].tolist())
                    left_for_good[b][h] |= E0 - E
                    arrivals = n - n_prev
                    assert len(E0 & E) >= ke - arrivals
                    overlap = len(set(prev_sel[b, h].tolist()) & set(sel[b, h].tolist()))
                    assert overlap >= ke - arrivals
        prev_sel, prev_st = sel, st.copy()


# --------------------------------------------------------------------------------------
# Decode append  ([P1] §3.1 pooled keys beside the cache; [P4] Method 1 block arrivals)
# --------------------------------------------------------------------------------------

def test_append_ramp_closed_form_and_skips():
    # Token p of row (b, h) carries p + 1000 c + 1e4 (b H + h).  Appended one at a time with ragged
    # lengths per sequence (a negative or past-the-end position leaves the sequence alone), every
    # written slot (p // 64, p % 64) holds its token, every other slot keeps the sentinel, and the
    # pooled keys of the finished sub-blocks are the ramp's mean in closed form.
    B, H, nbmax, bs, d, sbs = 3, 2, 3, 64, 4, 16
    lens = [0, 37, nbmax * bs]
    ks = np.full((B, H, nbmax, bs, d), -5.0)
    vs = np.full_like(ks, -5.0)
    for p in range(nbmax * bs + 2):
        pos = np.array([p if p < L else -1 for L in lens], dtype=np.int32)
        if p == nbmax * bs + 1:
            pos[2] = nbmax * bs          # past the end: skipped
        kn = np.empty((B, H, d))
        for b in range(B):
            for h in range(H):
                kn[b, h] = p + 1000.0 * np.arange(d) + 1e4 * (b * H + h)
        O.append_kv(ks, vs, kn, -kn, pos)
    for b, L in enumerate(lens):
        for h in range(H):
            flat = ks[b, h].reshape(nbmax * bs, d)
            for p in range(nbmax * bs):
                want = p + 1000.0 * np.arange(d) + 1e4 * (b * H + h) if p < L else np.full(d, -5.0)
                assert np.array_equal(flat[p], want)
                assert np.array_equal(vs[b, h].reshape(nbmax * bs, d)[p], -want if p < L else want)
    kp = O.pool_keys(ks, sbs)
    for b, L in enumerate(lens):
        for h in range(H):
            for j in range(L // sbs):
                want = sbs * j + (sbs - 1) / 2 + 1000.0 * np.arange(d) + 1e4 * (b * H + h)
                assert np.array_equal(kp[b, h, j], want)   # integer partial sums below 2^24: exact


# --------------------------------------------------------------------------------------
# Transfer granularity  ([P1] §3.2 block-wise vs element-wise; §4 fine-grained block transfer)
# --------------------------------------------------------------------------------------

def test_gather_units_hand_example():
    # 16-byte units of a byte ramp: unit i holds bytes 16 i .. 16 i + 15.
    src = np.arange(8 * 16, dtype=np.uint8)
    dst = np.full(5 * 16, 255, dtype=np.uint8)
    O.gather_units(src, dst, 16, np.array([3, 0, 7, 9, 2]), np.array([1, 4, 0, 2, 7]))
    want = np.full(5 * 16, 255, dtype=np.uint8)
    want[16:32] = np.arange(48, 64)       # unit 3 -> 1
    want[64:80] = np.arange(0, 16)        # unit 0 -> 4
    want[0:16] = np.arange(112, 128)      # unit 7 -> 0
    # (9 -> 2) source out of range, (2 -> 7) destination out of range: both skipped
    assert np.array_equal(dst, want)


def test_gather_units_block_granularity_equals_block_gather():
    # With one KV block as the unit, the unit transfer reproduces the block gather of the cache
    # update for the same miss list (two independent implementations of one copy).
    rng = np.random.default_rng(3)
    B, H, nb, C, bs, d = 2, 2, 6, 4, 64, 8
    host = rng.integers(0, 65535, size=(B, H, nb, bs, d), dtype=np.uint16)
    cache_a = np.zeros((B, H, C, bs, d), np.uint16)
    cache_b = np.zeros_like(cache_a)
    mcnt = np.array([[2, 0], [3, 1]], np.int32)
    ml = np.full((B, H, 4, 2), -1, np.int32)
    ml[0, 0, :2] = [[5, 1], [0, 3]]
    ml[1, 0, :3] = [[1, 0], [2, 2], [4, 1]]
    ml[1, 1, :1] = [[3, 3]]
    O.gather(mcnt, ml, host, cache_a)
    ub = bs * d * 2
    su, du = [], []
    for b in range(B):
        for h in range(H):
            r = b * H + h
            for i in range(mcnt[b, h]):
                su.append(r * nb + ml[b, h, i, 0])
                du.append(r * C + ml[b, h, i, 1])
    O.gather_units(host, cache_b, ub, np.array(su), np.array(du))
    assert np.array_equal(cache_a, cache_b)


def test_strict_eviction_holds_when_eviction_scores_change():
    # With scores fixed over time, top-ke of (previous members + arrivals) equals top-ke of all
    # visible blocks, so only a change of the scores between steps shows the rule itself: a block
    # outside Gamma_e stays out even when its eviction score rises; arrivals still compete.
    kw = dict(kq=1, ke=2)
    e0 = np.array([[[0.9, 0.8, 0.1, 0.2, 0.3, 0.05, 0.0]]], np.float32)
    sel, st, _ = O.select(np.zeros((1, 1, 6)), e0, **kw)
    assert st.tolist() == [[[0, 1]]]
    e1 = np.array([[[0.9, 0.1, 0.95, 0.2, 0.3, 0.05, 0.5]]], np.float32)
    s1 = np.zeros((1, 1, 6))
    s1[0, 0, 2] = 7.0
    sel, st, _ = O.select(s1, e1, n_prev=6, agn_state=st, **kw)
    assert st.tolist() == [[[0, 1]]]            # block 2 (now 0.95) may not re-enter
    assert sel.tolist() == [[[0, 1, 2]]]        # but the query-aware part recalls it
    sel, st, _ = O.select(np.zeros((1, 1, 7)), e1, n_prev=6, agn_state=st, **kw)
    assert st.tolist() == [[[0, 6]]]            # the arrival (0.5) beats member 1 (now 0.1)
