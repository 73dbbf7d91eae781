"""Parity of the HIP path (through the C ABI) with the CPU oracle, on reduced shapes that span
several workgroups, splits and parts with ragged tails, plus the edge cases of the method."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import f32_to_bf16_bits, generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

# name -> (workload kwargs, sub_block_size)
CASES = {
    "g4_d128_bf16_ragged": (dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=37, n_blocks_max=41,
                                 kq=5, ke=7, seed=21), 32),
    "g2_d64_bf16_sbs16": (dict(batch=3, n_q_heads=6, n_kv_heads=3, head_dim=64, n_blocks=50, kq=9, ke=4, seed=22), 16),
    "g8_d128_bf16_sbs64": (dict(batch=1, n_q_heads=8, n_kv_heads=1, head_dim=128, n_blocks=33, kq=3, ke=13,
                                seed=23), 64),
    "g1_d64_f32_ke_only": (dict(batch=2, n_q_heads=2, n_kv_heads=2, head_dim=64, n_blocks=20, kq=0, ke=6,
                                dtype="f32", seed=24), 8),
    "g4_d128_bf16_kq_only": (dict(batch=2, n_q_heads=4, n_kv_heads=1, head_dim=128, n_blocks=70, kq=20, ke=0,
                                  seed=25), 32),
    "g2_d64_f32_all_blocks": (dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64, n_blocks=12, kq=5, ke=7,
                                   dtype="f32", seed=26), 32),
    "g4_d64_f32": (dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, n_blocks=45, kq=6, ke=6, dtype="f32",
                        seed=27), 32),
    "g2_d128_f32": (dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, n_blocks=19, kq=4, ke=4, dtype="f32",
                         seed=28), 32),
}


def _setup(name):
    kw, sbs = CASES[name]
    w = small_workload(name, **kw)
    x = generate(w)
    return w, x, sbs


@pytest.mark.parametrize("name", sorted(CASES))
def test_pool_keys(name):
    w, x, sbs = _setup(name)
    shape = H.shape_of(w, sub_block_size=sbs)
    kp = H.host(H.gpu_pool(shape, H.dev(x["k"])))
    ref = O.pool_keys(x["k"], sbs).reshape(kp.shape)
    np.testing.assert_allclose(kp, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("parts", [0, 1, 3, 7])
@pytest.mark.parametrize("name", sorted(CASES))
def test_block_scores(name, parts):
    w, x, sbs = _setup(name)
    shape = H.shape_of(w, sub_block_size=sbs, select_parts=parts)
    spb = 64 // sbs
    kp_dev = H.gpu_pool(shape, H.dev(x["k"]))
    ws = N.workspace(shape)
    scores = torch.full((w.rows, w.nbmax), float("nan"), dtype=torch.float32, device="cuda")
    N.nosa_block_scores(shape, H.dev(x["q"]), kp_dev, scores, ws)
    s = H.host(scores)
    ref = O.block_scores(x["q"], O.pool_keys(x["k"], sbs), w.n_blocks, spb).reshape(w.rows, -1)
    assert np.all(np.isnan(s[:, w.n_blocks:]))          # entries past n_blocks untouched
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(s[:, :w.n_blocks] - ref) <= 1e-5 * scale + 1e-6)


@pytest.mark.parametrize("parts", [0, 1, 4])
@pytest.mark.parametrize("name", sorted(CASES))
def test_select(name, parts):
    w, x, sbs = _setup(name)
    shape = H.shape_of(w, sub_block_size=sbs, select_parts=parts)
    q_dev = H.dev(x["q"])
    kp_dev = H.gpu_pool(shape, H.dev(x["k"]))
    ws = N.workspace(shape)
    sel, agn = H.gpu_select(shape, q_dev, kp_dev, H.dev(x["evict"]), ws)
    s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], sbs), w.n_blocks, 64 // sbs)
    H.check_selection(H.host(sel), H.host(agn), s_ref, x["evict"][:, :, :w.n_blocks], w.kq, w.ke)
    # repeat: bitwise identical (deterministic)
    sel2, agn2 = H.gpu_select(shape, q_dev, kp_dev, H.dev(x["evict"]), ws)
    assert torch.equal(sel, sel2) and torch.equal(agn, agn2)


def test_select_ties_lowest_ids():
    # All-zero pooled keys: every block score is 0 -> Gamma_q takes the lowest ids outside Gamma_e.
    # Equal eviction scores -> Gamma_e takes the lowest ids.
    w = small_workload("ties", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=40, kq=6, ke=5, seed=30)
    x = generate(w)
    shape = H.shape_of(w)
    kp = torch.zeros((w.rows, w.nbmax * 2, 128), dtype=torch.float32, device="cuda")
    ev = torch.full((w.batch, w.n_kv_heads, w.nbmax), 0.5, dtype=torch.float32, device="cuda")
    sel, agn = H.gpu_select(shape, H.dev(x["q"]), kp, ev, N.workspace(shape))
    assert H.host(agn).tolist() == [[0, 1, 2, 3, 4]] * w.rows
    assert H.host(sel).tolist() == [list(range(11))] * w.rows


@pytest.mark.parametrize("many", [False, True])
def test_select_short_rows_match_general_topk_on_ties(many):
    # Rows of up to 64 blocks are selected with one block per lane when one workgroup scores and
    # selects a row (and in the one-launch step); scoring the same rows in two parts sends them
    # through the general top-k instead.  Eviction scores on a coarse grid and pooled sub-block keys
    # drawn from six vectors make many keys exactly equal, so the paths must agree on every tie
    # (lower id first) with each other and with the oracle, on a fresh step and on a step with
    # arrivals under strict eviction.
    B, Hkv, G, d = (64, 4, 4, 64) if many else (2, 2, 4, 128)
    n, extra, kq, ke = 48, 5, 6, 8
    nbmax, R, k = n + extra, B * Hkv, kq + ke
    rng = np.random.default_rng(4242 + int(many))
    q = f32_to_bf16_bits(rng.standard_normal((B, Hkv * G, d)).astype(np.float32))
    vecs = rng.standard_normal((6, d)).astype(np.float32)
    kp = np.ascontiguousarray(vecs[rng.integers(0, 6, size=(R, nbmax * 2))])
    ev = (rng.integers(0, 5, size=(B, Hkv, nbmax)) / 4.0).astype(np.float32)
    shape = N.make_shape(batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=d, n_blocks=n, n_blocks_max=nbmax,
                         kq=kq, ke=ke, dtype=N.NOSA_BF16)
    q_dev, kp_dev, ev_dev = H.dev(q), H.dev(kp), H.dev(ev)
    ws, ws2 = N.workspace(shape), N.workspace(shape.copy(select_parts=2))
    kp_ref = kp.reshape(B, Hkv, nbmax * 2, d).astype(np.float64)
    kv = torch.zeros((B, Hkv, nbmax, 64, d), dtype=torch.bfloat16, device="cuda") if many else None
    prev = prev2 = agn_ref = None
    for n_prev, nn in ((0, n), (n, nbmax)):
        sh = shape.copy(n_blocks=nn)
        sel_a, agn_a = H.gpu_select(sh, q_dev, kp_dev, ev_dev, ws, n_prev=n_prev, agn=None if prev is None else prev.clone())
        sel_b, agn_b = H.gpu_select(sh.copy(select_parts=2), q_dev, kp_dev, ev_dev, ws2, n_prev=n_prev,
                                    agn=None if prev2 is None else prev2.clone())
        assert torch.equal(sel_a, sel_b) and torch.equal(agn_a, agn_b), "step with n_prev %d" % n_prev
        sel_r, agn_r, _ = O.select(O.block_scores(q, kp_ref, nn, 2), ev, kq, ke, n_prev, agn_ref)
        assert np.array_equal(H.host(sel_a).reshape(B, Hkv, k), sel_r)
        assert np.array_equal(H.host(agn_a).reshape(B, Hkv, ke), agn_r)
        if many:   # 256 rows and one split per row: the one-launch step
            agn_c = torch.full((R, ke), -7, dtype=torch.int32, device="cuda") if prev is None else prev.clone()
            sel_c = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
            out = torch.empty((B, Hkv * G, d), dtype=torch.bfloat16, device="cuda")
            N.nosa_decode_step(sh, q_dev, kp_dev, ev_dev, n_prev, agn_c, sel_c, kv, kv, nbmax, 0.125, out, ws)
            torch.cuda.synchronize()
            assert torch.equal(sel_c, sel_a) and torch.equal(agn_c, agn_a)
        prev, prev2, agn_ref = agn_a, agn_b, agn_r


def test_select_planted_blocks():
    # Blocks whose keys carry an offset along the summed group query must be chosen by the
    # query-aware part whatever their eviction score.
    w = small_workload("planted", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=60, kq=3, ke=4,
                       seed=31, block_offset_sigma=0.0, dtype="f32")
    x = generate(w)
    k = x["k"].copy()
    planted = {(0, 0): [5, 17, 44], (0, 1): [0, 59, 30], (1, 0): [12, 13, 14], (1, 1): [58, 2, 40]}
    for (b, g), blks in planted.items():
        qs = x["q"][b, g * 4:(g + 1) * 4].sum(axis=0)
        for j, blk in enumerate(blks):
            k[b, g, blk] += (4.0 + j) * qs / np.linalg.norm(qs)
    ev = np.zeros_like(x["evict"])
    for (b, g), blks in planted.items():
        ev[b, g] = np.linspace(0, 1, w.nbmax, dtype=np.float32)  # Gamma_e = last 4 blocks
        ev[b, g, blks] = -1.0
    shape = H.shape_of(w)
    kp = H.gpu_pool(shape, H.dev(k))
    sel, agn = H.gpu_select(shape, H.dev(x["q"]), kp, H.dev(ev), N.workspace(shape))
    sel = H.host(sel).reshape(2, 2, 7)
    for (b, g), blks in planted.items():
        assert set(blks) <= set(sel[b, g].tolist())


@pytest.mark.parametrize("splits", [0, 1, 2, 5])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_decode(name, splits):
    w, x, sbs = _setup(name)
    shape = H.shape_of(w, sub_block_size=sbs, decode_splits=splits)
    rng = np.random.default_rng(w.seed)
    k = w.k
    table = np.stack([np.sort(rng.choice(w.n_blocks, k, replace=False)) for _ in range(w.rows)]).astype(np.int32)
    table = table.reshape(w.batch, w.n_kv_heads, k)
    out = H.gpu_decode(shape, H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), w.nbmax, H.dev(table), N.workspace(shape))
    ref = O.attention(x["q"], x["k"], x["v"], table)
    H.check_attention(H.host(out), ref, w.dtype, name)


def test_sparse_decode_store_layout_and_order_invariance():
    # Table in a shuffled order over a store with extra blocks gives the same attention (up to
    # rounding): the softmax runs over the set of selected tokens.
    w = small_workload("perm", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=30, n_blocks_max=35,
                       kq=6, ke=6, seed=32)
    x = generate(w)
    shape = H.shape_of(w)
    rng = np.random.default_rng(3)
    table = np.stack([rng.choice(w.nbmax, 12, replace=False) for _ in range(w.rows)]).astype(np.int32)
    table = table.reshape(2, 2, 12)
    ws = N.workspace(shape)
    o1 = H.host(H.gpu_decode(shape, H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), w.nbmax, H.dev(table), ws))
    ref = O.attention(x["q"], x["k"], x["v"], table)
    H.check_attention(o1, ref, "bf16", "shuffled table")


def test_sparse_decode_skips_out_of_range_ids():
    w = small_workload("skip", batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, n_blocks=10, kq=2, ke=2, seed=33)
    x = generate(w)
    shape = H.shape_of(w, decode_splits=1)
    table = np.array([[[1, 4, -1, 7]]], np.int32)
    out = H.host(H.gpu_decode(shape, H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), w.nbmax, H.dev(table),
                              N.workspace(shape)))
    ref = O.attention(x["q"], x["k"], x["v"], np.array([[[1, 4, 7]]], np.int32))
    H.check_attention(out, ref, "bf16", "skip")


def test_multistep_select_with_arrivals():
    # Strict eviction across steps: blocks arrive one by one; Gamma_e on the GPU follows the
    # oracle exactly, and the selection matches within the tie band.
    w = small_workload("multi", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=30, n_blocks_max=46,
                       kq=5, ke=6, seed=34)
    x = generate(w)
    shape0 = H.shape_of(w)
    kp_dev = H.gpu_pool(shape0, H.dev(x["k"]))
    ev_dev = H.dev(x["evict"])
    ws = N.workspace(shape0)
    kp_ref = O.pool_keys(x["k"], 32)
    rng = np.random.default_rng(5)
    qf = x["q"]
    n, agn_dev, agn_ref = 30, None, None
    for t in range(12):
        n_prev = 0 if t == 0 else n
        if t > 0:
            n = min(w.nbmax, n + int(rng.integers(0, 3)))
        q_t = H.dev(qf)
        shape = shape0.copy(n_blocks=n)
        sel, agn_dev = H.gpu_select(shape, q_t, kp_dev, ev_dev, ws, n_prev=n_prev, agn=agn_dev)
        s_ref = O.block_scores(qf, kp_ref[:, :, :n * 2], n, 2)
        H.check_selection(H.host(sel), H.host(agn_dev), s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref)
        _, agn_ref, _ = O.select(s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref)
        qf = (H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32)
        from nosa_inputs import f32_to_bf16_bits
        qf = f32_to_bf16_bits(qf)


@pytest.mark.parametrize("side_stream", [False, True])
def test_cache_update_and_offload_decode(side_stream):
    # Offload loop at reduced size: GPU maps, tables, miss lists and cache bytes follow the oracle's
    # cache simulation exactly; attention from the cache matches the oracle.
    w = small_workload("offload", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=40, n_blocks_max=44,
                       kq=6, ke=6, seed=35, cache_slots=15)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C = w.rows, w.k, w.cache_slots
    hk, hv = H.pinned(x["k"]), H.pinned(x["v"])
    ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, 128), dtype=torch.bfloat16, device="cuda")
    cv = torch.zeros_like(ck)
    sob = torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda")
    bos = torch.full((R, C), -1, dtype=torch.int32, device="cuda")
    table = torch.empty((R, k), dtype=torch.int32, device="cuda")
    mcnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    mlist = torch.empty((R, k, 2), dtype=torch.int32, device="cuda")
    sob_ref = np.full((R, w.nbmax), -1, np.int32)
    bos_ref = np.full((R, C), -1, np.int32)
    ck_ref = np.zeros((w.batch, w.n_kv_heads, C, 64, 128), np.uint16)
    cv_ref = np.zeros_like(ck_ref)
    kp_dev = H.gpu_pool(shape0, H.dev(x["k"]))
    ws = N.workspace(shape0)
    ev_dev = H.dev(x["evict"])
    copy_stream = torch.cuda.Stream() if side_stream else None
    rng = np.random.default_rng(6)
    qf = x["q"]
    n, agn = 40, None
    from nosa_inputs import f32_to_bf16_bits
    for t in range(10):
        n_prev = 0 if t == 0 else n
        if t in (3, 6, 7):
            n += 1
        shape = shape0.copy(n_blocks=n)
        q_dev = H.dev(qf)
        sel, agn = H.gpu_select(shape, q_dev, kp_dev, ev_dev, ws, n_prev=n_prev, agn=agn)
        N.nosa_cache_update(shape, sel, sob, bos, table, mcnt, mlist, hk, hv, ck, cv, copy=copy_stream)
        out = H.gpu_decode(shape, q_dev, ck, cv, C, table, ws)
        torch.cuda.synchronize()
        sel_h = H.host(sel)
        tab_ref, mc_ref, ml_ref = O.cache_step(sel_h, sob_ref, bos_ref)
        assert np.array_equal(H.host(sob), sob_ref) and np.array_equal(H.host(bos), bos_ref)
        assert np.array_equal(H.host(table), tab_ref) and np.array_equal(H.host(mcnt), mc_ref)
        ml = H.host(mlist)
        for r in range(R):
            assert np.array_equal(ml[r, :mc_ref[r]], ml_ref[r, :mc_ref[r]])
        O.gather(mc_ref.reshape(w.batch, w.n_kv_heads), ml_ref.reshape(w.batch, w.n_kv_heads, k, 2), x["k"], ck_ref)
        O.gather(mc_ref.reshape(w.batch, w.n_kv_heads), ml_ref.reshape(w.batch, w.n_kv_heads, k, 2), x["v"], cv_ref)
        assert np.array_equal(H.host(ck), ck_ref) and np.array_equal(H.host(cv), cv_ref)
        ref = O.attention(qf, x["k"], x["v"], sel_h.reshape(w.batch, w.n_kv_heads, k))
        H.check_attention(H.host(out), ref, "bf16", "offload step %d" % t)
        qf = f32_to_bf16_bits((H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32))


def test_c1_tiny_end_to_end():
    from nosa_inputs import WORKLOADS
    w = WORKLOADS["C1"]
    x = generate(w)
    shape = H.shape_of(w)
    q_dev = H.dev(x["q"])
    kp = H.gpu_pool(shape, H.dev(x["k"]))
    ws = N.workspace(shape)
    sel, agn = H.gpu_select(shape, q_dev, kp, H.dev(x["evict"]), ws)
    s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], 32), w.n_blocks, 2)
    H.check_selection(H.host(sel), H.host(agn), s_ref, x["evict"], w.kq, w.ke)
    out = H.gpu_decode(shape, q_dev, H.dev(x["k"]), H.dev(x["v"]), w.nbmax, sel, ws)
    ref = O.attention(x["q"], x["k"], x["v"], H.host(sel).reshape(1, 1, -1))
    H.check_attention(H.host(out), ref, "f32", "C1")


@pytest.mark.parametrize("n,kq,ke,parts", [(513, 16, 16, 0), (1300, 40, 24, 3), (1300, 40, 24, 1), (2048, 32, 32, 0),
                                           (5000, 32, 32, 7), (700, 300, 100, 0), (4100, 20, 30, 1),
                                           (3000, 8, 8, 5), (1500, 10, 90, 4), (2040, 64, 0, 7)])
def test_select_long_rows(n, kq, ke, parts):
    # Rows longer than 512 blocks take the bounded-candidate top-k; the next step (blocks arrive,
    # strict eviction) runs the same path with few query-agnostic candidates.  The cases cover one
    # to a few long scoring slices, a budget of 100 with 90 query-agnostic blocks, and ke = 0.
    rng = np.random.default_rng(n)
    B, Hkv, G, d = 2, 2, 4, 128
    nbmax = n + 9
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    kp = rng.standard_normal((B, Hkv, nbmax * 2, d)).astype(np.float32)
    ev = rng.random((B, Hkv, nbmax), dtype=np.float32)
    shape = N.make_shape(batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=d, n_blocks=n, n_blocks_max=nbmax,
                         kq=kq, ke=ke, dtype=N.NOSA_F32, select_parts=parts)
    ws = N.workspace(shape)
    q_dev, kp_dev, ev_dev = H.dev(q), H.dev(kp), H.dev(ev)
    sel, agn = H.gpu_select(shape, q_dev, kp_dev, ev_dev, ws)
    s_ref = O.block_scores(q, kp.astype(np.float64)[:, :, :2 * n], n, 2)
    H.check_selection(H.host(sel), H.host(agn), s_ref, ev, kq, ke)
    _, agn_ref, _ = O.select(s_ref, ev, kq, ke)
    n2 = n + 9
    shape2 = shape.copy(n_blocks=n2)
    sel2, agn2 = H.gpu_select(shape2, q_dev, kp_dev, ev_dev, ws, n_prev=n, agn=agn)
    s_ref2 = O.block_scores(q, kp.astype(np.float64), n2, 2)
    H.check_selection(H.host(sel2), H.host(agn2), s_ref2, ev, kq, ke, n, agn_ref)


def test_select_long_rows_exact_ties_go_to_lower_ids():
    # Integer-valued pooled keys and eviction scores make many keys exactly equal; with five scoring
    # slices of 600 blocks, ties must go to the lower block id in both subsets, exactly as in the
    # oracle.
    rng = np.random.default_rng(77)
    B, Hkv, G, d, n, kq, ke, parts = 2, 2, 2, 64, 3000, 6, 10, 5
    q = np.ones((B, Hkv * G, d), np.float32)
    kp = rng.integers(0, 2, size=(B, Hkv, n * 2, d)).astype(np.float32)
    ev = rng.integers(0, 3, size=(B, Hkv, n)).astype(np.float32)
    shape = N.make_shape(batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=d, n_blocks=n, kq=kq, ke=ke,
                         dtype=N.NOSA_F32, select_parts=parts)
    sel, agn = H.gpu_select(shape, H.dev(q), H.dev(kp), H.dev(ev), N.workspace(shape))
    s_ref = O.block_scores(q, kp, n, 2)
    sel_o, agn_o, _ = O.select(s_ref, ev, kq, ke)
    assert np.array_equal(H.host(agn).reshape(B, Hkv, ke), agn_o)
    assert np.array_equal(H.host(sel).reshape(B, Hkv, kq + ke), sel_o)


def test_select_long_rows_all_ties():
    # Equal scores everywhere: the winners are the lowest ids.  At 16384 blocks the chunk-maximum
    # bound leaves too many candidates, so this also runs the radix-select fallback.
    B, Hkv, G, d, n, kq, ke = 1, 2, 4, 64, 16384, 32, 32
    shape = N.make_shape(batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=d, n_blocks=n, kq=kq, ke=ke,
                         dtype=N.NOSA_BF16)
    q = torch.ones((B, Hkv * G, d), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((B * Hkv, n * 2, d), dtype=torch.float32, device="cuda")
    ev = torch.full((B, Hkv, n), 0.25, dtype=torch.float32, device="cuda")
    sel, agn = H.gpu_select(shape, q, kp, ev, N.workspace(shape))
    assert H.host(agn).tolist() == [list(range(ke))] * 2
    assert H.host(sel).tolist() == [list(range(kq + ke))] * 2


def test_select_many_rows_one_workgroup_each():
    # 256 rows: the plan gives every row its own 256-thread workgroup that scores and selects.
    w = small_workload("wide", batch=64, n_q_heads=16, n_kv_heads=4, head_dim=64, n_blocks=20, kq=3, ke=5, seed=36)
    x = generate(w)
    shape = H.shape_of(w)
    q_dev = H.dev(x["q"])
    kp = H.gpu_pool(shape, H.dev(x["k"]))
    ws = N.workspace(shape)
    sel, agn = H.gpu_select(shape, q_dev, kp, H.dev(x["evict"]), ws)
    s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], 32), w.n_blocks, 2)
    H.check_selection(H.host(sel), H.host(agn), s_ref, x["evict"], w.kq, w.ke)
    out = H.gpu_decode(shape, q_dev, H.dev(x["k"]), H.dev(x["v"]), w.nbmax, sel, ws)
    ref = O.attention(x["q"], x["k"], x["v"], H.host(sel).reshape(w.batch, w.n_kv_heads, w.k))
    H.check_attention(H.host(out), ref, "bf16", "wide")


@pytest.mark.parametrize("n,kq,ke,ns,nw,parts", [(40, 4, 10, 1, 4, 0), (64, 6, 12, 1, 11, 3), (300, 16, 48, 1, 16, 0),
                                                 (700, 16, 48, 2, 16, 0), (33, 3, 9, 0, 9, 1), (50, 5, 3, 3, 0, 0)])
def test_select_sink_window(n, kq, ke, ns, nw, parts):
    # Sink and window blocks always join the query-agnostic subset; the rest is ranked by
    # eviction score under strict eviction, over a few steps with blocks arriving.
    rng = np.random.default_rng(n + nw)
    B, Hkv, G, d = 2, 2, 4, 128
    nbmax = n + 12
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    kp = rng.standard_normal((B, Hkv, nbmax * 2, d)).astype(np.float32)
    ev = rng.random((B, Hkv, nbmax), dtype=np.float32)
    shape0 = N.make_shape(batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=d, n_blocks=n, n_blocks_max=nbmax,
                          kq=kq, ke=ke, dtype=N.NOSA_F32, select_parts=parts, sink_blocks=ns, window_blocks=nw)
    ws = N.workspace(shape0)
    q_dev, kp_dev, ev_dev = H.dev(q), H.dev(kp), H.dev(ev)
    kp64 = kp.astype(np.float64)
    agn_dev, agn_ref, cur, prev = None, None, n, 0
    for step, grow in enumerate([0, 1, 0, 3, 2, 1]):
        cur = min(nbmax, cur + grow)
        shape = shape0.copy(n_blocks=cur)
        sel, agn_dev = H.gpu_select(shape, q_dev, kp_dev, ev_dev, ws, n_prev=prev, agn=agn_dev)
        s_ref = O.block_scores(q, kp64[:, :, :2 * cur], cur, 2)
        H.check_selection(H.host(sel), H.host(agn_dev), s_ref, ev, kq, ke, prev, agn_ref, ns, nw)
        _, agn_ref, _ = O.select(s_ref, ev, kq, ke, prev, agn_ref, ns, nw)
        E = H.host(agn_dev)
        for r in range(B * Hkv):
            assert set(range(ns)) | set(range(cur - nw, cur)) <= set(E[r].tolist())
        prev = cur


@pytest.mark.parametrize("dtype,d,G,side_stream", [("bf16", 128, 4, True), ("bf16", 128, 4, False),
                                                   ("f32", 64, 2, True), ("bf16", 64, 8, True)])
def test_offload_decode_matches_cache_update_then_decode(dtype, d, G, side_stream):
    # nosa_offload_decode (hits attended while the misses are copied, then the misses, one merge)
    # against nosa_cache_update + nosa_sparse_decode run on a second copy of the state: maps, table,
    # miss list and cache bytes identical, attention within tolerance of the oracle at every step.
    # Step 0 is cold (every entry a miss: the hit launch has only empty splits); later steps mix.
    w = small_workload("offload2", batch=2, n_q_heads=2 * G, n_kv_heads=2, head_dim=d, n_blocks=40,
                       n_blocks_max=44, kq=6, ke=6, seed=36, cache_slots=15, dtype=dtype)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C = w.rows, w.k, w.cache_slots
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    hk, hv = H.pinned(x["k"]), H.pinned(x["v"])

    def state():
        ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, d), dtype=tdt, device="cuda")
        return dict(ck=ck, cv=torch.zeros_like(ck),
                    sob=torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda"),
                    bos=torch.full((R, C), -1, dtype=torch.int32, device="cuda"),
                    table=torch.full((R, k), -9, dtype=torch.int32, device="cuda"),
                    mcnt=torch.full((R,), -9, dtype=torch.int32, device="cuda"),
                    mlist=torch.full((R, k, 2), -9, dtype=torch.int32, device="cuda"))
    A, B = state(), state()
    kp_dev = H.gpu_pool(shape0, H.dev(x["k"]))
    ws_a, ws_b = N.workspace(shape0), N.workspace(shape0)
    ev_dev = H.dev(x["evict"])
    copy_stream = torch.cuda.Stream() if side_stream else None
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(8)
    qf = x["q"]
    n, agn = 40, None
    from nosa_inputs import f32_to_bf16_bits
    for t in range(8):
        n_prev = 0 if t == 0 else n
        if t in (2, 5):
            n += 1
        shape = shape0.copy(n_blocks=n)
        q_dev = H.dev(qf)
        sel, agn = H.gpu_select(shape, q_dev, kp_dev, ev_dev, ws_a, n_prev=n_prev, agn=agn)
        N.nosa_cache_update(shape, sel, A["sob"], A["bos"], A["table"], A["mcnt"], A["mlist"], hk, hv, A["ck"],
                            A["cv"])
        out_a = H.gpu_decode(shape, q_dev, A["ck"], A["cv"], C, A["table"], ws_a, scale)
        out_b = torch.full_like(out_a, float("nan"))
        N.nosa_offload_decode(shape, q_dev, sel, B["sob"], B["bos"], B["table"], B["mcnt"], B["mlist"], hk, hv,
                              B["ck"], B["cv"], scale, out_b, ws_b, copy=copy_stream)
        torch.cuda.synchronize()
        mc = H.host(A["mcnt"])
        for key in ("sob", "bos", "table", "mcnt", "ck", "cv"):
            assert torch.equal(A[key].view(torch.int16) if A[key].dtype == torch.bfloat16 else A[key],
                               B[key].view(torch.int16) if B[key].dtype == torch.bfloat16 else B[key]), (t, key)
        mla, mlb = H.host(A["mlist"]), H.host(B["mlist"])
        for r in range(R):
            assert np.array_equal(mla[r, :mc[r]], mlb[r, :mc[r]])
        if t == 0:
            assert np.all(mc == k)            # cold cache: every entry misses
        sel_h = H.host(sel).reshape(w.batch, w.n_kv_heads, k)
        ref = O.attention(qf, x["k"], x["v"], sel_h, scale)
        H.check_attention(H.host(out_b), ref, dtype, "offload_decode step %d" % t)
        H.check_attention(H.host(out_a), ref, dtype, "cache_update + sparse_decode step %d" % t)
        if dtype == "bf16":
            qf = f32_to_bf16_bits((H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32))
        else:
            qf = (qf + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32)


def test_sparse_decode_split_with_no_valid_block():
    # A split whose every table entry is skipped contributes an empty partial, not a NaN: the
    # result equals attention over the remaining valid entries.
    w = small_workload("empty_split", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=32, kq=8, ke=8,
                       seed=37)
    x = generate(w)
    shape = H.shape_of(w, decode_splits=4)
    table = np.tile(np.arange(16, dtype=np.int32), (2, 1))
    table[:, 4:8] = -1                  # split 1 (entries 4..7) has nothing to attend
    table[1, 12:16] = 999               # and split 3 of row 1: out of range, skipped
    ws = N.workspace(shape)
    out = H.gpu_decode(shape, H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), w.nbmax, H.dev(table), ws)
    torch.cuda.synchronize()
    keep = [[i for i in range(16) if table[r, i] >= 0 and table[r, i] < w.nbmax] for r in range(2)]
    for r in range(2):
        sub = np.array(keep[r], dtype=np.int32)
        ref = O.attention(x["q"][:, 4 * r:4 * r + 4].copy(), x["k"][:, r:r + 1].copy(), x["v"][:, r:r + 1].copy(),
                          sub.reshape(1, 1, -1))
        H.check_attention(H.host(out)[:, 4 * r:4 * r + 4], ref, "bf16", "row %d" % r)


@pytest.mark.parametrize("unit_bytes,pinned_src", [(16, False), (256, True), (256, False), (16384, True)])
def test_gather_units_matches_oracle(unit_bytes, pinned_src):
    # Random transfer lists (distinct destinations, some pairs out of range) at the granularity of a
    # 16-byte chunk, one token's key row (256 B) and one KV block (16 KiB): the destination matches
    # the oracle byte for byte, untouched units included.
    rng = np.random.default_rng(unit_bytes)
    ns, nd = 3000 if unit_bytes < 16384 else 96, 2000 if unit_bytes < 16384 else 64
    n = nd // 2
    src = rng.integers(0, 2 ** 31, size=ns * unit_bytes // 4, dtype=np.int64).astype(np.int32)
    dst0 = rng.integers(0, 2 ** 31, size=nd * unit_bytes // 4, dtype=np.int64).astype(np.int32)
    su = rng.integers(0, ns, size=n).astype(np.int32)
    du = rng.permutation(nd)[:n].astype(np.int32)
    su[::97] = ns + 5                 # out of range: skipped
    du[5::101] = -1
    ref = dst0.copy()
    O.gather_units(src, ref, unit_bytes, su, du)
    s_t = H.pinned(src) if pinned_src else H.dev(src)
    d_t = H.dev(dst0)
    N.nosa_gather_units(s_t, ns, d_t, nd, unit_bytes, H.dev(su), H.dev(du), n)
    torch.cuda.synchronize()
    assert np.array_equal(H.host(d_t), ref)
    N.nosa_gather_units(s_t, ns, d_t, nd, unit_bytes, H.dev(su), H.dev(du), 0)   # no-op
    torch.cuda.synchronize()
    assert np.array_equal(H.host(d_t), ref)


def test_multistep_select_with_changing_eviction_scores():
    # Eviction scores redrawn every step: strict eviction on the GPU still admits only previous
    # members and arrivals, exactly as the oracle (with fixed scores the rule is invisible).
    w = small_workload("evict_change", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=40,
                       n_blocks_max=48, kq=5, ke=6, seed=38)
    x = generate(w)
    shape0 = H.shape_of(w)
    kp_dev = H.gpu_pool(shape0, H.dev(x["k"]))
    ws = N.workspace(shape0)
    kp_ref = O.pool_keys(x["k"], 32)
    rng = np.random.default_rng(12)
    n, agn_dev, agn_ref = 40, None, None
    s_ref = O.block_scores(x["q"], kp_ref[:, :, :2 * n], n, 2)
    for t in range(8):
        n_prev = 0 if t == 0 else n
        if t in (3, 5):
            n += 2
            s_ref = O.block_scores(x["q"], kp_ref[:, :, :2 * n], n, 2)
        ev = rng.random((w.batch, w.n_kv_heads, w.nbmax), dtype=np.float32)
        shape = shape0.copy(n_blocks=n)
        sel, agn_dev = H.gpu_select(shape, H.dev(x["q"]), kp_dev, H.dev(ev), ws, n_prev=n_prev, agn=agn_dev)
        H.check_selection(H.host(sel), H.host(agn_dev), s_ref, ev, w.kq, w.ke, n_prev, agn_ref)
        _, agn_ref, _ = O.select(s_ref, ev, w.kq, w.ke, n_prev, agn_ref)
        if t > 0:
            # members are previous members or arrivals only
            prev = set(np.asarray(prev_agn).reshape(-1, w.ke)[0].tolist())
            cur = set(agn_ref.reshape(-1, w.ke)[0].tolist())
            assert cur <= prev | set(range(n_prev, n))
        prev_agn = agn_ref.copy()


@pytest.mark.parametrize("k,splits,G,d", [(600, 0, 8, 128), (600, 37, 4, 128), (257, 0, 1, 64), (1000, 0, 2, 64)])
def test_sparse_decode_large_budget(k, splits, G, d):
    # Budgets of hundreds of blocks (tens of thousands of tokens): many splits, a merge over many
    # partials, ragged last splits (600 = 37 * 16 + 8), and the automatic plan.
    n = k + 40
    w = small_workload("large_k", batch=1, n_q_heads=2 * G, n_kv_heads=2, head_dim=d, n_blocks=n, kq=k // 2,
                       ke=k - k // 2, seed=40 + k % 7)
    x = generate(w)
    shape = H.shape_of(w, decode_splits=splits)
    rng = np.random.default_rng(k)
    table = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(w.rows)]).astype(np.int32)
    table = table.reshape(w.batch, w.n_kv_heads, k)
    out = H.gpu_decode(shape, H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), w.nbmax, H.dev(table), N.workspace(shape))
    torch.cuda.synchronize()
    ref = O.attention(x["q"], x["k"], x["v"], table)
    print(H.check_attention(H.host(out), ref, w.dtype, "k=%d" % k))


def test_offload_decode_from_two_host_threads():
    # Two host threads drive independent offload loops, each with its own compute and copy streams:
    # every step's maps, table, cache bytes and output are bit-identical to the same loop run alone.
    import threading
    w = small_workload("threads", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=40, n_blocks_max=44,
                       kq=6, ke=6, seed=39, cache_slots=12)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C = w.rows, w.k, w.cache_slots
    hk, hv = H.pinned(x["k"]), H.pinned(x["v"])
    kp_dev = H.gpu_pool(shape0, H.dev(x["k"]))
    ev_dev = H.dev(x["evict"])
    rng = np.random.default_rng(10)
    from nosa_inputs import f32_to_bf16_bits
    qs = [x["q"]]
    for _ in range(7):
        qs.append(f32_to_bf16_bits((H.as_f64(qs[-1]) + 0.4 * rng.standard_normal(x["q"].shape)).astype(np.float32)))
    q_dev = [H.dev(q) for q in qs]
    torch.cuda.synchronize()

    def run(results, key):
        torch.cuda.set_device(0)
        compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
        with torch.cuda.stream(compute):
            ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, 128), dtype=torch.bfloat16, device="cuda")
            cv = torch.zeros_like(ck)
            sob = torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda")
            bos = torch.full((R, C), -1, dtype=torch.int32, device="cuda")
            table = torch.zeros((R, k), dtype=torch.int32, device="cuda")
            mcnt = torch.zeros((R,), dtype=torch.int32, device="cuda")
            mlist = torch.zeros((R, k, 2), dtype=torch.int32, device="cuda")
            agn = torch.zeros((R, w.ke), dtype=torch.int32, device="cuda")
            sel = torch.zeros((R, k), dtype=torch.int32, device="cuda")
            ws = N.workspace(shape0)
            rec = []
            for t in range(8):
                out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
                N.nosa_select(shape0, q_dev[t], kp_dev, ev_dev, 0 if t == 0 else w.n_blocks, agn, sel, ws, compute)
                N.nosa_offload_decode(shape0, q_dev[t], sel, sob, bos, table, mcnt, mlist, hk, hv, ck, cv,
                                      1.0 / np.sqrt(128), out, ws, compute, copy)
                rec.append((out, table.clone(), mcnt.clone(), sob.clone()))
            rec.append((ck, cv))
        compute.synchronize()
        results[key] = rec

    alone = {}
    run(alone, "a")
    both = {}
    th = [threading.Thread(target=run, args=(both, i)) for i in range(2)]
    for t_ in th:
        t_.start()
    for t_ in th:
        t_.join()
    torch.cuda.synchronize()
    for i in range(2):
        for step_a, step_b in zip(alone["a"], both[i]):
            for a_, b_ in zip(step_a, step_b):
                if a_.dtype == torch.bfloat16:
                    a_, b_ = a_.view(torch.int16), b_.view(torch.int16)
                assert torch.equal(a_, b_), "thread %d differs from the loop run alone" % i


@pytest.mark.parametrize("dtype,splits", [("bf16", 1), ("bf16", 4), ("f32", 1), ("f32", 3)])
def test_sparse_decode_row_with_no_valid_block_gives_zero(dtype, splits):
    # A row whose every table entry lies outside the store attends to no token: its output is 0
    # (defined in the header; the oracle rejects such a table).  The other row is unaffected and
    # matches the oracle over its valid entries.
    w = small_workload("empty_row_" + dtype, batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=24, kq=6,
                       ke=6, dtype=dtype, seed=38)
    x = generate(w)
    print("case", dtype, splits, flush=True)
    shape = H.shape_of(w, decode_splits=splits)
    table = np.tile(np.arange(12, dtype=np.int32) * 2, (2, 1))
    table[0, :] = -1
    table[0, 5] = w.nbmax            # past the store: skipped as well
    ws = N.workspace(shape)
    out = H.host(H.gpu_decode(shape, H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), w.nbmax, H.dev(table), ws))
    torch.cuda.synchronize()
    assert np.all(H.as_f64(out[:, 0:4]) == 0.0)
    ref = O.attention(x["q"][:, 4:8].copy(), x["k"][:, 1:2].copy(), x["v"][:, 1:2].copy(), table[1].reshape(1, 1, -1))
    H.check_attention(out[:, 4:8], ref, dtype, "valid row")


def test_host_map_resolves_pinned_and_device_memory_and_rejects_pageable():
    pinned = torch.empty(4096, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(4096, dtype=torch.uint8, device="cuda")
    assert N.host_map(dev) == dev.data_ptr()
    addr = N.host_map(pinned)
    assert addr != 0
    # the mapped address is what the kernels read: a gather through it copies the pinned bytes
    pinned.copy_(torch.arange(4096, dtype=torch.int32).to(torch.uint8))
    su = torch.arange(16, dtype=torch.int32, device="cuda")
    N.nosa_gather_units(addr, 256, dev, 256, 16, su, su, 16)
    torch.cuda.synchronize()
    assert torch.equal(dev[:256].cpu(), pinned[:256])
    pageable = np.zeros(4096, np.uint8)
    with pytest.raises(N.NosaError) as ei:
        N.nosa_host_map(pageable.ctypes.data)
    assert ei.value.code == N.NOSA_EINVAL
