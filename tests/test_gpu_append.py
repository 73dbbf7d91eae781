"""Parity of the decode append path (nosa_append_kv) with the oracle: stores written token by
token (device and pinned host pools, ragged lengths, skipped sequences), pooled keys built
incrementally and bit-identical to nosa_pool_keys, and a decode loop whose blocks arrive through
appends into the query-agnostic subset under strict eviction, gathered from the host pool."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import f32_to_bf16_bits, generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

BS = 64


def _token(a: np.ndarray, p: int) -> np.ndarray:
    """Token p of every row of a [B, Hkv, nb, 64, d] array -> [B, Hkv, d]."""
    return np.ascontiguousarray(a[:, :, p // BS, p % BS, :])


def _sentinel_like(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return np.full(x.shape, 0x7FC1, np.uint16)     # a NaN pattern no token carries
    return np.full(x.shape, np.nan, np.float32)


@pytest.mark.parametrize("dtype,d,sbs,pinned_store", [("bf16", 128, 32, False), ("f32", 64, 16, False),
                                                      ("bf16", 128, 64, True), ("bf16", 64, 8, True)])
def test_append_tokens_ragged(dtype, d, sbs, pinned_store):
    w = small_workload("append", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=d, n_blocks=4, kq=1, ke=1,
                       dtype=dtype, seed=41)
    x = generate(w)
    shape = H.shape_of(w, sub_block_size=sbs)
    R, nbmax, spb = w.rows, w.nbmax, BS // sbs
    lens = [0, 37 + sbs, nbmax * BS]                   # empty, ragged, full
    place = H.pinned if pinned_store else H.dev
    ks, vs = place(_sentinel_like(x["k"])), place(_sentinel_like(x["v"]))
    kp = torch.full((R, nbmax * spb, d), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((R, d), float("nan"), dtype=torch.float32, device="cuda")
    for p in range(nbmax * BS):
        pos = torch.tensor([p if p < L else -1 for L in lens], dtype=torch.int32, device="cuda")
        N.nosa_append_kv(shape, H.dev(_token(x["k"], p)), H.dev(_token(x["v"], p)), pos, ks, vs, acc, kp)
    torch.cuda.synchronize()
    ksh, vsh = H.host(ks), H.host(vs)
    sent = _sentinel_like(x["k"][:, :, :1, :1, :1]).reshape(-1)[0]
    for b, L in enumerate(lens):
        fk = ksh[b].reshape(w.n_kv_heads, nbmax * BS, d)
        fv = vsh[b].reshape(w.n_kv_heads, nbmax * BS, d)
        src_k = x["k"][b].reshape(w.n_kv_heads, nbmax * BS, d)
        src_v = x["v"][b].reshape(w.n_kv_heads, nbmax * BS, d)
        assert np.array_equal(fk[:, :L].view(np.uint8), src_k[:, :L].view(np.uint8))
        assert np.array_equal(fv[:, :L].view(np.uint8), src_v[:, :L].view(np.uint8))
        tail = fk[:, L:].view(np.uint16 if dtype == "bf16" else np.uint32)
        assert np.all(tail == np.array(sent).view(tail.dtype)), "sequence %d: a token past its length was written" % b
    # pooled keys: finished sub-blocks bit-identical to nosa_pool_keys over the full store, the
    # open ones untouched; and within fp32 rounding of the oracle's fp64 means
    kp_full = H.gpu_pool(shape, H.dev(x["k"]))
    kp_ref = O.pool_keys(x["k"], sbs)
    kph, kfh = H.host(kp).reshape(w.batch, w.n_kv_heads, -1, d), H.host(kp_full).reshape(w.batch, w.n_kv_heads, -1, d)
    for b, L in enumerate(lens):
        m = L // sbs
        assert np.array_equal(kph[b, :, :m].view(np.uint32), kfh[b, :, :m].view(np.uint32))
        assert np.all(np.isnan(kph[b, :, m:]))
        np.testing.assert_allclose(kph[b, :, :m], kp_ref[b, :, :m], rtol=1e-6, atol=1e-6)


def test_append_decode_loop_blocks_arrive_from_host_pool():
    # Prompt of 6 blocks, then 3 blocks' worth of decode tokens appended into the pinned host pool.
    # At step t >= 1 the token of step t-1 (position 6*64 + t - 1) is appended first; a block is
    # visible from the step its last token lands, as an arrival for the query-agnostic subset.
    # Each step selects over the complete blocks, updates the cache from the host pool and attends.
    # Selections, maps and attention follow the oracle.
    w = small_workload("append_loop", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=6,
                       n_blocks_max=9, kq=2, ke=3, seed=42, cache_slots=7)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C, nbmax, d = w.rows, w.k, w.cache_slots, w.nbmax, w.head_dim
    n0 = w.n_blocks
    prompt_k, prompt_v = x["k"].copy(), x["v"].copy()
    prompt_k[:, :, n0:] = 0
    prompt_v[:, :, n0:] = 0
    hk, hv = H.pinned(prompt_k), H.pinned(prompt_v)
    kp = torch.full((R, nbmax * 2, d), float("nan"), dtype=torch.float32, device="cuda")
    N.nosa_pool_keys(shape0, H.dev(prompt_k), 0, n0, kp)        # the prompt's pooled keys
    acc = torch.zeros((R, d), dtype=torch.float32, device="cuda")
    ck = torch.zeros((w.batch, w.n_kv_heads, C, BS, d), dtype=torch.bfloat16, device="cuda")
    cv = torch.zeros_like(ck)
    sob = torch.full((R, nbmax), -1, dtype=torch.int32, device="cuda")
    bos = torch.full((R, C), -1, dtype=torch.int32, device="cuda")
    table = torch.empty((R, k), dtype=torch.int32, device="cuda")
    mcnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    mlist = torch.empty((R, k, 2), dtype=torch.int32, device="cuda")
    ws = N.workspace(shape0)
    ev_dev = H.dev(x["evict"])
    sob_ref = np.full((R, nbmax), -1, np.int32)
    bos_ref = np.full((R, C), -1, np.int32)
    kp_ref = O.pool_keys(x["k"], 32)
    rng = np.random.default_rng(7)
    qf = x["q"]
    agn, agn_ref, n_prev, arrivals = None, None, 0, 0
    steps = 3 * BS + 1
    for t in range(steps):
        if t > 0:
            pos = n0 * BS + t - 1
            N.nosa_append_kv(shape0, H.dev(_token(x["k"], pos)), H.dev(_token(x["v"], pos)),
                             torch.full((w.batch,), pos, dtype=torch.int32, device="cuda"), hk, hv, acc, kp)
        n = (n0 * BS + t) // BS
        shape = shape0.copy(n_blocks=n)
        q_dev = H.dev(qf)
        sel, agn_new = H.gpu_select(shape, q_dev, kp, ev_dev, ws, n_prev=n_prev, agn=agn)
        N.nosa_cache_update(shape, sel, sob, bos, table, mcnt, mlist, hk, hv, ck, cv)
        out = H.gpu_decode(shape, q_dev, ck, cv, C, table, ws)
        torch.cuda.synchronize()
        arrivals += int(t > 0 and n > n_prev)
        check = t in (0, 1, 63, 65, 127, 129, steps - 2) or (t > 0 and n != n_prev)
        sel_h = H.host(sel)
        tab_ref, mc_ref, ml_ref = O.cache_step(sel_h, sob_ref, bos_ref)
        assert np.array_equal(H.host(table), tab_ref) and np.array_equal(H.host(mcnt), mc_ref)
        s_ref = O.block_scores(qf, kp_ref[:, :, :2 * n], n, 2)
        if check:
            H.check_selection(sel_h, H.host(agn_new), s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref)
            ref = O.attention(qf, x["k"], x["v"], sel_h.reshape(w.batch, w.n_kv_heads, k))
            H.check_attention(H.host(out), ref, "bf16", "append loop step %d" % t)
            # the pooled keys of every complete block match the oracle's
            kph = H.host(kp).reshape(w.batch, w.n_kv_heads, -1, d)
            np.testing.assert_allclose(kph[:, :, :2 * n], kp_ref[:, :, :2 * n], rtol=1e-6, atol=1e-6)
        _, agn_ref, _ = O.select(s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref)
        agn, n_prev = agn_new, n
        qf = f32_to_bf16_bits((H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32))
    assert arrivals == 3 and n_prev == nbmax
    # the host pool holds every appended token
    assert np.array_equal(H.host(hk), x["k"]) and np.array_equal(H.host(hv), x["v"])
