"""K/V stores beyond 4 GiB, through attention, selection, the offload gather and the append:
bs32 at 128K context (256 rows of 2048 blocks, 8 GiB per bf16 store), the size class a 288 GB
device holds.  Row r of a store starts at r x 32 MiB, so rows from 64 on sit past 2^31 bytes and
rows from 128 on past 2^31 elements: any 32-bit offset in pooling, scoring, selection, attention,
gather or append would wrap there.  The inputs follow the resident workloads' recipe (K noise
plus per-block mean offsets, V ~ N(0, 1), eviction scores ~ U(0, 1)) but are drawn on the device
with torch's seeded generator, since the host-side draw of 2 x 4.3e9 values would take minutes;
the oracle recomputes each sampled row from host copies of the same inputs."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import WORKLOADS  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

B, HQ, HKV, D, NB, KQ, KE = 32, 32, 8, 128, 2048, 32, 32
G = HQ // HKV
ROWS = (0, 63, 64, 127, 128, 191, 255)          # before and after 2^31 bytes and 2^31 elements


def _inputs(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    sigma = WORKLOADS["C5"].block_offset_sigma
    q = torch.randn((B, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, HKV, NB, 64, D), generator=g, device="cuda", dtype=torch.bfloat16)
    k.add_((torch.randn((B, HKV, NB, 1, D), generator=g, device="cuda") * sigma).to(torch.bfloat16))
    v = torch.randn((B, HKV, NB, 64, D), generator=g, device="cuda", dtype=torch.bfloat16)
    ev = torch.rand((B * HKV, NB), generator=g, device="cuda")
    return q, k, v, ev


def test_stores_beyond_4gib_step_and_two_calls_match_oracle_on_sampled_rows():
    need = 2 * B * HKV * NB * 64 * D * 2 + (6 << 30)
    torch.cuda.empty_cache()                        # release what earlier tests left reserved
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip("needs %.1f GiB of free device memory, %.1f GiB free" % (need / 2**30, free / 2**30))
    q, k, v, ev = _inputs(20261204)
    assert k.numel() * k.element_size() == 8 << 30
    shape = N.make_shape(batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, n_blocks=NB, n_blocks_max=NB,
                         kq=KQ, ke=KE, sub_block_size=32, dtype=N.NOSA_BF16)
    kp = H.gpu_pool(shape, k)
    ws = N.workspace(shape)
    R, kk = B * HKV, KQ + KE
    scale = 1.0 / np.sqrt(D)
    # the one-call step, as the benchmark runs it at this shape
    agn1 = torch.full((R, KE), -7, dtype=torch.int32, device="cuda")
    sel1 = torch.full((R, kk), -7, dtype=torch.int32, device="cuda")
    out1 = torch.full((B, HQ, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    N.nosa_decode_step(shape, q, kp, ev, 0, agn1, sel1, k, v, NB, scale, out1, ws)
    # the two calls
    sel2, agn2 = H.gpu_select(shape, q, kp, ev, ws)
    out2 = H.gpu_decode(shape, q, k, v, NB, sel2, ws, scale)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel2) and torch.equal(agn1, agn2)
    sel_h, agn_h, ev_h = H.host(sel1), H.host(agn1), H.host(ev)
    q_h = H.host(q)
    for r in ROWS:
        b, h = divmod(r, HKV)
        k_r = H.host(k[b, h]).reshape(1, 1, NB, 64, D)
        v_r = H.host(v[b, h]).reshape(1, 1, NB, 64, D)
        q_r = q_h[b:b + 1, h * G:(h + 1) * G]
        kp_ref = O.pool_keys(k_r, 32)
        np.testing.assert_allclose(H.host(kp[r]).reshape(kp_ref.shape), kp_ref, rtol=1e-6, atol=1e-6)
        s_ref = O.block_scores(q_r, kp_ref, NB, 2)
        H.check_selection(sel_h[r].reshape(1, 1, kk), agn_h[r].reshape(1, 1, KE), s_ref,
                          ev_h[r].reshape(1, 1, NB), KQ, KE)
        ref = O.attention(q_r, k_r, v_r, sel_h[r].reshape(1, 1, kk))
        for out in (out1, out2):
            H.check_attention(H.host(out[b:b + 1, h * G:(h + 1) * G]), ref, "bf16", "row %d" % r)


def test_offload_from_host_pool_beyond_4gib_matches_oracle():
    # The pinned host pool holds 8 GiB per store; a cold step (every entry missed) and a step after
    # a query drift (hits and misses) run through nosa_offload_decode with the gather on a copy
    # stream.  Maps, tables, miss lists and every byte of the GPU cache follow the oracle's cache
    # simulation and gather on all 256 rows; selection and attention are checked on sampled rows.
    import psutil
    C = 64
    store = B * HKV * NB * 64 * D * 2
    torch.cuda.empty_cache()                        # release what earlier tests left reserved
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * store + (6 << 30) or psutil.virtual_memory().available < 3 * store + (8 << 30):
        pytest.skip("needs 22 GiB of free device memory and 32 GiB of free host memory")
    q, k, v, ev = _inputs(20261205)
    shape = N.make_shape(batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, n_blocks=NB, n_blocks_max=NB,
                         kq=KQ, ke=KE, sub_block_size=32, cache_slots=C, dtype=N.NOSA_BF16)
    kp = H.gpu_pool(shape, k)
    hk = torch.empty(k.shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(v.shape, dtype=torch.bfloat16, pin_memory=True)
    hk.copy_(k)
    hv.copy_(v)
    del k, v
    torch.cuda.empty_cache()
    hk_h, hv_h = H.host(hk), H.host(hv)              # views of the pinned pool, no copy
    R, kk = B * HKV, KQ + KE
    ck = torch.zeros((B, HKV, C, 64, D), dtype=torch.bfloat16, device="cuda")
    cv = torch.zeros_like(ck)
    sob = torch.full((R, NB), -1, dtype=torch.int32, device="cuda")
    bos = torch.full((R, C), -1, dtype=torch.int32, device="cuda")
    table = torch.full((R, kk), -9, dtype=torch.int32, device="cuda")
    mcnt = torch.full((R,), -9, dtype=torch.int32, device="cuda")
    mlist = torch.full((R, kk, 2), -9, dtype=torch.int32, device="cuda")
    sob_o, bos_o = np.full((R, NB), -1, np.int32), np.full((R, C), -1, np.int32)
    ck_o, cv_o = np.zeros((B, HKV, C, 64, D), np.uint16), np.zeros((B, HKV, C, 64, D), np.uint16)
    ws = N.workspace(shape)
    copy = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(7)
    scale = 1.0 / np.sqrt(D)
    ev_h = H.host(ev)
    for t in range(2):
        if t == 1:
            q = (q.float() + 0.3 * torch.randn(q.shape, generator=g, device="cuda")).to(torch.bfloat16)
        sel, agn = H.gpu_select(shape, q, kp, ev, ws)
        out = torch.full((B, HQ, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        N.nosa_offload_decode(shape, q, sel, sob, bos, table, mcnt, mlist, hk, hv, ck, cv, scale, out, ws,
                              copy=copy)
        torch.cuda.synchronize()
        sel_h, agn_h, q_h = H.host(sel), H.host(agn), H.host(q)
        tab_o, mc_o, ml_o = O.cache_step(sel_h, sob_o, bos_o)
        assert np.array_equal(H.host(sob), sob_o) and np.array_equal(H.host(bos), bos_o)
        assert np.array_equal(H.host(table), tab_o) and np.array_equal(H.host(mcnt), mc_o)
        ml = H.host(mlist)
        used = np.arange(kk)[None, :] < mc_o[:, None]
        assert np.array_equal(ml[used], ml_o[used])
        if t == 0:
            assert np.all(mc_o == kk)
        else:
            assert 0 < mc_o.sum() < R * kk
        O.gather(mc_o.reshape(B, HKV), ml_o.reshape(B, HKV, kk, 2), hk_h, ck_o)
        O.gather(mc_o.reshape(B, HKV), ml_o.reshape(B, HKV, kk, 2), hv_h, cv_o)
        assert np.array_equal(H.host(ck), ck_o) and np.array_equal(H.host(cv), cv_o)
        for r in ROWS:
            b, h = divmod(r, HKV)
            k_r = hk_h[b, h].reshape(1, 1, NB, 64, D)
            v_r = hv_h[b, h].reshape(1, 1, NB, 64, D)
            q_r = q_h[b:b + 1, h * G:(h + 1) * G]
            s_ref = O.block_scores(q_r, O.pool_keys(k_r, 32), NB, 2)
            H.check_selection(sel_h[r].reshape(1, 1, kk), agn_h[r].reshape(1, 1, KE), s_ref,
                              ev_h[r].reshape(1, 1, NB), KQ, KE)
            ref = O.attention(q_r, k_r, v_r, sel_h[r].reshape(1, 1, kk))
            H.check_attention(H.host(out[b:b + 1, h * G:(h + 1) * G]), ref, "bf16", "step %d row %d" % (t, r))


def test_append_into_stores_beyond_4gib():
    # The last sub-block of every row is written token by token through nosa_append_kv (32 calls);
    # odd sequences skip the final token, so their sub-block stays open.  On the sampled rows the
    # stores hold the appended tokens, and the pooled key of a closed sub-block equals the oracle's
    # mean over the updated store (an open one keeps its old value).
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = 2 * B * HKV * NB * 64 * D * 2 + (4 << 30)
    if free < need:
        pytest.skip("needs %.1f GiB of free device memory, %.1f GiB free" % (need / 2**30, free / 2**30))
    _, k, v, _ = _inputs(20261206)
    shape = N.make_shape(batch=B, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, n_blocks=NB, n_blocks_max=NB,
                         kq=KQ, ke=KE, sub_block_size=32, dtype=N.NOSA_BF16)
    kp = H.gpu_pool(shape, k)
    R = B * HKV
    kp_before = kp.clone()
    k_tail, v_tail = k[:, :, NB - 1, 63].clone(), v[:, :, NB - 1, 63].clone()
    g = torch.Generator(device="cuda").manual_seed(11)
    kn = torch.randn((32, B, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((32, B, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    acc = torch.full((R, D), float("nan"), dtype=torch.float32, device="cuda")
    for i in range(32):
        pos = torch.full((B,), NB * 64 - 32 + i, dtype=torch.int32, device="cuda")
        if i == 31:
            pos[1::2] = -1
        N.nosa_append_kv(shape, kn[i], vn[i], pos, k, v, acc, kp)
    torch.cuda.synchronize()
    kn_h, vn_h = H.host(kn), H.host(vn)
    for r in ROWS:
        b, h = divmod(r, HKV)
        k_r, v_r = H.host(k[b, h]), H.host(v[b, h])
        closed = b % 2 == 0
        n_new = 32 if closed else 31
        assert np.array_equal(k_r[NB - 1, 32:32 + n_new], kn_h[:n_new, b, h])
        assert np.array_equal(v_r[NB - 1, 32:32 + n_new], vn_h[:n_new, b, h])
        if not closed:
            assert np.array_equal(k_r[NB - 1, 63], H.host(k_tail[b, h]))
            assert np.array_equal(v_r[NB - 1, 63], H.host(v_tail[b, h]))
        kp_r = H.host(kp[r])
        assert np.array_equal(kp_r[:-1], H.host(kp_before[r])[:-1])          # earlier sub-blocks untouched
        if closed:
            ref = O.pool_keys(k_r.reshape(1, 1, NB, 64, D), 32)[0, 0, -1]
            np.testing.assert_allclose(kp_r[-1], ref, rtol=1e-6, atol=1e-6)
        else:
            assert np.array_equal(kp_r[-1], H.host(kp_before[r])[-1])
