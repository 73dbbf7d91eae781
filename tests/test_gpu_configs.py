"""Full-size parity on the configured workloads, in the launch configuration the benchmark
times (automatic splits and parts): C2 (B16, 16K ctx), C3 (B64, 4K ctx), C5 (B4, 128K ctx) and the
sink + window split end to end against the oracle element by element, through the two calls and
through nosa_decode_step (the call the benchmark times), and the C4 offload loop (128 steps, decode
tokens appended through nosa_append_kv, the gather overlapped with attention by
nosa_offload_decode on a copy stream) with per-step invariants and oracle checks on sampled
steps."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import WORKLOADS, generate, visible_blocks  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402


@pytest.mark.parametrize("cfg", ["C2", "C3", "C5", "F1"])
def test_resident_config_end_to_end(cfg):
    w = WORKLOADS[cfg]
    print("case", cfg, flush=True)
    x = generate(w)
    shape = H.shape_of(w)
    q_dev, k_dev, v_dev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"])
    kp = H.gpu_pool(shape, k_dev)
    ws = N.workspace(shape)
    sel, agn = H.gpu_select(shape, q_dev, kp, H.dev(x["evict"]), ws)
    out = H.gpu_decode(shape, q_dev, k_dev, v_dev, w.nbmax, sel, ws)
    torch.cuda.synchronize()
    kp_ref = O.pool_keys(x["k"], 32)
    np.testing.assert_allclose(H.host(kp).reshape(kp_ref.shape), kp_ref, rtol=1e-6, atol=1e-6)
    s_ref = O.block_scores(x["q"], kp_ref, w.n_blocks, 2)
    ties = H.check_selection(H.host(sel), H.host(agn), s_ref, x["evict"], w.kq, w.ke, n_sink=w.n_sink,
                             n_window=w.n_window)
    sel_h = H.host(sel).reshape(w.batch, w.n_kv_heads, w.k)
    ref = O.attention(x["q"], x["k"], x["v"], sel_h)
    stats = H.check_attention(H.host(out), ref, w.dtype, cfg)
    print(cfg, "tie rows", ties, stats)
    # the same step again: bitwise identical
    sel2, _ = H.gpu_select(shape, q_dev, kp, H.dev(x["evict"]), ws)
    out2 = H.gpu_decode(shape, q_dev, k_dev, v_dev, w.nbmax, sel2, ws)
    assert torch.equal(sel, sel2) and torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("cfg", ["C2", "C3", "C5", "F1"])
def test_decode_step_at_the_timed_shapes(cfg):
    """nosa_decode_step, the call the benchmark times, in the benchmark's launch configuration
    (automatic splits and parts) on the full workload: bs16/16K and the sink + window split take the
    pick inside the attention launch (128 rows, two Gamma_e and two Gamma_q splits per row), bs64/4K
    the one-launch step with its 64-block rows, bs4/128K its long-row plan.  Its selection must be
    the oracle's (tie band) and bit-identical to nosa_select's, its output the oracle's attention
    over that selection elementwise, and a repeat bit-identical."""
    w = WORKLOADS[cfg]
    print("case", cfg, flush=True)
    x = generate(w)
    shape = H.shape_of(w)
    q_dev, k_dev, v_dev, ev_dev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.gpu_pool(shape, k_dev)
    ws = N.workspace(shape)
    scale = 1.0 / np.sqrt(w.head_dim)

    def step():
        agn = torch.full((w.rows, w.ke), -7, dtype=torch.int32, device="cuda")
        sel = torch.full((w.rows, w.k), -7, dtype=torch.int32, device="cuda")
        out = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), dtype=q_dev.dtype, device="cuda")
        N.nosa_decode_step(shape, q_dev, kp, ev_dev, 0, agn, sel, k_dev, v_dev, w.nbmax, scale, out, ws)
        return sel, agn, out

    sel, agn, out = step()
    sel_2c, agn_2c = H.gpu_select(shape, q_dev, kp, ev_dev, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_2c) and torch.equal(agn[:, :w.ke], agn_2c[:, :w.ke])
    s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], 32), w.n_blocks, 2)
    ties = H.check_selection(H.host(sel), H.host(agn), s_ref, x["evict"], w.kq, w.ke, n_sink=w.n_sink,
                             n_window=w.n_window)
    ref = O.attention(x["q"], x["k"], x["v"], H.host(sel).reshape(w.batch, w.n_kv_heads, w.k))
    stats = H.check_attention(H.host(out), ref, w.dtype, cfg + " step")
    print(cfg, "step: tie rows", ties, stats)
    sel2, agn2, out2 = step()
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2) and torch.equal(agn, agn2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("cfg", ["C4", "C4P", "C4S", "C4PS"])
def test_c4_offload_loop(cfg):
    """The 128-step offload loop: C4 (32 + 32, one token per step), C4P (the pages' 16 + 48 split with
    1 sink and a 16-block window), and the stress variants C4S / C4PS (one whole block arriving per
    step, so that the query-agnostic subset drops its lowest member or the arrival every step).
    Steps t = 0 mod 3 run nosa_offload_step as the benchmark times it (selection and offloaded decode in
    one call, no copy stream); steps t = 1 mod 3 run nosa_select + nosa_offload_decode without a copy
    stream (the gather and the attention over the hits in one launch), steps t = 2 mod 3 with the
    gather on a copy stream."""
    w = WORKLOADS[cfg]
    print("case", cfg, flush=True)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C = w.rows, w.k, w.cache_slots
    n0 = w.n_blocks
    append = w.blocks_per_step == 0
    if append:
        # The host pool and the pooled keys start with the prompt; the decode tokens join them
        # through nosa_append_kv, one per step.
        prompt_k, prompt_v = x["k"].copy(), x["v"].copy()
        prompt_k[:, :, n0:] = 0
        prompt_v[:, :, n0:] = 0
        hk, hv = H.pinned(prompt_k), H.pinned(prompt_v)
        del prompt_k, prompt_v
    else:
        # whole blocks arrive: the pool holds them beforehand, and visibility grows a block per step
        hk, hv = H.pinned(x["k"]), H.pinned(x["v"])
    hkd, hvd = N.host_map(hk), N.host_map(hv)
    kp = torch.full((R, w.nbmax * 2, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    N.nosa_pool_keys(shape0, H.dev(x["k"]), 0, n0 if append else w.nbmax, kp)
    acc = torch.zeros((R, w.head_dim), dtype=torch.float32, device="cuda")
    kn_all = H.dev(np.ascontiguousarray(x["k"][:, :, n0:].reshape(w.batch, w.n_kv_heads, -1, w.head_dim)
                                         .transpose(2, 0, 1, 3)))
    vn_all = H.dev(np.ascontiguousarray(x["v"][:, :, n0:].reshape(w.batch, w.n_kv_heads, -1, w.head_dim)
                                         .transpose(2, 0, 1, 3)))
    torch.cuda.synchronize()
    ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, w.head_dim), dtype=torch.bfloat16, device="cuda")
    cv = torch.zeros_like(ck)
    sob = torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda")
    bos = torch.full((R, C), -1, dtype=torch.int32, device="cuda")
    table = torch.empty((R, k), dtype=torch.int32, device="cuda")
    mcnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    mlist = torch.empty((R, k, 2), dtype=torch.int32, device="cuda")
    ws = N.workspace(shape0)
    ev_dev = H.dev(x["evict"])
    q_all = H.dev(x["q_steps"])
    copy_stream = torch.cuda.Stream()
    scale = 1.0 / np.sqrt(w.head_dim)
    kp_ref = None
    sampled = {0, 1, 63, 64, 65, w.steps - 1}
    agn = None
    prev_sel = None
    n_prev = 0
    gammas, hits = [], []
    for t in range(w.steps):
        n = visible_blocks(w, t)
        shape = shape0.copy(n_blocks=n)
        if t in sampled:
            torch.cuda.synchronize()
            snap = {"agn": None if agn is None else H.host(agn).copy(), "sob": H.host(sob).copy(),
                    "bos": H.host(bos).copy()}
        if append and t > 0:
            pos = w.n_tokens + t - 1
            N.nosa_append_kv(shape0, kn_all[t - 1], vn_all[t - 1],
                             torch.full((w.batch,), pos, dtype=torch.int32, device="cuda"), hkd, hvd, acc, kp)
        q_t = q_all[t]
        out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        if t % 3 == 0:
            if agn is None:
                agn = torch.full((R, w.ke), -7, dtype=torch.int32, device="cuda")
            sel = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
            N.nosa_offload_step(shape, q_t, kp, ev_dev, n_prev, agn, sel, sob, bos, table, mcnt, mlist, hkd, hvd, ck,
                                cv, scale, out, ws)
        else:
            sel, agn = H.gpu_select(shape, q_t, kp, ev_dev, ws, n_prev=n_prev, agn=agn)
            N.nosa_offload_decode(shape, q_t, sel, sob, bos, table, mcnt, mlist, hkd, hvd, ck, cv, scale, out, ws,
                                  copy=copy_stream if t % 3 == 2 else None)
        torch.cuda.synchronize()
        sel_h = H.host(sel)
        mc = H.host(mcnt)
        assert np.all(np.diff(sel_h, axis=1) > 0) and sel_h.min() >= 0 and sel_h.max() < n
        if prev_sel is not None:
            gam = O.locality(prev_sel, sel_h, w.nbmax)
            agn_h = H.host(agn)
            admitted = np.array([len(set(agn_h[r].tolist()) & set(range(n_prev, n))) for r in range(R)])
            # strict eviction: Gamma_e(t) within Gamma_e(t-1) and the arrivals, so the overlap bound
            for r in range(R):
                assert set(agn_h[r].tolist()) <= set(prev_agn[r].tolist()) | set(range(n_prev, n))
            assert np.all(gam >= (w.ke - admitted) / k - 1e-12)
            # cache = budget: the cache after step t-1 holds exactly Gamma(t-1), so hits = k * gamma
            assert np.array_equal(k - mc, np.rint(k * gam).astype(np.int32))
            gammas.append(gam)
        hits.append(k - mc)
        if t in sampled:
            if kp_ref is None:
                kp_ref = O.pool_keys(x["k"], 32)
            s_ref = O.block_scores(x["q_steps"][t], kp_ref[:, :, :2 * n], n, 2)
            H.check_selection(sel_h, H.host(agn), s_ref, x["evict"], w.kq, w.ke, n_prev,
                              None if snap["agn"] is None else snap["agn"].reshape(w.batch, w.n_kv_heads, w.ke),
                              n_sink=w.n_sink, n_window=w.n_window)
            sob_ref, bos_ref = snap["sob"], snap["bos"]
            tab_ref, mc_ref, ml_ref = O.cache_step(sel_h, sob_ref, bos_ref)
            assert np.array_equal(H.host(sob), sob_ref) and np.array_equal(H.host(bos), bos_ref)
            assert np.array_equal(H.host(table), tab_ref) and np.array_equal(mc, mc_ref)
            ref = O.attention(x["q_steps"][t], x["k"], x["v"], sel_h.reshape(w.batch, w.n_kv_heads, k))
            H.check_attention(H.host(out), ref, "bf16", "C4 step %d" % t)
            # every cache slot holds the bytes of the block the map says it holds
            ckh, cvh, bosh = H.host(ck), H.host(cv), H.host(bos)
            for r in range(0, R, 17):
                b, g = divmod(r, w.n_kv_heads)
                for s_, blk in enumerate(bosh[r]):
                    if blk >= 0:
                        assert np.array_equal(ckh[b, g, s_], x["k"][b, g, blk])
                        assert np.array_equal(cvh[b, g, s_], x["v"][b, g, blk])
        prev_sel = sel_h
        prev_agn = H.host(agn).copy()
        n_prev = n
        if t % 32 == 0:
            print("C4 step %d ok" % t, flush=True)
    if append:
        # pooled keys built by the appends: bit-identical to pooling the full store at once
        torch.cuda.synchronize()
        n_end = visible_blocks(w, w.steps - 1)
        kp_once = H.gpu_pool(shape0, H.dev(x["k"]))
        assert torch.equal(kp[:, :2 * n_end].view(torch.int32), kp_once[:, :2 * n_end].view(torch.int32))
    g = np.concatenate(gammas)
    print("%s gamma min %.3f mean %.3f; hit rate (warm) %.3f" % (cfg, g.min(), g.mean(), np.mean(hits[1:]) / k))
    # at most one block arrives per step in every variant, so locality never drops below (ke - 1) / k
    assert g.min() >= (w.ke - 1) / k - 1e-12
