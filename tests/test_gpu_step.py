"""Parity of the one-call decode step (nosa_decode_step) with the oracle and with nosa_select +
nosa_sparse_decode: the fused path (Gamma_q ranked inside the attention launch) on row shapes that
take it, with sink / window blocks and with arrivals across steps; the one-workgroup-per-row step
on shapes with enough rows for a single split each; and the two calls on shapes that take neither
(fp32, one subset empty, short rows, long rows)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import f32_to_bf16_bits, generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

CASES = {
    # fused: fewer than 256 rows, rows above 64 KiB of pooled keys, bf16, kq and ke > 0
    "fused_g4": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, n_blocks_max=160, kq=20,
                     ke=12, seed=51),
    "fused_g8_ragged": dict(batch=3, n_q_heads=8, n_kv_heads=1, head_dim=128, n_blocks=301, kq=37, ke=29, seed=52),
    "fused_d64_g2": dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, n_blocks=500, kq=40, ke=24, seed=53),
    # rows of 513 to 2048 blocks with both subsets of at most 64 blocks: Gamma_q ranked from registers
    "fused_regs_700": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=700, kq=20, ke=20,
                           seed=62),
    "fused_regs_2048_kq64": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=2048, kq=64, ke=64,
                                 seed=72),
    "fused_regs_1500_sink_window": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=1500,
                                        n_blocks_max=1600, kq=23, ke=41, n_sink=2, n_window=7, seed=73),
    "fused_regs_140_d64": dict(batch=2, n_q_heads=8, n_kv_heads=1, head_dim=64, n_blocks=140, kq=5, ke=3, seed=74),
    "fused_regs_100_g8": dict(batch=2, n_q_heads=8, n_kv_heads=1, head_dim=128, n_blocks=100, kq=6, ke=9, seed=76),
    # longer rows, or a subset above 64 blocks: the two calls
    "fallback_long_rows": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=2100, kq=20, ke=20,
                               seed=62),
    "fallback_kq_above_64": dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=700, kq=65, ke=20,
                                 seed=75),
    "fused_sink_window": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=200, kq=16, ke=48,
                              n_sink=1, n_window=16, seed=54),
    # fallback: fp32, an empty subset, short rows, many rows
    "fallback_f32": dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, n_blocks=300, kq=8, ke=8, dtype="f32",
                         seed=55),
    "fallback_kq0": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, kq=0, ke=24, seed=56),
    "fallback_ke0": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, kq=24, ke=0, seed=57),
    "fallback_short": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=40, kq=6, ke=6, seed=58),
    # one workgroup per row scores, selects and attends (256 rows or more, single split): GQA
    # groups 1 to 8, d 64 and 128, ragged budgets, an empty subset, sink / window blocks, long rows
    "rowstep_many_rows": dict(batch=64, n_q_heads=8, n_kv_heads=4, head_dim=128, n_blocks=20, kq=4, ke=4, seed=59),
    "rowstep_g8_ragged": dict(batch=128, n_q_heads=16, n_kv_heads=2, head_dim=128, n_blocks=77, kq=9, ke=5,
                              seed=63),
    "rowstep_g1_d64": dict(batch=64, n_q_heads=4, n_kv_heads=4, head_dim=64, n_blocks=50, kq=7, ke=6, seed=64),
    "rowstep_sink_window": dict(batch=64, n_q_heads=8, n_kv_heads=4, head_dim=64, n_blocks=100, kq=5, ke=10,
                                n_sink=1, n_window=4, seed=65),
    "rowstep_kq0": dict(batch=64, n_q_heads=16, n_kv_heads=4, head_dim=128, n_blocks=30, kq=0, ke=8, seed=66),
    "rowstep_ke0": dict(batch=64, n_q_heads=16, n_kv_heads=4, head_dim=128, n_blocks=30, kq=8, ke=0, seed=67),
    "rowstep_long_rows": dict(batch=32, n_q_heads=16, n_kv_heads=8, head_dim=128, n_blocks=1500, kq=8, ke=7,
                              seed=68),
    # 512 rows keep a single split with a 70-block budget: the attention walks more than one
    # 64-entry window of block ids
    "rowstep_wide_budget": dict(batch=128, n_q_heads=16, n_kv_heads=4, head_dim=64, n_blocks=80, kq=40, ke=30,
                                seed=70),
}


def _two_calls(shape, q, kp, ev, n_prev, agn_in, k, v, nbmax, ws):
    agn = agn_in.clone()
    R = shape.batch * shape.n_kv_heads
    sel = torch.full((R, shape.kq + shape.ke), -7, dtype=torch.int32, device="cuda")
    N.nosa_select(shape, q, kp, ev, n_prev, agn, sel, ws)
    out = H.gpu_decode(shape, q, k, v, nbmax, sel, ws)
    return sel, agn, out


def _step(shape, q, kp, ev, n_prev, agn_in, k, v, nbmax, ws):
    agn = agn_in.clone()
    R = shape.batch * shape.n_kv_heads
    sel = torch.full((R, shape.kq + shape.ke), -7, dtype=torch.int32, device="cuda")
    out = torch.full((shape.batch, shape.n_q_heads, shape.head_dim), float("nan"), dtype=q.dtype, device="cuda")
    N.nosa_decode_step(shape, q, kp, ev, n_prev, agn, sel, k, v, nbmax, 1.0 / np.sqrt(shape.head_dim), out, ws)
    return sel, agn, out


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_step_matches_two_calls_and_oracle(name):
    w = small_workload(name, **CASES[name])
    ns, nw = w.n_sink, w.n_window
    x = generate(w)
    shape = H.shape_of(w)
    q, k, v, ev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.gpu_pool(shape, k)
    ws = N.workspace(shape)
    R = w.rows
    agn0 = torch.full((R, max(w.ke, 1)), -7, dtype=torch.int32, device="cuda")
    sel_a, agn_a, out_a = _two_calls(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    sel_b, agn_b, out_b = _step(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(agn_a[:, :w.ke], agn_b[:, :w.ke])
    kp_ref = O.pool_keys(x["k"], 32)
    s_ref = O.block_scores(x["q"], kp_ref, w.n_blocks, 2)
    H.check_selection(H.host(sel_b), H.host(agn_b), s_ref, x["evict"], w.kq, w.ke, n_sink=ns, n_window=nw)
    ref = O.attention(x["q"], x["k"], x["v"], H.host(sel_b).reshape(w.batch, w.n_kv_heads, w.k))
    print(name, H.check_attention(H.host(out_b), ref, w.dtype, name + " (one call)"))
    H.check_attention(H.host(out_a), ref, w.dtype, name + " (two calls)")
    # repeatable bit for bit
    sel_c, _, out_c = _step(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel_b, sel_c)
    assert torch.equal(out_b.view(torch.int16) if out_b.dtype == torch.bfloat16 else out_b,
                       out_c.view(torch.int16) if out_c.dtype == torch.bfloat16 else out_c)


@pytest.mark.parametrize("kq", [32, 64])
def test_decode_step_clustered_scores(kq):
    """Block scores rising with the block id, from crafted pooled keys: the best blocks crowd into the
    last chunks, so the chunk-maximum bound lets nearly every block of the kq best 16-block chunks
    through (2048 blocks per row).  That is about 500 candidates for kq = 32, which the register
    ranking keeps, and about 1000 for kq = 64, more than its candidate buffer holds, so the LDS
    ranking takes over.  Both must give the oracle's selection exactly (the scores are distinct and
    computed identically on both sides) and the two calls' results."""
    w = small_workload("clustered_%d" % kq, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=2048,
                       kq=kq, ke=32, seed=71)
    x = generate(w)
    B, Hkv, d, n = w.batch, w.n_kv_heads, w.head_dim, w.n_blocks
    G = w.n_q_heads // Hkv
    print("case clustered kq", kq, flush=True)
    # every sub-block of block b pools to (b + 1) * sign(qs_0) * e_0, qs the row's summed query heads,
    # so that the block score is (b + 1) * |qs_0|
    qs0 = H.as_f64(x["q"]).reshape(B, Hkv, G, d)[..., 0].sum(axis=-1)
    kp_host = np.zeros((B, Hkv, 2 * n, d), dtype=np.float32)
    kp_host[..., 0] = (np.repeat(np.arange(1, n + 1, dtype=np.float32), 2)[None, None, :] *
                       np.sign(qs0).astype(np.float32)[..., None])
    shape = H.shape_of(w)
    q, k, v, ev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.dev(kp_host.reshape(B * Hkv, 2 * n, d))
    ws = N.workspace(shape)
    agn0 = torch.full((w.rows, w.ke), -7, dtype=torch.int32, device="cuda")
    sel_a, agn_a, out_a = _two_calls(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    sel_b, agn_b, out_b = _step(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(agn_a, agn_b)
    s_ref = O.block_scores(x["q"], kp_host, n, 2)
    assert H.check_selection(H.host(sel_b), H.host(agn_b), s_ref, x["evict"], w.kq, w.ke) == 0
    # the query-aware part is the kq highest block ids outside Gamma_e
    sel_h, agn_h = H.host(sel_b).reshape(B, Hkv, -1), H.host(agn_b).reshape(B, Hkv, -1)
    for b in range(B):
        for g in range(Hkv):
            rest = [i for i in range(n - 1, -1, -1) if i not in set(agn_h[b, g].tolist())][:kq]
            assert sorted(set(sel_h[b, g].tolist()) - set(agn_h[b, g].tolist())) == sorted(rest)
    ref = O.attention(x["q"], x["k"], x["v"], sel_h)
    print("clustered kq", kq, H.check_attention(H.host(out_b), ref, w.dtype, "clustered (one call)"))
    sel_c, _, out_c = _step(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel_b, sel_c) and torch.equal(out_b.view(torch.int16), out_c.view(torch.int16))


MULTI = {
    "fused": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, kq=14, ke=18, seed=60),
    "rowstep": dict(batch=64, n_q_heads=16, n_kv_heads=4, head_dim=128, kq=6, ke=9, seed=69),
}


@pytest.mark.parametrize("plan", sorted(MULTI))
def test_decode_step_multistep_with_arrivals(plan):
    # Strict eviction across steps through the one-call step: Gamma_e follows the oracle exactly,
    # selections within the tie band, attention within tolerance, at every step.
    w = small_workload("step_multi_" + plan, n_blocks=120, n_blocks_max=140, **MULTI[plan])
    x = generate(w)
    shape0 = H.shape_of(w)
    k, v, ev = H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.gpu_pool(shape0, k)
    ws = N.workspace(shape0)
    kp_ref = O.pool_keys(x["k"], 32)
    rng = np.random.default_rng(61)
    qf = x["q"]
    n, agn, agn_ref = 120, torch.zeros((w.rows, w.ke), dtype=torch.int32, device="cuda"), None
    for t in range(8):
        n_prev = 0 if t == 0 else n
        if t in (2, 3, 6):
            n += 3
        shape = shape0.copy(n_blocks=n)
        sel, agn_new, out = _step(shape, H.dev(qf), kp, ev, n_prev, agn, k, v, w.nbmax, ws)
        torch.cuda.synchronize()
        s_ref = O.block_scores(qf, kp_ref[:, :, :2 * n], n, 2)
        H.check_selection(H.host(sel), H.host(agn_new), s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref)
        ref = O.attention(qf, x["k"], x["v"], H.host(sel).reshape(w.batch, w.n_kv_heads, w.k))
        H.check_attention(H.host(out), ref, "bf16", "step %d" % t)
        _, agn_ref, _ = O.select(s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref)
        agn = agn_new
        qf = f32_to_bf16_bits((H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32))


EVERY_BLOCK = {
    # one workgroup per row (512 rows, one split), the pick inside attention (rows above 64 KiB of
    # pooled keys), and the two calls (short rows)
    "rowstep": dict(batch=128, n_q_heads=16, n_kv_heads=4, head_dim=64, n_blocks=12, kq=5, ke=7, seed=71),
    "fused": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, kq=90, ke=60, seed=72),
    "two_calls": dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=30, kq=10, ke=20, seed=73),
}


@pytest.mark.parametrize("plan", sorted(EVERY_BLOCK))
def test_decode_step_selects_every_block(plan):
    # A budget equal to the visible blocks selects all of them: the selection is 0..n-1 in every row,
    # and sparse attention is dense decode attention over the whole context.
    w = small_workload("every_" + plan, **EVERY_BLOCK[plan])
    assert w.k == w.n_blocks
    x = generate(w)
    shape = H.shape_of(w)
    q, k, v, ev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.gpu_pool(shape, k)
    ws = N.workspace(shape)
    agn0 = torch.full((w.rows, w.ke), -7, dtype=torch.int32, device="cuda")
    sel, agn, out = _step(shape, q, kp, ev, 0, agn0, k, v, w.nbmax, ws)
    assert (H.host(sel) == np.arange(w.n_blocks, dtype=np.int32)).all()
    s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], 32), w.n_blocks, 2)
    H.check_selection(H.host(sel), H.host(agn), s_ref, x["evict"], w.kq, w.ke)
    every = np.broadcast_to(np.arange(w.n_blocks, dtype=np.int32), (w.batch, w.n_kv_heads, w.n_blocks)).copy()
    ref = O.attention(x["q"], x["k"], x["v"], every)
    H.check_attention(H.host(out), ref, "bf16", "every block (%s)" % plan)
