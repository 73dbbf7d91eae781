"""Parity of the one-call offloaded step (nosa_offload_step) with nosa_select + nosa_offload_decode
run on a second copy of the state, over several decode steps with query drift and arriving blocks:
the query-agnostic state, the selection, both slot maps, the block table, the miss list, the cache
bytes and the output are identical bit for bit (the same kernels attend the same blocks in the same
order; only the cache map moves into the end of the Gamma_q pick when the rows are scored in parts),
and the selection and attention match the oracle."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import f32_to_bf16_bits, generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

CASES = {
    # rows scored in parts (more than 64 KiB of pooled keys per row, fewer than 256 rows): the map
    # runs at the end of the Gamma_q pick
    "parts_bf16": (dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, n_blocks_max=156, kq=12, ke=10,
                        cache_slots=30, seed=91), False),
    "parts_bf16_side_stream": (dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, n_blocks_max=156,
                                    kq=12, ke=10, cache_slots=30, seed=92), True),
    "parts_f32_d64_g8": (dict(batch=1, n_q_heads=16, n_kv_heads=2, head_dim=64, n_blocks=140, n_blocks_max=146, kq=7,
                              ke=9, cache_slots=16, dtype="f32", seed=93), False),
    "parts_sink_window_kq64": (dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, n_blocks=300, n_blocks_max=306,
                                    kq=64, ke=40, n_sink=1, n_window=8, cache_slots=120, seed=94), False),
    "parts_kq0": (dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=150, n_blocks_max=156, kq=0, ke=12,
                       cache_slots=12, seed=95), False),
    # short rows: one workgroup per row scores and selects, then the map kernel as usual
    "one_workgroup_rows": (dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=40, n_blocks_max=46, kq=6,
                                ke=6, cache_slots=15, seed=96), False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_offload_step_matches_select_then_offload_decode(name):
    kw, side_stream = CASES[name]
    w = small_workload(name, **kw)
    print("case", name, kw, "side stream", side_stream, flush=True)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C, d = w.rows, w.k, w.cache_slots, w.head_dim
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    hk, hv = H.pinned(x["k"]), H.pinned(x["v"])
    hkd, hvd = N.host_map(hk), N.host_map(hv)

    def state():
        ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, d), dtype=tdt, device="cuda")
        return dict(ck=ck, cv=torch.zeros_like(ck),
                    sob=torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda"),
                    bos=torch.full((R, C), -1, dtype=torch.int32, device="cuda"),
                    table=torch.full((R, k), -9, dtype=torch.int32, device="cuda"),
                    mcnt=torch.full((R,), -9, dtype=torch.int32, device="cuda"),
                    mlist=torch.full((R, k, 2), -9, dtype=torch.int32, device="cuda"),
                    agn=torch.full((R, max(w.ke, 1)), -9, dtype=torch.int32, device="cuda"),
                    sel=torch.full((R, k), -9, dtype=torch.int32, device="cuda"),
                    out=torch.full((w.batch, w.n_q_heads, d), float("nan"), dtype=tdt, device="cuda"),
                    ws=N.workspace(shape0))
    A, B = state(), state()
    kp = H.gpu_pool(shape0, H.dev(x["k"]))
    kp_ref = O.pool_keys(x["k"], 32)
    ev = H.dev(x["evict"])
    copy_stream = torch.cuda.Stream() if side_stream else None
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(17)
    qf = x["q"]
    n, agn_ref = w.n_blocks, None
    for t in range(6):
        n_prev = 0 if t == 0 else n
        if t in (2, 4):
            n += 2
        shape = shape0.copy(n_blocks=n)
        q = H.dev(qf)
        N.nosa_select(shape, q, kp, ev, n_prev, A["agn"], A["sel"], A["ws"])
        N.nosa_offload_decode(shape, q, A["sel"], A["sob"], A["bos"], A["table"], A["mcnt"], A["mlist"], hkd, hvd,
                              A["ck"], A["cv"], scale, A["out"], A["ws"], copy=copy_stream)
        N.nosa_offload_step(shape, q, kp, ev, n_prev, B["agn"], B["sel"], B["sob"], B["bos"], B["table"], B["mcnt"],
                            B["mlist"], hkd, hvd, B["ck"], B["cv"], scale, B["out"], B["ws"], copy=copy_stream)
        torch.cuda.synchronize()
        for key in ("agn", "sel", "sob", "bos", "table", "mcnt", "ck", "cv", "out"):
            a, b = A[key], B[key]
            if a.dtype in (torch.bfloat16, torch.float32):
                a, b = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32), \
                    b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
            assert torch.equal(a, b), (name, t, key)
        mc = H.host(A["mcnt"])
        mla, mlb = H.host(A["mlist"]), H.host(B["mlist"])
        for r in range(R):
            assert np.array_equal(mla[r, :mc[r]], mlb[r, :mc[r]]), (name, t, r)
        if t == 0:
            assert np.all(mc == k)            # cold cache: every entry misses
        sel_h = H.host(B["sel"])
        s_ref = O.block_scores(qf, kp_ref[:, :, :2 * n], n, 2)
        H.check_selection(sel_h, H.host(B["agn"])[:, :w.ke], s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref,
                          n_sink=w.n_sink, n_window=w.n_window)
        _, agn_ref, _ = O.select(s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref, w.n_sink, w.n_window)
        ref = O.attention(qf, x["k"], x["v"], sel_h.reshape(w.batch, w.n_kv_heads, k), scale)
        H.check_attention(H.host(B["out"]), ref, w.dtype, "%s step %d" % (name, t))
        if w.dtype == "bf16":
            qf = f32_to_bf16_bits((H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32))
        else:
            qf = (qf + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32)
