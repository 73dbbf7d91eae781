"""A seeded sweep of random shapes through the offloaded step, nosa_select + nosa_offload_decode and
nosa_offload_step on alternate steps: cache size, GQA group, head dim, dtype, budget split and the
copy stream vary.  Over five steps with query drift
and arriving blocks, the GPU's slot maps, block table, miss list and cache bytes must equal the
oracle's cache simulation exactly, and attention over the cache must match the oracle's attention
over the selected blocks."""

import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import f32_to_bf16_bits, generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

# NOSA_SWEEP_CASES / NOSA_SWEEP_SEED widen the sweep (default: 16 cases, seed 31415)
N_CASES = int(os.environ.get("NOSA_SWEEP_CASES", "16"))
STEPS = 5


def _cases():
    rng = np.random.default_rng(int(os.environ.get("NOSA_SWEEP_SEED", "31415")))
    out = []
    for i in range(N_CASES):
        G = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        n = int(rng.integers(20, 300))
        k = int(rng.integers(2, min(n, 48) + 1))
        ke = int(rng.integers(0, k + 1))
        out.append(dict(batch=int(rng.integers(1, 4)), n_q_heads=hkv * G, n_kv_heads=hkv,
                        head_dim=int(rng.choice([64, 128])), n_blocks=n, n_blocks_max=n + STEPS, kq=k - ke, ke=ke,
                        cache_slots=k + int(rng.integers(0, 21)), dtype="f32" if rng.random() < 0.25 else "bf16",
                        seed=2000 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", range(N_CASES))
def test_offload_decode_random_shapes(case):
    c = CASES[case]
    side_stream = case % 2 == 1
    print("case", case, c, "side stream", side_stream)
    w = small_workload("offload_sweep%d" % case, **c)
    x = generate(w)
    shape0 = H.shape_of(w)
    R, k, C, d = w.rows, w.k, w.cache_slots, w.head_dim
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    hk, hv = H.pinned(x["k"]), H.pinned(x["v"])
    ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, d), dtype=tdt, device="cuda")
    cv = torch.zeros_like(ck)
    sob = torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda")
    bos = torch.full((R, C), -1, dtype=torch.int32, device="cuda")
    table = torch.full((R, k), -9, dtype=torch.int32, device="cuda")
    mcnt = torch.full((R,), -9, dtype=torch.int32, device="cuda")
    mlist = torch.full((R, k, 2), -9, dtype=torch.int32, device="cuda")
    sob_ref = np.full((R, w.nbmax), -1, np.int32)
    bos_ref = np.full((R, C), -1, np.int32)
    ck_ref = np.zeros(tuple(ck.shape), x["k"].dtype)
    cv_ref = np.zeros_like(ck_ref)
    kp = H.gpu_pool(shape0, H.dev(x["k"]))
    ws = N.workspace(shape0)
    ev = H.dev(x["evict"])
    copy_stream = torch.cuda.Stream() if side_stream else None
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(case)
    qf = x["q"]
    n, agn = c["n_blocks"], None
    for t in range(STEPS):
        n_prev = 0 if t == 0 else n
        if t in (1, 3):
            n += 1 + t // 2
        shape = shape0.copy(n_blocks=n)
        q_dev = H.dev(qf)
        out = torch.full((w.batch, w.n_q_heads, d), float("nan"), dtype=tdt, device="cuda")
        if (case + t) % 2 == 0:
            # selection and offloaded decode in one call (the cache map inside the pick on rows scored
            # in parts)
            if agn is None:
                agn = torch.full((R, max(w.ke, 1)), -7, dtype=torch.int32, device="cuda")
            sel = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
            N.nosa_offload_step(shape, q_dev, kp, ev, n_prev, agn, sel, sob, bos, table, mcnt, mlist, hk, hv, ck, cv,
                                scale, out, ws, copy=copy_stream)
        else:
            sel, agn = H.gpu_select(shape, q_dev, kp, ev, ws, n_prev=n_prev, agn=agn)
            N.nosa_offload_decode(shape, q_dev, sel, sob, bos, table, mcnt, mlist, hk, hv, ck, cv, scale, out, ws,
                                  copy=copy_stream)
        torch.cuda.synchronize()
        sel_h = H.host(sel)
        tab_ref, mc_ref, ml_ref = O.cache_step(sel_h, sob_ref, bos_ref)
        assert np.array_equal(H.host(sob), sob_ref) and np.array_equal(H.host(bos), bos_ref), t
        assert np.array_equal(H.host(table), tab_ref) and np.array_equal(H.host(mcnt), mc_ref), t
        ml = H.host(mlist)
        for r in range(R):
            assert np.array_equal(ml[r, :mc_ref[r]], ml_ref[r, :mc_ref[r]]), (t, r)
        O.gather(mc_ref.reshape(w.batch, w.n_kv_heads), ml_ref.reshape(w.batch, w.n_kv_heads, k, 2), x["k"], ck_ref)
        O.gather(mc_ref.reshape(w.batch, w.n_kv_heads), ml_ref.reshape(w.batch, w.n_kv_heads, k, 2), x["v"], cv_ref)
        assert np.array_equal(H.host(ck).view(ck_ref.dtype), ck_ref), t
        assert np.array_equal(H.host(cv).view(cv_ref.dtype), cv_ref), t
        if t == 0:
            assert np.all(mc_ref == k)        # cold cache: every entry misses
        ref = O.attention(qf, x["k"], x["v"], sel_h.reshape(w.batch, w.n_kv_heads, k), scale)
        H.check_attention(H.host(out), ref, w.dtype, "case %d step %d" % (case, t))
        if w.dtype == "bf16":
            qf = f32_to_bf16_bits((H.as_f64(qf) + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32))
        else:
            qf = (qf + 0.3 * rng.standard_normal(qf.shape)).astype(np.float32)
