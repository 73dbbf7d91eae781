"""A seeded sweep of random shapes through nosa_decode_step, so that every plan it can take runs
against the oracle and against nosa_select + nosa_sparse_decode:
  * the one-workgroup-per-row step (256 rows or more, one split per row), with and without the
    prefetch of the first two Gamma_e blocks;
  * the pick inside the attention launch (long rows, few rows);
  * the two calls (everything else).
Shapes vary over GQA groups 1 to 8, d 64 and 128, ragged budgets, empty query-aware or
query-agnostic subsets, and sink / window blocks; a second set covers rows of 513 to 2048 blocks
with both subsets of at most 64 blocks (the pick ranked from registers). Each case runs a second
step in which three blocks arrive under strict eviction."""

import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

# NOSA_SWEEP_CASES / NOSA_SWEEP_SEED widen the sweep (default: 48 cases, seed 20261203)
N_CASES = int(os.environ.get("NOSA_SWEEP_CASES", "48"))


def _cases():
    rng = np.random.default_rng(int(os.environ.get("NOSA_SWEEP_SEED", "20261203")))
    out = []
    for i in range(N_CASES):
        G = int(rng.choice([1, 2, 4, 8]))
        many = i % 3 == 0                       # 256 or 512 rows: one workgroup per row selects
        if many:
            hkv = int(rng.choice([2, 4]))
            batch = (512 if i % 6 == 0 else 256) // hkv   # 512 rows: one split each, so one launch
            n = int(rng.integers(12, 48))
            d = 64 if rng.random() < 0.6 else 128
        else:
            hkv = int(rng.choice([1, 2]))
            batch = int(rng.integers(1, 4))
            n = int(rng.integers(20, 600))
            d = int(rng.choice([64, 128]))
        k = int(rng.integers(2, min(n, 80) + 1))
        ke = int(rng.integers(0, k + 1))
        kq = k - ke
        ns = nw = 0
        if ke >= 3 and rng.random() < 0.4:
            ns = int(rng.integers(0, 2))
            nw = int(rng.integers(0, (ke - ns) // 2 + 1))
        out.append(dict(batch=batch, n_q_heads=hkv * G, n_kv_heads=hkv, head_dim=d, n_blocks=n, n_blocks_max=n + 5,
                        kq=kq, ke=ke, n_sink=ns, n_window=nw, seed=1000 + i))
    return out


CASES = _cases()


def _long_cases():
    # few rows of 513 to 2045 blocks with both subsets of at most 64 blocks: the query-aware pick
    # runs from registers inside the attention launch (the second step adds 3 blocks, still <= 2048)
    rng = np.random.default_rng(int(os.environ.get("NOSA_SWEEP_SEED", "20261203")) + 1)
    out = []
    for i in range(N_LONG):
        G = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2]))
        n = int(rng.integers(513, 2046))
        ke = int(rng.integers(1, 65))
        kq = int(rng.integers(1, 65))
        ns = nw = 0
        if ke >= 3 and rng.random() < 0.4:
            ns = int(rng.integers(0, 2))
            nw = int(rng.integers(0, (ke - ns) // 2 + 1))
        out.append(dict(batch=int(rng.integers(1, 3)), n_q_heads=hkv * G, n_kv_heads=hkv,
                        head_dim=int(rng.choice([64, 128])), n_blocks=n, n_blocks_max=n + 3, kq=kq, ke=ke,
                        n_sink=ns, n_window=nw, seed=2000 + i))
    return out


N_LONG = int(os.environ.get("NOSA_SWEEP_LONG_CASES", "12"))
LONG_CASES = _long_cases()


def _run(shape, q, kp, ev, n_prev, agn_in, k, v, nbmax, ws, one_call):
    R = shape.batch * shape.n_kv_heads
    agn = agn_in.clone()
    sel = torch.full((R, shape.kq + shape.ke), -7, dtype=torch.int32, device="cuda")
    if one_call:
        out = torch.full((shape.batch, shape.n_q_heads, shape.head_dim), float("nan"), dtype=q.dtype, device="cuda")
        N.nosa_decode_step(shape, q, kp, ev, n_prev, agn, sel, k, v, nbmax, 1.0 / np.sqrt(shape.head_dim), out, ws)
    else:
        N.nosa_select(shape, q, kp, ev, n_prev, agn, sel, ws)
        out = H.gpu_decode(shape, q, k, v, nbmax, sel, ws)
    torch.cuda.synchronize()
    return sel, agn, out


@pytest.mark.parametrize("case", range(N_CASES))
def test_decode_step_random_shapes(case):
    _sweep_case(CASES[case], "sweep%d" % case)


@pytest.mark.parametrize("case", range(N_LONG))
def test_decode_step_random_long_rows(case):
    _sweep_case(LONG_CASES[case], "long%d" % case)


def _sweep_case(c, label):
    print("case", label, c, flush=True)
    w = small_workload(label, **c)
    x = generate(w)
    shape0 = H.shape_of(w)
    q, k, v, ev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.gpu_pool(shape0, k)
    ws = N.workspace(shape0)
    kp_ref = O.pool_keys(x["k"], 32)
    R, ns, nw = w.rows, w.n_sink, w.n_window
    agn0 = torch.full((R, max(w.ke, 1)), -7, dtype=torch.int32, device="cuda")
    n = c["n_blocks"]
    agn_ref = None
    for step, (n_prev, n_now) in enumerate(((0, n), (n, n + 3))):
        shape = shape0.copy(n_blocks=n_now)
        sel_a, agn_a, out_a = _run(shape, q, kp, ev, n_prev, agn0, k, v, w.nbmax, ws, one_call=False)
        sel_b, agn_b, out_b = _run(shape, q, kp, ev, n_prev, agn0, k, v, w.nbmax, ws, one_call=True)
        assert torch.equal(sel_a, sel_b), "step %d: the two calls and the one-call step select differently" % step
        assert torch.equal(agn_a[:, :w.ke], agn_b[:, :w.ke])
        s_ref = O.block_scores(x["q"], kp_ref[:, :, :2 * n_now], n_now, 2)
        H.check_selection(H.host(sel_b), H.host(agn_b), s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref, n_sink=ns,
                          n_window=nw)
        ref = O.attention(x["q"], x["k"], x["v"], H.host(sel_b).reshape(w.batch, w.n_kv_heads, w.k))
        H.check_attention(H.host(out_b), ref, w.dtype, "%s step %d (one call)" % (label, step))
        H.check_attention(H.host(out_a), ref, w.dtype, "%s step %d (two calls)" % (label, step))
        _, agn_ref, _ = O.select(s_ref, x["evict"], w.kq, w.ke, n_prev, agn_ref, ns, nw)
        agn0 = agn_b
