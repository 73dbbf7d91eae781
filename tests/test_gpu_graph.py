"""HIP-graph capture of the offloaded decode step (append, select, offload decode, either with the
gather and the attention over the hits in one launch or with the gather forked onto a copy stream):
every replay is bit-identical to the same step run eagerly, with eager steps and synchronisations
interleaved between replays, across the steps where blocks arrive."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from block_sparse_kv_decode_amd.step_graph import OffloadStepGraphs  # noqa: E402
from nosa_inputs import f32_to_bf16_bits, generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

BS = 64


def _setup():
    w = small_workload("graph", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=6, n_blocks_max=9,
                       kq=2, ke=3, seed=43, cache_slots=8)
    x = generate(w)
    R, k, C, d, n0 = w.rows, w.k, w.cache_slots, w.head_dim, w.n_blocks
    prompt_k, prompt_v = x["k"].copy(), x["v"].copy()
    prompt_k[:, :, n0:] = 0
    prompt_v[:, :, n0:] = 0
    st = dict(host_k=H.pinned(prompt_k), host_v=H.pinned(prompt_v),
              pooled_k=torch.zeros((R, w.nbmax * 2, d), dtype=torch.float32, device="cuda"),
              pool_acc=torch.zeros((R, d), dtype=torch.float32, device="cuda"),
              evict=H.dev(x["evict"]), agn=torch.zeros((R, w.ke), dtype=torch.int32, device="cuda"),
              selected=torch.zeros((R, k), dtype=torch.int32, device="cuda"),
              slot_of_block=torch.full((R, w.nbmax), -1, dtype=torch.int32, device="cuda"),
              block_of_slot=torch.full((R, C), -1, dtype=torch.int32, device="cuda"),
              block_table=torch.zeros((R, k), dtype=torch.int32, device="cuda"),
              miss_cnt=torch.zeros((R,), dtype=torch.int32, device="cuda"),
              miss_list=torch.zeros((R, k, 2), dtype=torch.int32, device="cuda"),
              cache_k=torch.zeros((w.batch, w.n_kv_heads, C, BS, d), dtype=torch.bfloat16, device="cuda"),
              cache_v=torch.zeros((w.batch, w.n_kv_heads, C, BS, d), dtype=torch.bfloat16, device="cuda"),
              out=torch.zeros((w.batch, w.n_q_heads, d), dtype=torch.bfloat16, device="cuda"))
    shape0 = H.shape_of(w)
    st["ws"] = N.workspace(shape0)
    kfull = H.dev(x["k"])
    rng = np.random.default_rng(9)
    qs = [x["q"]]
    for _ in range(3 * BS):
        qs.append(f32_to_bf16_bits((H.as_f64(qs[-1]) + 0.3 * rng.standard_normal(x["q"].shape)).astype(np.float32)))
    return w, x, st, shape0, kfull, qs


def _reset(w, st, shape0, kfull):
    st["slot_of_block"].fill_(-1)
    st["block_of_slot"].fill_(-1)
    st["cache_k"].zero_()
    st["cache_v"].zero_()
    N.nosa_pool_keys(shape0, kfull, 0, w.n_blocks, st["pooled_k"])
    torch.cuda.synchronize()


def _run(w, x, st, g, qs, steps, mode):
    """mode(t) -> 'eager' | 'graph'.  Returns per-step copies of out, selected, table, miss_cnt."""
    n0 = w.n_blocks
    rec = []
    n_prev = 0
    for t in range(steps):
        n = (n0 * BS + t) // BS
        g.q.copy_(H.dev(qs[t]))
        append = t > 0
        if append:
            pos = n0 * BS + t - 1
            g.k_new.copy_(H.dev(np.ascontiguousarray(x["k"][:, :, pos // BS, pos % BS])))
            g.v_new.copy_(H.dev(np.ascontiguousarray(x["v"][:, :, pos // BS, pos % BS])))
            g.positions.fill_(pos)
        if mode(t) == "graph":
            g.replay(n, n_prev, append)
        else:
            g.enqueue(n, n_prev, append)
        torch.cuda.synchronize()
        rec.append({kk: st[kk].clone() for kk in ("out", "selected", "block_table", "miss_cnt", "agn")})
        n_prev = n
    return rec


@pytest.mark.parametrize("side_stream", [False, True])
def test_offload_step_graph_replays_match_eager(side_stream):
    w, x, st, shape0, kfull, qs = _setup()
    copy_stream = torch.cuda.Stream() if side_stream else None
    print("case side_stream", side_stream, flush=True)
    g = OffloadStepGraphs(shape0, st, copy_stream, 1.0 / np.sqrt(w.head_dim))
    steps = 2 * BS + 3           # blocks arrive at steps 64 and 128
    _reset(w, st, shape0, kfull)
    eager = _run(w, x, st, g, qs, steps, lambda t: "eager")
    _reset(w, st, shape0, kfull)
    mixed = _run(w, x, st, g, qs, steps, lambda t: "eager" if t % 7 == 3 else "graph")
    # one graph per (n_blocks, n_blocks_prev, append): the first step, then steady and arrival steps
    # at 6, 7 and 8 visible blocks
    assert sorted(g.graphs) == [(6, 0, False), (6, 6, True), (7, 6, True), (7, 7, True), (8, 7, True),
                                (8, 8, True)], sorted(g.graphs)
    for t in range(steps):
        for kk in eager[t]:
            a, b = eager[t][kk], mixed[t][kk]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), "step %d: %s differs between the graph replay and the eager step" % (t, kk)
    # and the replayed steps are right, not only repeatable: attention of the last step vs the oracle
    sel_h = H.host(mixed[-1]["selected"]).reshape(w.batch, w.n_kv_heads, w.k)
    ref = O.attention(qs[steps - 1], x["k"], x["v"], sel_h)
    H.check_attention(H.host(mixed[-1]["out"]), ref, "bf16", "graph last step")
