"""nosa_decode_step_noalloc (the step with the library's fixed per-GPU scratch as its workspace)
against nosa_decode_step with a caller workspace: two calls in a row on one GPU, the second on a
smaller input, each bit-identical to the workspace call (same kernels, same plan) and matching the
oracle (selection within the tie band, attention elementwise)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_sparse_kv_decode_amd as N  # noqa: E402
from nosa_inputs import generate, small_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpuhelp as H  # noqa: E402

CALLS = [
    # rows scored in parts, with the query-aware pick inside the attention launch
    small_workload("noalloc_big", batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, n_blocks=256, kq=32, ke=32,
                   seed=61),
    # then a smaller input on the same scratch: fewer rows, shorter rows, a smaller budget
    small_workload("noalloc_small", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_blocks=100, kq=8, ke=8,
                   seed=62),
]


def _run(w, x, noalloc):
    shape = H.shape_of(w)
    q, k, v, ev = H.dev(x["q"]), H.dev(x["k"]), H.dev(x["v"]), H.dev(x["evict"])
    kp = H.gpu_pool(shape, k)
    agn = torch.full((w.rows, w.ke), -7, dtype=torch.int32, device="cuda")
    sel = torch.full((w.rows, w.k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / np.sqrt(w.head_dim)
    if noalloc:
        N.nosa_decode_step_noalloc(shape, q, kp, ev, 0, agn, sel, k, v, w.nbmax, scale, out)
    else:
        N.nosa_decode_step(shape, q, kp, ev, 0, agn, sel, k, v, w.nbmax, scale, out, N.workspace(shape))
    torch.cuda.synchronize()
    return sel, agn, out


def test_noalloc_step_matches_the_workspace_step_on_two_calls():
    for w in CALLS:
        print("case", w.name, flush=True)
        x = generate(w)
        sel_a, agn_a, out_a = _run(w, x, noalloc=True)
        sel_b, agn_b, out_b = _run(w, x, noalloc=False)
        assert torch.equal(sel_a, sel_b) and torch.equal(agn_a, agn_b)
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], 32), w.n_blocks, 2)
        H.check_selection(H.host(sel_a), H.host(agn_a), s_ref, x["evict"], w.kq, w.ke)
        ref = O.attention(x["q"], x["k"], x["v"], H.host(sel_a).reshape(w.batch, w.n_kv_heads, w.k))
        print(w.name, H.check_attention(H.host(out_a), ref, "bf16", w.name))


def test_noalloc_step_rejects_a_shape_beyond_the_scratch():
    big = N.make_shape(batch=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, n_blocks=2048, kq=32, ke=32)
    assert N.nosa_workspace_bytes(big) > 16 << 20
    with pytest.raises(N.NosaError) as ei:
        N.nosa_decode_step_noalloc(big, 16, 16, 16, 0, 16, 16, 16, 16, 2048, 0.1, 16, stream=0)
    assert ei.value.code == N.NOSA_ECAPACITY
