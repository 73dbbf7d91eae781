"""Shared helpers of the GPU parity tests: device transfers, one-call wrappers around the C ABI,
and the comparison rules (tie band for selections, tolerances for attention)."""

from __future__ import annotations

import numpy as np
import torch

import block_sparse_kv_decode_amd as N
from nosa_inputs import BLOCK, Workload, bf16_bits_to_f32
from oracle import oracle as O

# Tolerances.  bf16 outputs: |gpu - ref| / max(|ref|, 1e-3) <= 1e-2 elementwise and mean |gpu - ref|
# <= 2e-3.  fp32 outputs: max |gpu - ref| <= 1e-5 (fp32 accumulation over a few thousand tokens
# stays near 1e-7).  Selections: exact, except where the oracle's kq-th / (kq+1)-th score gap is
# below 1e-4 relative (tie band).
BF16_REL, BF16_FLOOR, BF16_MEAN_ABS = 1e-2, 1e-3, 2e-3
F32_ABS = 1e-5
TIE_REL = 1e-4


def dev(x: np.ndarray) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def pinned(x: np.ndarray) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    src = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 else torch.from_numpy(x)
    t = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
    t.copy_(src)
    return t


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def shape_of(w: Workload, *, sub_block_size=32, n_blocks=None, decode_splits=0, select_parts=0) -> N.NosaShape:
    return N.make_shape(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                        n_blocks=w.n_blocks if n_blocks is None else n_blocks, n_blocks_max=w.nbmax,
                        kq=w.kq, ke=w.ke, sub_block_size=sub_block_size, cache_slots=w.cache_slots,
                        dtype=N.NOSA_BF16 if w.dtype == "bf16" else N.NOSA_F32, decode_splits=decode_splits,
                        select_parts=select_parts, sink_blocks=w.n_sink, window_blocks=w.n_window)


def gpu_pool(shape: N.NosaShape, k_dev: torch.Tensor) -> torch.Tensor:
    spb = shape.block_size // shape.sub_block_size
    R = shape.batch * shape.n_kv_heads
    kp = torch.full((R, shape.n_blocks_max * spb, shape.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    N.nosa_pool_keys(shape, k_dev, 0, shape.n_blocks_max, kp)
    return kp


def gpu_select(shape, q_dev, kp_dev, ev_dev, ws, n_prev=0, agn=None):
    R = shape.batch * shape.n_kv_heads
    k = shape.kq + shape.ke
    if agn is None:
        agn = torch.full((R, max(shape.ke, 1)), -7, dtype=torch.int32, device="cuda")
    sel = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    N.nosa_select(shape, q_dev, kp_dev, ev_dev, n_prev, agn, sel, ws)
    return sel, agn


def gpu_decode(shape, q_dev, k_store, v_store, store_blocks, table, ws, scale=None):
    if scale is None:
        scale = 1.0 / np.sqrt(shape.head_dim)
    out = torch.full((shape.batch, shape.n_q_heads, shape.head_dim), float("nan"), dtype=q_dev.dtype, device="cuda")
    N.nosa_sparse_decode(shape, q_dev, k_store, v_store, store_blocks, table, scale, out, ws)
    return out


def check_attention(out_gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    g = as_f64(out_gpu) if out_gpu.dtype == np.uint16 else out_gpu.astype(np.float64)
    assert np.all(np.isfinite(g)), "%s: non-finite GPU output" % what
    err = np.abs(g - ref)
    # normwise error of every output row (one query head of one sequence), reported
    d = ref.shape[-1]
    norm_rel = np.linalg.norm((g - ref).reshape(-1, d), axis=1) / np.maximum(
        np.linalg.norm(ref.reshape(-1, d), axis=1), 1e-30)
    if dtype == "bf16":
        rel = err / np.maximum(np.abs(ref), BF16_FLOOR)
        stats = {"max_rel": float(rel.max()), "mean_abs": float(err.mean()), "max_row_normwise": float(norm_rel.max())}
        assert rel.max() <= BF16_REL, "%s: max relative error %.3g > %g" % (what, rel.max(), BF16_REL)
        assert err.mean() <= BF16_MEAN_ABS, "%s: mean abs error %.3g > %g" % (what, err.mean(), BF16_MEAN_ABS)
    else:
        stats = {"max_abs": float(err.max()), "max_row_normwise": float(norm_rel.max())}
        assert err.max() <= F32_ABS, "%s: max abs error %.3g > %g" % (what, err.max(), F32_ABS)
    return stats


def check_selection(sel_gpu: np.ndarray, agn_gpu: np.ndarray, s_oracle: np.ndarray, evict: np.ndarray,
                    kq: int, ke: int, n_prev: int = 0, agn_prev=None, n_sink: int = 0, n_window: int = 0) -> int:
    """Compare a GPU selection with the oracle's on the same inputs.

    Gamma_e compares raw eviction scores, so it must match exactly.  The full selection must match
    exactly unless, in that row, the oracle's kq-th and (kq+1)-th best scores outside Gamma_e lie
    within TIE_REL of each other; then any set is accepted that holds every block scored clearly
    above the kq-th score, no block clearly below it, and exactly kq blocks.
    Returns the number of rows decided inside the tie band."""
    sel_o, agn_o, _ = O.select(s_oracle, evict, kq, ke, n_prev, agn_prev, n_sink, n_window)
    B, H, n = s_oracle.shape
    k = kq + ke
    sel_gpu = sel_gpu.reshape(B, H, k)
    if ke > 0:
        agn_gpu = agn_gpu.reshape(B, H, -1)[:, :, :ke]
        assert np.array_equal(agn_gpu, agn_o), "query-agnostic subset differs from the oracle"
    ties = 0
    for b in range(B):
        for h in range(H):
            if np.array_equal(sel_gpu[b, h], sel_o[b, h]):
                continue
            E = set(agn_o[b, h].tolist()) if ke > 0 else set()
            comp = np.array([i for i in range(n) if i not in E])
            sc = s_oracle[b, h, comp]
            order = np.lexsort((comp, -sc))
            T = sc[order[kq - 1]]
            nxt = sc[order[kq]] if kq < len(comp) else -np.inf
            gap = T - nxt
            assert gap < TIE_REL * max(abs(T), abs(nxt)), \
                "row (%d,%d): selection differs outside the tie band: gpu %s oracle %s" % (
                    b, h, sel_gpu[b, h].tolist(), sel_o[b, h].tolist())
            Q = set(sel_gpu[b, h].tolist()) - E
            assert len(Q) == kq and len(set(sel_gpu[b, h].tolist())) == k
            assert np.all(np.diff(sel_gpu[b, h]) > 0)
            band = TIE_REL * abs(T)
            for i, s_ in zip(comp, sc):
                if s_ > T + band:
                    assert i in Q
                if s_ < T - band:
                    assert i not in Q
            ties += 1
    return ties
