"""Seeded synthetic inputs for the NOSA decode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, scoring, selection, caching or attention).
Both the CPU oracle (tests) and the HIP path (tests, bench) take their inputs
from here, so the two sides always consume identical values.

Every array is drawn with NumPy's PCG64 (``np.random.default_rng(seed)``) in
float32 and, for bf16 workloads, rounded to bfloat16 with round-to-nearest-even.
bf16 values are carried as their raw 16-bit patterns (``uint16``); the helper
``bf16_bits_to_f32`` widens them exactly.

Workloads follow the decode setting of "NOSA: Native and Offloadable Sparse
Attention" (paperlayer.ai summary, §B.2.2 and §3.2): blocks of 64 tokens,
head dim 128, a 4096-token (64-block) budget at 16K context.  The pages name no
public data set for the efficiency runs, so these synthetic tensors stand in.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BLOCK = 64       # tokens per KV block
SUB_BLOCK = 32   # tokens per mean-pooled sub-block


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporary memory on the large workloads
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        # finite values cannot overflow uint32 here; NaNs are patched afterwards
        r = ((v + np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
        nan = (v & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = ((v[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
        flat_o[s:s + step] = r
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes of one decode-step workload (one attention layer)."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int            # context length visible at the (first) step
    kq: int                  # query-aware budget, blocks
    ke: int                  # query-agnostic budget, blocks
    dtype: str               # "bf16" or "f32"
    seed: int
    block_offset_sigma: float = 0.5   # std of the per-block mean offset added to K (0 = none)
    n_blocks_max: Optional[int] = None   # allocated blocks (>= n_tokens/BLOCK)
    cache_slots: int = 0              # GPU cache slots per KV head (offload loop only)
    steps: int = 1                    # decode steps (offload loop only)
    drift_sigma: float = 0.0          # std of the per-step query drift (offload loop only)
    n_sink: int = 0                   # first blocks always in the query-agnostic subset
    n_window: int = 0                 # most recent blocks always in the query-agnostic subset
    blocks_per_step: int = 0          # offload loop: 0 = one token per step (appended); b > 0 = b whole
                                      # blocks become visible per step (written to the pool beforehand)
    description: str = ""

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // BLOCK

    @property
    def nbmax(self) -> int:
        return self.n_blocks_max if self.n_blocks_max is not None else self.n_blocks

    @property
    def rows(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def k(self) -> int:
        return self.kq + self.ke


# The five workloads of the build's configuration list.
WORKLOADS: Dict[str, Workload] = {
    "C1": Workload("C1", 1, 2, 1, 64, 1024, 4, 4, "f32", seed=1, block_offset_sigma=0.0,
                   description="tiny single step: B1, 2q/1kv heads, d64, 1K ctx, 4+4 blocks, fp32"),
    "C2": Workload("C2", 16, 32, 8, 128, 16384, 32, 32, "bf16", seed=2,
                   description="single step: B16, GQA 32/8, d128, 16K ctx, 32+32 blocks, bf16"),
    "C3": Workload("C3", 64, 32, 8, 128, 4096, 8, 8, "bf16", seed=3,
                   description="single step: B64, GQA 32/8, d128, 4K ctx, 8+8 blocks, bf16"),
    # 258 blocks allocated: block 256 fills during the first 64 decode steps, and the tokens of
    # steps 65..127 go to block 257, which is still open (never visible) when the loop ends.
    "C4": Workload("C4", 16, 32, 8, 128, 16384, 32, 32, "bf16", seed=4, n_blocks_max=258,
                   cache_slots=64, steps=128, drift_sigma=0.3,
                   description="offload loop: C2 shape, 128 steps, 64-slot GPU cache, pinned host pool"),
    "C5": Workload("C5", 4, 32, 8, 128, 131072, 32, 32, "bf16", seed=5,
                   description="long context: B4, GQA 32/8, d128, 128K ctx, 32+32 blocks, bf16"),
    # The paper's own budget split on the C2 tensors (same seed): 16 query-aware blocks and 48
    # query-agnostic ones that include 1 sink block and a 16-block sliding window.
    "F1": Workload("F1", 16, 32, 8, 128, 16384, 16, 48, "bf16", seed=2, n_sink=1, n_window=16,
                   description="C2 tensors with the paper split: 16 query-aware + 48 agnostic (1 sink, 16 window)"),
    # The offload loop with the paper's split (the C4 tensors): the window slides as blocks fill.
    "C4P": Workload("C4P", 16, 32, 8, 128, 16384, 16, 48, "bf16", seed=4, n_blocks_max=258, cache_slots=64,
                    steps=128, drift_sigma=0.3, n_sink=1, n_window=16,
                    description="offload loop, paper split 16 + 48 (1 sink, 16 window), 1 token per step"),
    # Stress variants: one whole block arrives at every step (blocks 256 .. 382 become visible at
    # steps 1 .. 127), so the query-agnostic subset drops its lowest member (or the arrival) every step.
    "C4S": Workload("C4S", 16, 32, 8, 128, 16384, 32, 32, "bf16", seed=6, n_blocks_max=383, cache_slots=64,
                    steps=128, drift_sigma=0.3, blocks_per_step=1,
                    description="offload loop, 32 + 32, one block arriving per step"),
    "C4PS": Workload("C4PS", 16, 32, 8, 128, 16384, 16, 48, "bf16", seed=6, n_blocks_max=383, cache_slots=64,
                     steps=128, drift_sigma=0.3, n_sink=1, n_window=16, blocks_per_step=1,
                     description="offload loop, paper split 16 + 48 (1 sink, 16 window), one block per step"),
}


def small_workload(name: str = "small", *, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                   n_blocks=37, kq=5, ke=7, dtype="bf16", seed=11, n_blocks_max=None,
                   cache_slots=0, steps=1, drift_sigma=0.0, block_offset_sigma=0.5, n_sink=0,
                   n_window=0) -> Workload:
    """A reduced workload with the same generator, for tests the oracle finishes in seconds."""
    return Workload(name, batch, n_q_heads, n_kv_heads, head_dim, n_blocks * BLOCK, kq, ke, dtype,
                    seed=seed, block_offset_sigma=block_offset_sigma, n_blocks_max=n_blocks_max,
                    cache_slots=cache_slots, steps=steps, drift_sigma=drift_sigma, n_sink=n_sink,
                    n_window=n_window)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def generate(w: Workload) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w``.

    Returns a dict with
      q      [B, Hq, d]                     (uint16 bf16 bits, or float32)
      k, v   [B, Hkv, nbmax, BLOCK, d]      (same dtype as q)
      evict  [B, Hkv, nbmax] float32        per-block query-agnostic scores, U(0,1)
      q_steps [steps, B, Hq, d]             (only when steps > 1) query at every step,
                                            q_t = q_{t-1} + N(0, drift_sigma^2), rounded per step
    Draw order: q, k noise, k block offsets, v, evict, drift.
    """
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, d, nb = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.nbmax
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, nb, BLOCK, d), dtype=np.float32)
    if w.block_offset_sigma > 0:
        mu = rng.standard_normal((B, Hkv, nb, 1, d), dtype=np.float32) * np.float32(w.block_offset_sigma)
        k += mu
        del mu
    k_out = _round(k, w.dtype)
    del k
    v = rng.standard_normal((B, Hkv, nb, BLOCK, d), dtype=np.float32)
    v_out = _round(v, w.dtype)
    del v
    evict = rng.random((B, Hkv, nb), dtype=np.float32)
    out = {"q": _round(q, w.dtype), "k": k_out, "v": v_out, "evict": evict}
    if w.steps > 1:
        qs = np.empty((w.steps, B, Hq, d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
        cur = q.copy()
        for t in range(w.steps):
            if t > 0:
                cur = cur + rng.standard_normal((B, Hq, d), dtype=np.float32) * np.float32(w.drift_sigma)
            qs[t] = _round(cur, w.dtype)
        out["q_steps"] = qs
    return out


def visible_blocks(w: Workload, step: int) -> int:
    """Blocks visible at decode step ``step``.

    One token appended per step (blocks_per_step = 0): the context holds ``n_tokens + step``
    tokens at step ``step``, and only whole blocks are visible to selection and attention.
    Otherwise ``blocks_per_step`` whole blocks join the visible context at every step.
    """
    if w.blocks_per_step:
        return min(w.nbmax, w.n_tokens // BLOCK + step * w.blocks_per_step)
    return min(w.nbmax, (w.n_tokens + step) // BLOCK)


def to_f32(x: np.ndarray) -> np.ndarray:
    """Widen an input array (bf16 bits or float32) to float32 exactly."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)
