"""HIP-graph capture of one offloaded decode step (launch orchestration only; no compute here).

A decode step of the offload loop is a short chain of library calls -- nosa_append_kv,
nosa_select, nosa_offload_decode (which, without a copy stream, gathers the missed blocks of a bf16
step in the same launch as the attention over the hits, and with one forks the gather onto it and
joins it back) -- whose kernels run for tens of microseconds each.  A serving loop that waits for every
step pays the host-side launch cost of the whole chain on each step; replaying a captured graph
pays one launch.

The library entry points are capture-safe: they only enqueue kernels and event record/wait pairs
on the streams they are given, allocate nothing and never synchronise.  Kernel arguments are
frozen at capture, so the per-step inputs (query, new token, its position) live in static buffers
that the caller refills before each replay, and one graph is kept per (n_blocks, n_blocks_prev,
append) combination -- in a decode loop only a few occur (the first step, steady steps, and the
steps where a block arrives).
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import torch

from . import binding as N


class OffloadStepGraphs:
    """Captured offload decode steps over fixed state buffers.

    ``state`` holds the tensors the step reads and writes (pooled keys, eviction scores, the
    query-agnostic state, selection, cache maps and cache, host pools, workspace, output), all
    allocated by the caller and kept alive as long as this object.  ``q``, ``k_new``, ``v_new`` and
    ``positions`` are the static input buffers refilled before each replay."""

    def __init__(self, shape0: N.NosaShape, state: dict, copy_stream: Optional[torch.cuda.Stream], scale: float):
        self.shape0 = shape0
        self.s = state
        self.copy = copy_stream
        self.scale = float(scale)
        B, Hq, Hkv, d = shape0.batch, shape0.n_q_heads, shape0.n_kv_heads, shape0.head_dim
        dt = state["cache_k"].dtype
        self.q = torch.zeros((B, Hq, d), dtype=dt, device="cuda")
        self.k_new = torch.zeros((B, Hkv, d), dtype=dt, device="cuda")
        self.v_new = torch.zeros((B, Hkv, d), dtype=dt, device="cuda")
        self.positions = torch.zeros((B,), dtype=torch.int32, device="cuda")
        # the host pool's device addresses, resolved once: the captured calls make no pointer query
        self.hk = N.host_map(state["host_k"])
        self.hv = N.host_map(state["host_v"])
        self.graphs: Dict[Tuple[int, int, bool], torch.cuda.CUDAGraph] = {}

    def enqueue(self, n_blocks: int, n_prev: int, append: bool, stream=None) -> None:
        """The step's library calls on ``stream`` (the current stream when None), eagerly."""
        s = self.s
        shape = self.shape0.copy(n_blocks=n_blocks)
        if append:
            N.nosa_append_kv(self.shape0, self.k_new, self.v_new, self.positions, self.hk, self.hv, s["pool_acc"],
                             s["pooled_k"], stream)
        N.nosa_select(shape, self.q, s["pooled_k"], s["evict"], n_prev, s["agn"], s["selected"], s["ws"], stream)
        N.nosa_offload_decode(shape, self.q, s["selected"], s["slot_of_block"], s["block_of_slot"], s["block_table"],
                              s["miss_cnt"], s["miss_list"], self.hk, self.hv, s["cache_k"], s["cache_v"],
                              self.scale, s["out"], s["ws"], stream, self.copy)

    def replay(self, n_blocks: int, n_prev: int, append: bool) -> None:
        key = (n_blocks, n_prev, append)
        g = self.graphs.get(key)
        if g is None:
            g = torch.cuda.CUDAGraph()
            # default (global) capture mode: the calls only enqueue kernels and event record / wait
            # pairs; the host pool mapping was resolved before capture
            with torch.cuda.graph(g):
                self.enqueue(n_blocks, n_prev, append)
            self.graphs[key] = g
        g.replay()
