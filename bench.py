"""Benchmark of the NOSA decode-step hot path on one MI355X.

A step is one decode step of one attention layer for every sequence of the batch, GPU-resident:
nosa_decode_step, which is nosa_select (pooled-key block scoring + query-agnostic / query-aware
selection) followed by nosa_sparse_decode (split-K GQA attention over the selected blocks) in one
call.  Pooled keys are state built once before timing (they change only when a block fills up).
tokens/s = batch / step time.  The timed steps are fresh ones (n_blocks_prev = 0: the query-agnostic
part ranks every visible block); ms_per_step_steady_state times the same step with n_blocks_prev =
n_blocks, where it ranks the previous step's members under strict eviction.

  python bench.py [--gpus 1] [--steps 1000] [--warmup 50] [--config C2] [--also C3,F1,C5]
                  [--no-cpu-baseline] [--no-offload] [--no-transfer]

Prints one JSON line.  `value` is the headline workload (bs16 / 16K context by default); the
same line carries the bs64 / 4K workload and the sink + window split under "also", the decode
kernel's roofline and the CPU oracle baseline, the 128-step offload loop (pinned host KV pool,
64-slot GPU cache, decode tokens appended each step) under "offload", and the block- vs
element-wise transfer sweep under "transfer_granularity".
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LAYERS = 4   # independent buffer sets the resident step rotates over (see run_resident)
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak, GB/s
PROFILES = os.path.join(ROOT, "profiles")


def traffic_path(cfg, kernel):
    """Counter record of HBM bytes per launch of one kernel on one workload (rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs scaled by the plain-copy calibration; written by --record-traffic)."""
    return os.path.join(PROFILES, "traffic_%s_%s.json" % (kernel, cfg))
# the sources the attention and step kernels are compiled from
KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_kv_decode_amd", "csrc", f)
               for f in ("decode.hip", "select_core.h", "nosa_device.h", "nosa_internal.h")]


def kernel_src_sha256():
    """SHA-256 of the kernel sources' code: comments and blank space are dropped first, so an edit
    to a comment does not void counter records taken on the same code."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        text = re.sub(r"/\*.*?\*/", " ", open(f).read(), flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_INPUTS = {}


def inputs(cfg):
    """Generated host inputs of a workload, drawn once per process (workloads that draw the same
    tensors, e.g. a different budget split on the same seed, share them)."""
    from nosa_inputs import WORKLOADS, generate
    w = WORKLOADS[cfg]
    key = (w.seed, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.nbmax, w.dtype, w.block_offset_sigma,
           w.steps, w.drift_sigma)
    if key not in _INPUTS:
        t0 = time.time()
        _INPUTS[key] = generate(w)
        log("[bench] %s inputs generated in %.1fs" % (cfg, time.time() - t0))
    return _INPUTS[key]


def algorithmic_bytes(w):
    """Bytes the method must move per step: the selected K and V blocks, the fp32 pooled keys and
    the eviction scores of every visible block, q, the output, and the selected ids."""
    eb = 2 if w.dtype == "bf16" else 4
    R, k, d, B, Hq = w.rows, w.k, w.head_dim, w.batch, w.n_q_heads
    kv_sel = R * k * 64 * d * eb * 2                      # selected K and V blocks
    kp = R * w.n_blocks * 2 * d * 4                       # pooled keys, fp32, 2 sub-blocks per block
    ev = R * w.n_blocks * 4                               # eviction scores
    q = B * Hq * d * eb
    o = B * Hq * d * eb
    ids = R * k * 4                                       # selected ids
    decode = kv_sel + q + o + ids                         # decode kernel: K/V, q, out, table
    select = kp + q + ev + ids + R * w.ke * 4             # select kernel: pooled keys, q, e, out ids + state
    step = kv_sel + kp + ev + q + o + ids
    # The dominant kernel of nosa_decode_step, per launch (32 KiB of K + V per selected block at bf16 /
    # d 128, times the R * k selected blocks, plus what else that kernel must read or write):
    #   row_step_kernel     the whole step in one launch: the step's bytes;
    #   step_decode_kernel  attention with the query-aware pick inside: K/V, q, each row's block
    #                       scores and query-agnostic ids it ranks from, the selection it writes (the
    #                       output is written by the merge kernel after it);
    #   decode_*_kernel     attention of the two-call plan: K/V, q, the block ids (output by the merge).
    kernel = {"row_step_kernel": step,
              "step_decode_kernel": kv_sel + q + R * w.n_blocks * 4 + R * w.ke * 4 + ids,
              "decode_mfma_kernel": kv_sel + q + ids, "decode_valu_kernel": kv_sel + q + ids}
    return {"step": step, "decode": decode, "select": select, "kernel": kernel}


class HipTimingEvents:
    """HIP timing events created with hipEventDisableSystemFence.  A default event performs a
    system-scope fence (cache writeback and invalidation) when it completes, which lengthens and
    disturbs the kernels it brackets; timing-only events can skip it.  The calls go to the HIP
    runtime torch has loaded (found in the process map, so no second runtime is opened)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.ct = ctypes
        self.L = ctypes.CDLL(path)
        self.L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.owned = []

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.L.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        assert rc == 0, "hipEventCreateWithFlags failed (%d)" % rc
        self.owned.append(ev)
        return ev

    def record(self, ev, stream_handle):
        rc = self.L.hipEventRecord(ev, self.ct.c_void_p(stream_handle))
        assert rc == 0, "hipEventRecord failed (%d)" % rc

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.L.hipEventElapsedTime(self.ct.byref(ms), a, b)
        assert rc == 0, "hipEventElapsedTime failed (%d)" % rc
        return float(ms.value)

    def close(self):
        for ev in self.owned:
            self.L.hipEventDestroy(ev)
        self.owned = []


def run_resident(cfg, steps, warmup, want_events=True, decode_splits=0, select_parts=0, layers=LAYERS):
    """The resident decode step, timed.  Consecutive steps rotate over `layers` independent sets of
    device buffers (q, K/V stores, pooled keys, eviction scores, outputs), as the attention layers
    of a model would: one layer's selected K/V (268 MB at bs16 / 16K) is about the size of the
    GPU's 256 MB last-level cache, and repeating a single layer's step would let that cache serve
    part of every step.  The sets are copies of one synthetic layer at different addresses."""
    import numpy as np
    import torch

    import block_sparse_kv_decode_amd as N
    from nosa_inputs import WORKLOADS

    w = WORKLOADS[cfg]
    x = inputs(cfg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    shape = N.make_shape(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                         n_blocks=w.n_blocks, n_blocks_max=w.nbmax, kq=w.kq, ke=w.ke, sub_block_size=32,
                         dtype=N.NOSA_BF16 if w.dtype == "bf16" else N.NOSA_F32, decode_splits=decode_splits,
                         select_parts=select_parts, sink_blocks=w.n_sink, window_blocks=w.n_window)
    R = w.rows
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    first = dict(q=dev(x["q"]), k=dev(x["k"]), v=dev(x["v"]), ev=dev(x["evict"]))
    sets = []
    for li in range(layers):
        t = {name: (a if li == 0 else a.clone()) for name, a in first.items()}
        t["kp"] = torch.empty((R, w.nbmax * 2, w.head_dim), dtype=torch.float32, device="cuda")
        t["agn"] = torch.empty((R, max(w.ke, 1)), dtype=torch.int32, device="cuda")
        t["sel"] = torch.empty((R, w.k), dtype=torch.int32, device="cuda")
        t["out"] = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=t["q"].dtype, device="cuda")
        N.nosa_pool_keys(shape, t["k"], 0, w.nbmax, t["kp"], sh)           # state, off the step timer
        sets.append(t)
    ws = N.workspace(shape)
    torch.cuda.synchronize()
    scale = 1.0 / (w.head_dim ** 0.5)
    # raw pointers, resolved once: the timed loop only enqueues
    P = [{name: a.data_ptr() for name, a in t.items()} for t in sets]
    wsp = ws.data_ptr()

    T = HipTimingEvents() if want_events else None

    def step(i):
        """The product's decode step: one nosa_decode_step call."""
        p = P[i % layers]
        N.nosa_decode_step(shape, p["q"], p["kp"], p["ev"], 0, p["agn"], p["sel"], p["k"], p["v"], w.nbmax, scale,
                           p["out"], wsp, sh)

    def steady(i):
        """The same step in steady state: n_blocks_prev = n_blocks, so the query-agnostic part ranks
        the previous step's members (agn_state, left by the fresh steps) under strict eviction."""
        p = P[i % layers]
        N.nosa_decode_step(shape, p["q"], p["kp"], p["ev"], w.n_blocks, p["agn"], p["sel"], p["k"], p["v"], w.nbmax,
                           scale, p["out"], wsp, sh)

    def two_calls(i, evs=None):
        """The same step as nosa_select + nosa_sparse_decode, with events between the two calls."""
        p = P[i % layers]
        if evs is not None:
            T.record(evs[0], sh)
        N.nosa_select(shape, p["q"], p["kp"], p["ev"], 0, p["agn"], p["sel"], wsp, sh)
        if evs is not None:
            T.record(evs[1], sh)
        N.nosa_sparse_decode(shape, p["q"], p["k"], p["v"], w.nbmax, p["sel"], scale, p["out"], wsp, sh)
        if evs is not None:
            T.record(evs[2], sh)

    def wall(fn, warm=True):
        if warm:
            for i in range(warmup):
                fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # timed region 1: the plain step loop (headline value): `warmup` untimed steps, then exactly
    # `steps` timed steps between two synchronisations
    wall_s = wall(step)
    # the same region repeated (reported beside the headline, which stays the first region), with
    # events at both ends of each repeat: the GPU-side span shows how much of the wall time per step
    # is host latency at the region's two ends.  The events skip the system-scope fence: a default
    # event's fence adds a fixed 10-16 us to the region (measured on MI355X: 20-step C2 regions
    # 0.0623 ms per step without events, 0.0631 with default events, 0.0628 with these; no
    # difference over 1000 steps).
    RT = T if T is not None else HipTimingEvents()
    repeats, spans = [], []
    for _ in range(3):
        e0, e1 = RT.create(), RT.create()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        RT.record(e0, sh)
        for i in range(steps):
            step(i)
        RT.record(e1, sh)
        torch.cuda.synchronize()
        repeats.append(1e3 * (time.perf_counter() - t0) / steps)
        spans.append(RT.elapsed_ms(e0, e1) / steps)
    if RT is not T:
        RT.close()
    res = {"wall_s": wall_s, "ms_per_step": 1e3 * wall_s / steps, "tokens_per_s": w.batch * steps / wall_s,
           "ms_per_step_repeats": repeats, "gpu_span_ms_per_step_repeats": spans, "layers": layers,
           "ms_per_step_two_calls": 1e3 * wall(two_calls) / steps,
           "ms_per_step_steady": 1e3 * wall(steady) / steps}
    if want_events:
        # A bounded spin kernel holds the stream while the host enqueues the event-timed steps, so
        # the GPU never waits on the host inside an event pair (Python can take longer to enqueue a
        # step than the GPU takes to run it).
        def hold():
            torch.cuda.synchronize()
            torch.cuda._sleep(int(2.4e9 * (steps * 80e-6 + 2e-3)))

        # timed region 2: the two-call step with events around each call
        evs = [[T.create() for _ in range(3)] for _ in range(steps)]
        hold()
        for i in range(steps):
            two_calls(i, evs[i])
        torch.cuda.synchronize()
        sel_ms = [T.elapsed_ms(e[0], e[1]) for e in evs]
        dec_ms = [T.elapsed_ms(e[1], e[2]) for e in evs]
        # timed region 3: events around every nosa_decode_step call
        evs1 = [[T.create() for _ in range(2)] for _ in range(steps)]
        hold()
        for i in range(steps):
            T.record(evs1[i][0], sh)
            step(i)
            T.record(evs1[i][1], sh)
        torch.cuda.synchronize()
        stp_ms = [T.elapsed_ms(e[0], e[1]) for e in evs1]
        # timed region 4: the step's dominant kernel alone, bracketed by the library's profiling
        # hook (events recorded on the launch stream right before and after that kernel)
        evs2 = [[T.create() for _ in range(2)] for _ in range(steps)]
        hold()
        names = set()
        for i in range(steps):
            N.nosa_profile_next_kernel(evs2[i][0].value, evs2[i][1].value)
            step(i)
            names.add(N.nosa_profile_last_kernel())
        torch.cuda.synchronize()
        assert len(names) == 1, names
        ker_ms = [T.elapsed_ms(e[0], e[1]) for e in evs2]
        T.close()
        res.update({
            "select_ms_mean": statistics.mean(sel_ms), "decode_ms_mean": statistics.mean(dec_ms),
            "step_ms_median": statistics.median(stp_ms),
            "step_ms_p10": float(np.percentile(stp_ms, 10)), "step_ms_p90": float(np.percentile(stp_ms, 90)),
            "kernel": names.pop(), "kernel_ms_mean": statistics.mean(ker_ms),
            "kernel_ms_median": statistics.median(ker_ms),
        })
    # The step's outputs, checked against the oracle: every buffer set holds a copy of the same layer,
    # so every set's last step must give one result, bit for bit; set 0's is compared with the oracle.
    torch.cuda.synchronize()
    for t in sets[1:min(steps, layers)]:
        assert torch.equal(t["sel"], sets[0]["sel"]) and torch.equal(t["agn"], sets[0]["agn"])
        assert torch.equal(t["out"].view(torch.int16) if t["out"].dtype == torch.bfloat16 else t["out"],
                           sets[0]["out"].view(torch.int16) if t["out"].dtype == torch.bfloat16 else sets[0]["out"])
    res["outputs"] = {name: sets[0][name].cpu() for name in ("sel", "agn", "out")}
    res["bytes"] = algorithmic_bytes(w)
    res["workload"] = w
    return res


def check_step_outputs(cfg, res):
    """Compares the timed step's selection and output with the oracle on the same inputs: the
    selection exactly (outside the 1e-4 relative tie band at the query-aware cut), the output
    elementwise (bf16: |err| / max(|ref|, 1e-3) <= 1e-2 and mean |err| <= 2e-3).  Raises on a
    mismatch; returns the error figures."""
    import numpy as np
    import torch

    from nosa_inputs import WORKLOADS
    from oracle import oracle as O
    from tests.gpuhelp import check_attention, check_selection

    w = WORKLOADS[cfg]
    x = inputs(cfg)
    t0 = time.perf_counter()
    o = res["outputs"]
    sel = o["sel"].numpy()
    agn = o["agn"].numpy()[:, :w.ke]
    out = o["out"].view(torch.int16).numpy().view(np.uint16) if o["out"].dtype == torch.bfloat16 else o["out"].numpy()
    s_ref = O.block_scores(x["q"], O.pool_keys(x["k"], 32), w.n_blocks, 2)
    ties = check_selection(sel, agn, s_ref, x["evict"], w.kq, w.ke, n_sink=w.n_sink, n_window=w.n_window)
    ref = O.attention(x["q"], x["k"], x["v"], sel.reshape(w.batch, w.n_kv_heads, w.k))
    stats = check_attention(out, ref, w.dtype, cfg + " timed step")
    return dict(checked=True, oracle="fp32 CPU oracle (selection and attention on the same inputs)",
                tie_band_rows=ties, seconds=round(time.perf_counter() - t0, 2), **stats)


def run_offload(cfg="C4", full=True, steps_cap=None):
    """The 128-step offload loop of workload cfg (pinned host KV pool, 64-slot cache per KV head).

    A step appends the previous step's token (nosa_append_kv into the pinned host pool and the
    pooled keys; workloads with whole blocks arriving per step have them in the pool beforehand),
    selects and runs the offloaded decode in one nosa_offload_step call (the cache map at the end of the
    query-aware pick; the gather of the misses and attention over the cache hits in one launch).  Every pass starts from the same state (empty cache, prompt pooled keys): one
    pass records miss counts, selections and query-agnostic subsets (for hit rate, bytes per step,
    locality, and a check of the strict-eviction bounds), three timed passes run the overlapped path;
    with `full`, three more run the serial calls (cache_update on the compute stream, then
    sparse_decode), one serial pass with events between the calls gives the per-phase breakdown and
    the gather rate, and the synchronised-step passes compare eager launches with HIP graphs."""
    import numpy as np
    import torch

    import block_sparse_kv_decode_amd as N
    from nosa_inputs import WORKLOADS, generate, visible_blocks

    w = WORKLOADS[cfg]
    x = generate(w)
    n0 = w.n_blocks
    append = w.blocks_per_step == 0

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    def pin(a):
        src = bf16(a)
        t = torch.empty(src.shape, dtype=torch.bfloat16, pin_memory=True)
        t.copy_(src)
        return t

    if append:   # the pool holds the prompt; the decode tokens are appended step by step
        prompt_k, prompt_v = x["k"].copy(), x["v"].copy()
        prompt_k[:, :, n0:] = 0
        prompt_v[:, :, n0:] = 0
        hk, hv = pin(prompt_k), pin(prompt_v)
        del prompt_k, prompt_v
    else:        # blocks arriving whole: written to the pool beforehand, made visible step by step
        hk, hv = pin(x["k"]), pin(x["v"])
    hkd, hvd = N.host_map(hk), N.host_map(hv)     # the pool's device addresses, resolved once
    kdev = bf16(x["k"]).cuda()
    shape0 = N.make_shape(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                          n_blocks=w.n_blocks, n_blocks_max=w.nbmax, kq=w.kq, ke=w.ke, cache_slots=w.cache_slots,
                          sink_blocks=w.n_sink, window_blocks=w.n_window)
    R, k, C, d = w.rows, w.k, w.cache_slots, w.head_dim
    kp = torch.empty((R, w.nbmax * 2, d), dtype=torch.float32, device="cuda")
    acc = torch.empty((R, d), dtype=torch.float32, device="cuda")
    if append:
        # the decode tokens, step-major: token t of the decode is position n_tokens + t
        new_k = bf16(x["k"][:, :, n0:].reshape(w.batch, w.n_kv_heads, -1, d).transpose(2, 0, 1, 3)).cuda()
        new_v = bf16(x["v"][:, :, n0:].reshape(w.batch, w.n_kv_heads, -1, d).transpose(2, 0, 1, 3)).cuda()
        positions = (torch.arange(w.steps, dtype=torch.int32, device="cuda").view(-1, 1) + (w.n_tokens - 1)) \
            .expand(w.steps, w.batch).contiguous()
    qs = bf16(x["q_steps"]).cuda()
    ev = torch.from_numpy(x["evict"]).cuda()
    del x
    ck = torch.zeros((w.batch, w.n_kv_heads, C, 64, d), dtype=torch.bfloat16, device="cuda")
    cv = torch.zeros_like(ck)
    sob = torch.empty((R, w.nbmax), dtype=torch.int32, device="cuda")
    bos = torch.empty((R, C), dtype=torch.int32, device="cuda")
    table = torch.empty((R, k), dtype=torch.int32, device="cuda")
    mcnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    mlist = torch.empty((R, k, 2), dtype=torch.int32, device="cuda")
    agn = torch.empty((R, w.ke), dtype=torch.int32, device="cuda")
    sel = torch.empty((R, k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, d), dtype=torch.bfloat16, device="cuda")
    ws = N.workspace(shape0)
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream()
    scale = 1.0 / (d ** 0.5)
    steps = w.steps if steps_cap is None else min(w.steps, steps_cap)
    mc_hist = torch.empty((steps, R), dtype=torch.int32, device="cuda")
    sel_hist = torch.empty((steps, R, k), dtype=torch.int32, device="cuda")
    agn_hist = torch.empty((steps, R, w.ke), dtype=torch.int32, device="cuda")

    def reset():
        sob.fill_(-1)
        bos.fill_(-1)
        # prompt blocks only when tokens are appended; every block otherwise (visibility limits use)
        N.nosa_pool_keys(shape0, kdev, 0, n0 if append else w.nbmax, kp)
        torch.cuda.synchronize()

    def loop(overlap, timed=False, stats=False, phases=False):
        """One pass of the loop from the reset state.  timed: events only after step 0 and after
        the last step (warm mean over steps 1..); stats: copies of miss counts, selections and
        query-agnostic subsets per step; phases: events between the calls of every step (each event
        adds a few us)."""
        reset()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)] if phases else None
        ta, tb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_prev = 0
        for t in range(steps):
            if timed and t == 1:
                ta.record(stream)
            n = visible_blocks(w, t)
            shape = shape0.copy(n_blocks=n)
            if phases:
                evs[t][0].record(stream)
            if append and t > 0:
                N.nosa_append_kv(shape0, new_k[t - 1], new_v[t - 1], positions[t], hkd, hvd, acc, kp, stream)
            if overlap == "step":
                # nosa_select + nosa_offload_decode in one call (the cache map folded into the pick)
                N.nosa_offload_step(shape, qs[t], kp, ev, n_prev, agn, sel, sob, bos, table, mcnt, mlist, hkd, hvd,
                                    ck, cv, scale, out, ws, stream, None)
            else:
                N.nosa_select(shape, qs[t], kp, ev, n_prev, agn, sel, ws, stream)
            if phases:
                evs[t][1].record(stream)
            if overlap == "step":
                pass
            elif overlap:
                # "side": the gather on a copy stream; otherwise gather and hit attention in one launch
                N.nosa_offload_decode(shape, qs[t], sel, sob, bos, table, mcnt, mlist, hkd, hvd, ck, cv, scale,
                                      out, ws, stream, copy_stream if overlap == "side" else None)
            else:
                N.nosa_cache_update(shape, sel, sob, bos, table, mcnt, mlist, hkd, hvd, ck, cv, stream, stream)
                if phases:
                    evs[t][2].record(stream)
                N.nosa_sparse_decode(shape, qs[t], ck, cv, C, table, scale, out, ws, stream)
            if phases:
                evs[t][3].record(stream)
            if stats:
                mc_hist[t].copy_(mcnt)
                sel_hist[t].copy_(sel)
                agn_hist[t].copy_(agn)
            n_prev = n
        if timed:
            tb.record(stream)
        torch.cuda.synchronize()
        res = {}
        if timed:
            res["warm_ms"] = ta.elapsed_time(tb) / (steps - 1)
        if phases:
            res["select"] = [e[0].elapsed_time(e[1]) for e in evs]
            res["cache"] = [e[1].elapsed_time(e[2]) for e in evs]
            res["decode"] = [e[2].elapsed_time(e[3]) for e in evs]
        return res

    loop("step", stats=True)                      # warm-up pass (code objects, host pool pages) + stats
    misses = mc_hist.sum(dim=1).cpu().numpy().tolist()
    s_h = sel_hist.cpu().numpy()
    a_h = agn_hist.cpu().numpy()
    mean_ms = statistics.median([loop("step", timed=True)["warm_ms"] for _ in range(3)])
    # Locality and the strict-eviction bounds, every row and step: the query-agnostic subset changes
    # only by admitting arrivals (Gamma_e(t) within Gamma_e(t-1) and the arrivals A(t)), so adjacent
    # selections share at least ke - a(t) blocks, a(t) = admitted arrivals; gamma >= (ke - a(t)) / k.
    gam, bound, evicted = [], [], 0
    for t in range(1, steps):
        n_prev, n = visible_blocks(w, t - 1), visible_blocks(w, t)
        for r in range(R):
            E0, E1 = set(a_h[t - 1, r].tolist()), set(a_h[t, r].tolist())
            arrivals = set(range(n_prev, n))
            assert E1 <= E0 | arrivals, (cfg, t, r)
            a_t = len(E1 & arrivals)
            evicted += len(E0 - E1)
            ov = len(set(s_h[t - 1, r].tolist()) & set(s_h[t, r].tolist()))
            assert ov >= w.ke - a_t, (cfg, t, r, ov, a_t)
            gam.append(ov / k)
            bound.append((w.ke - a_t) / k)
    warm = slice(1, steps)
    blk_bytes = 64 * d * 2 * 2
    fetched = [m * blk_bytes for m in misses]
    res = {
        "workload": "%s: B16, GQA 32/8, d128, 16K ctx (%s), %d+%d blocks%s, 64-slot GPU cache per KV head, %d steps" % (
            cfg, "+1 token/step, appended to the pinned host pool" if append else
            "+%d block(s) arriving per step" % w.blocks_per_step, w.kq, w.ke,
            " (agnostic part incl. %d sink + %d window blocks)" % (w.n_sink, w.n_window) if w.n_window else "", steps),
        "path": "%snosa_offload_step (the selection, the cache map folded into the query-aware pick, the gather of "
                "the misses and attention over the hits in one launch, the misses, the merge)" % (
                    "nosa_append_kv + " if append else ""),
        "hit_rate_warm": 1.0 - statistics.mean(misses[warm]) / (R * k),
        "fetched_bytes_per_step_warm": statistics.mean(fetched[warm]),
        "cold_step_fetched_bytes": fetched[0],
        "gamma_min": min(gam), "gamma_mean": statistics.mean(gam),
        "gamma_guarantee_min": min(bound),
        "agnostic_evictions_per_row_step": evicted / (R * (steps - 1)),
        "strict_eviction_bounds_checked": True,
        "step_ms_mean_warm": mean_ms,
        "tokens_per_s": w.batch / (mean_ms * 1e-3),
    }
    if not full:
        return res
    serial_ms = statistics.median([loop(False, timed=True)["warm_ms"] for _ in range(3)])
    side_ms = statistics.median([loop("side", timed=True)["warm_ms"] for _ in range(3)])
    two_call_ms = statistics.median([loop(True, timed=True)["warm_ms"] for _ in range(3)])
    ph = loop(False, phases=True)
    # A serving loop waits for every step.  Host wall time per step with a synchronisation after
    # each, the step's calls launched eagerly vs replayed from captured HIP graphs (inputs copied
    # into static buffers first in both cases).
    from block_sparse_kv_decode_amd.step_graph import OffloadStepGraphs
    st = dict(host_k=hk, host_v=hv, pooled_k=kp, pool_acc=acc, evict=ev, agn=agn, selected=sel, slot_of_block=sob,
              block_of_slot=bos, block_table=table, miss_cnt=mcnt, miss_list=mlist, cache_k=ck, cache_v=cv, out=out,
              ws=ws)
    graphs = OffloadStepGraphs(shape0, st, None, scale)

    def sync_loop(use_graph):
        reset()
        wall = []
        n_prev = 0
        for t in range(steps):
            n = visible_blocks(w, t)
            t0 = time.perf_counter()
            graphs.q.copy_(qs[t])
            if append and t > 0:
                graphs.k_new.copy_(new_k[t - 1])
                graphs.v_new.copy_(new_v[t - 1])
                graphs.positions.copy_(positions[t])
            if use_graph:
                graphs.replay(n, n_prev, append and t > 0)
            else:
                graphs.enqueue(n, n_prev, append and t > 0)
            torch.cuda.synchronize()
            wall.append((time.perf_counter() - t0) * 1e3)
            n_prev = n
        return statistics.median(wall[1:])

    sync_loop(True)                               # captures the graphs
    sync_eager_ms = statistics.median([sync_loop(False) for _ in range(3)])
    sync_graph_ms = statistics.median([sync_loop(True) for _ in range(3)])
    cache_ms = statistics.mean(ph["cache"][warm])
    res.update({
        "serial_step_ms_mean_warm": serial_ms,
        "side_stream_step_ms_mean_warm": side_ms,
        "select_then_offload_decode_ms_mean_warm": two_call_ms,
        "serial_phase_ms_mean_warm": {"append_select": statistics.mean(ph["select"][warm]),
                                      "cache_update": cache_ms, "sparse_decode": statistics.mean(ph["decode"][warm])},
        "h2d_gbps_warm_serial_cache_update": statistics.mean(fetched[warm]) / (cache_ms * 1e-3) / 1e9,
        "tokens_per_s_serial": w.batch / (serial_ms * 1e-3),
        "sync_every_step_wall_ms_median": {"eager": sync_eager_ms, "hip_graph": sync_graph_ms,
                                           "graphs_captured": len(graphs.graphs)},
    })
    return res


def run_transfer(reps=20):
    """Block-wise vs element-wise host-to-GPU transfer at batch 64, 4096-token context, d 128 bf16,
    2 KV heads (128 rows).  Per row a 1024-token (16-block) GPU cache; at locality gamma a fraction
    1 - gamma of it is refilled per step, either as whole 64-token blocks (16 KiB units) or as
    single tokens (256-byte units) scattered over the row's context, K and V each.  Both moves carry
    the same bytes through nosa_gather_units; lists are in ascending source order."""
    import numpy as np
    import torch

    import block_sparse_kv_decode_amd as N

    R, ctx, cache_tok, d, bs = 64 * 2, 4096, 1024, 128, 64
    tok_b, blk_b = d * 2, bs * d * 2
    host_k = torch.empty(R * ctx * d, dtype=torch.bfloat16, pin_memory=True).fill_(1.0)
    host_v = torch.empty(R * ctx * d, dtype=torch.bfloat16, pin_memory=True).fill_(2.0)
    dev_k = torch.zeros(R * cache_tok * d, dtype=torch.bfloat16, device="cuda")
    dev_v = torch.zeros_like(dev_k)
    rng = np.random.default_rng(11)
    stream = torch.cuda.current_stream()
    out = []

    def timed(unit_bytes, su, du, n_src, n_dst):
        su_t, du_t = torch.from_numpy(su).cuda(), torch.from_numpy(du).cuda()
        n = len(su)
        for _ in range(3):
            N.nosa_gather_units(host_k, n_src, dev_k, n_dst, unit_bytes, su_t, du_t, n, stream)
            N.nosa_gather_units(host_v, n_src, dev_v, n_dst, unit_bytes, su_t, du_t, n, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            N.nosa_gather_units(host_k, n_src, dev_k, n_dst, unit_bytes, su_t, du_t, n, stream)
            N.nosa_gather_units(host_v, n_src, dev_v, n_dst, unit_bytes, su_t, du_t, n, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for gamma in (0.5, 0.8, 0.9, 0.95, 0.99):
        nb = max(1, int(round((1 - gamma) * (cache_tok // bs) * R)))
        dst = rng.choice(R * (cache_tok // bs), nb, replace=False)
        src = (dst // (cache_tok // bs)) * (ctx // bs) + rng.integers(0, ctx // bs, nb)
        o = np.argsort(src, kind="stable")
        t_blk = timed(blk_b, src[o].astype(np.int32), dst[o].astype(np.int32), R * (ctx // bs), R * (cache_tok // bs))
        nt = nb * bs
        dst = rng.choice(R * cache_tok, nt, replace=False)
        src = (dst // cache_tok) * ctx + rng.integers(0, ctx, nt)
        o = np.argsort(src, kind="stable")
        t_tok = timed(tok_b, src[o].astype(np.int32), dst[o].astype(np.int32), R * ctx, R * cache_tok)
        by = 2 * nb * blk_b
        out.append({"gamma": gamma, "bytes_per_step": by, "block_units": 2 * nb, "element_units": 2 * nt,
                    "block_ms": t_blk, "element_ms": t_tok,
                    "block_gbps": by / (t_blk * 1e-3) / 1e9, "element_gbps": by / (t_tok * 1e-3) / 1e9})
    return {"workload": "batch 64, context 4096, d 128 bf16, 2 KV heads: a 1024-token GPU cache per row, "
                        "refilled by a fraction 1 - gamma per step (K and V)",
            "block_unit_bytes": blk_b, "element_unit_bytes": tok_b, "by_locality": out}


def measure_link_peak():
    """Pinned host -> device copy bandwidth of a large hipMemcpyAsync (SDMA), GB/s."""
    import torch
    n = 512 << 20
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    return 5 * n / (time.perf_counter() - t0) / 1e9


def cpu_baseline(cfg, budget_s=10.0, single_s=4.0, max_s=30.0):
    """The CPU oracle (fp32, sequential sums, OpenMP over rows) on the same workload: scores +
    selection + attention per step, repeated until about budget_s of wall time on every allowed core,
    then for about single_s on one thread."""
    from nosa_inputs import WORKLOADS
    from oracle import oracle as O

    w = WORKLOADS[cfg]
    x = inputs(cfg)
    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))
    kp = O.pool_keys(x["k"], 32)      # state, excluded like on the GPU

    def run(n_threads, budget):
        O.set_threads(n_threads)
        reps, t0 = 0, time.perf_counter()
        while True:
            O.decode_step(x["q"], kp, x["evict"], x["k"], x["v"], w.n_blocks, w.kq, w.ke, 2, n_sink=w.n_sink,
                          n_window=w.n_window)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or el + el / reps > max_s:
                return reps, el

    reps, el = run(threads, budget_s)
    cores = O.get_threads()
    reps1, el1 = run(1, single_s)
    O.set_threads(threads)
    step_bytes = algorithmic_bytes(w)["step"]
    return {"value": w.batch * reps / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d full %s decode steps (block scores + selection + attention, all %d rows), "
                      "%.1f s wall, fp32 oracle" % (reps, cfg, w.rows, el),
            "effective_gbps": step_bytes * reps / el / 1e9,
            "single_thread": {"value": w.batch * reps1 / el1, "unit": "tokens/s",
                              "sample": "%d steps, %.1f s wall" % (reps1, el1)}}


def traffic_record(cfg, kernel):
    """HBM bytes per launch of `kernel` on workload `cfg` from the committed rocprofv3 counter runs, if
    they were taken on the current kernel sources."""
    path = traffic_path(cfg, kernel)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_src_sha256") != kernel_src_sha256() or rec.get("workload") != cfg or \
            rec.get("kernel") != kernel:
        return None
    return rec.get("bytes_per_launch")


def _counter_kib(csv_dir, counter, kernel, contains=""):
    """Mean value of `counter` per dispatch of the kernels whose base name is `kernel` (and whose full
    name contains `contains`), from the counter_collection CSV files rocprofv3 wrote under csv_dir."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            name = row.get("Kernel_Name", "")
            base = name.split("(")[0].split("<")[0].split(" ")[-1].split("::")[-1]
            if row.get("Counter_Name") == counter and base == kernel and contains in name:
                key = (f, row.get("Dispatch_Id"))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit("no %s samples of %s under %s" % (counter, kernel, csv_dir))
    return statistics.mean(vals.values()), len(vals)


def record_traffic(cfg, kernel, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, commands):
    """Writes profiles/traffic_<kernel>_<cfg>.json: FETCH_SIZE and WRITE_SIZE per dispatch of `kernel`
    (KiB, from two rocprofv3 --pmc runs of the benchmark), each scaled by what the same counter reads
    for a plain copy of 256 MiB read + 256 MiB written (bench.py --copy-calibration)."""
    from nosa_inputs import WORKLOADS
    fk, nf = _counter_kib(fetch_dir, "FETCH_SIZE", kernel)
    wk, nw = _counter_kib(write_dir, "WRITE_SIZE", kernel)
    # the copy: torch's elementwise multiply by 1 (the tensor fill before it is another kernel)
    cf, _ = _counter_kib(cal_fetch_dir, "FETCH_SIZE", "vectorized_elementwise_kernel", "MulFunctor")
    cw, _ = _counter_kib(cal_write_dir, "WRITE_SIZE", "vectorized_elementwise_kernel", "MulFunctor")
    true_kib = (64 << 20) * 4 / 1024.0
    ff, wf = true_kib / cf, true_kib / cw
    fetch_b, write_b = fk * 1024 * ff, wk * 1024 * wf
    rec = {"workload": cfg, "kernel": kernel,
           "what": "HBM bytes per dispatch of %s in nosa_decode_step on %s (%d / %d dispatches)" % (kernel, cfg, nf, nw),
           "commands": commands,
           "raw_kib_per_dispatch": {"FETCH_SIZE": fk, "WRITE_SIZE": wk},
           "calibration": {"copy_kernel": "elementwise x*1 over 256 MiB float32 (reads and writes 268435456 B)",
                           "FETCH_SIZE_kib": cf, "WRITE_SIZE_kib": cw, "fetch_factor": ff, "write_factor": wf},
           "bytes_per_launch": int(round(fetch_b + write_b)), "fetch_bytes_per_launch": int(round(fetch_b)),
           "write_bytes_per_launch": int(round(write_b)),
           "algorithmic_bytes_per_launch": algorithmic_bytes(WORKLOADS[cfg])["kernel"][kernel],
           "kernel_src_sha256": kernel_src_sha256(),
           "kernel_src_hash_of": "decode.hip, select_core.h, nosa_device.h, nosa_internal.h with comments and "
                                 "blank space removed"}
    with open(traffic_path(cfg, kernel), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def describe(w):
    extra = ""
    if w.n_sink or w.n_window:
        extra = " (agnostic part incl. %d sink + %d window blocks)" % (w.n_sink, w.n_window)
    return "%s: B%d, GQA %d/%d, d%d, ctx %d, budget %d+%d blocks of 64 tokens%s, %s" % (
        w.name, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.kq, w.ke, extra, w.dtype)


def kernel_roofline(cfg, r):
    """Roofline entry of the step's dominant kernel: algorithmic bytes per launch over its mean
    duration (HIP events from the library's profiling hook, on the launch stream)."""
    kb = r["bytes"]["kernel"][r["kernel"]]
    achieved = kb / (r["kernel_ms_mean"] * 1e-3) / 1e9
    return {"kernel": r["kernel"], "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_record(cfg, r["kernel"]),
            "algorithmic_bytes_per_launch": kb, "avg_launch_ms": r["kernel_ms_mean"],
            "median_launch_ms": r["kernel_ms_median"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps (about 70 ms at bs16 / 16K): the first launches after a synchronisation take a few
    # hundred microseconds, which 100 steps would spread as several microseconds per step
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--also", default="C3,F1,C5", help="comma list of extra resident workloads ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU timing and the check of the timed outputs)")
    ap.add_argument("--no-offload", action="store_true", help="skip the 128-step offload loops (C4)")
    ap.add_argument("--no-transfer", action="store_true", help="skip the block- vs element-wise transfer sweep")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of 256 MiB (reference for HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=6, metavar=("CONFIG", "KERNEL", "FETCH_DIR", "WRITE_DIR",
                                                          "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write profiles/traffic_<KERNEL>_<CONFIG>.json from rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--record-commands", default="", help="';;'-separated commands quoted in the record")
    args = ap.parse_args()
    if args.record_traffic:
        cfg, kernel, fd, wd, cfd, cwd = args.record_traffic
        record_traffic(cfg, kernel, fd, wd, cfd, cwd, [c for c in args.record_commands.split(";;") if c])
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (rows would shard "
              "across GPUs with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 64 << 20                      # float32 elements: 256 MiB read + 256 MiB written per launch
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel": "elementwise mul by 1 (float32)", "bytes_read_per_launch": 4 * n,
                          "bytes_written_per_launch": 4 * n, "launches": 5}), flush=True)
        return

    main_res = run_resident(args.config, args.steps, args.warmup)
    w = main_res["workload"]
    by = main_res["bytes"]
    dec_s = main_res["decode_ms_mean"] * 1e-3
    step_gbps = by["step"] / (main_res["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": "sparse-decode tokens/s and achieved HBM GB/s (bs64 ctx4K, bs16 ctx16K)",
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded PCG64; K with per-block mean offsets, V ~N(0,1), eviction scores ~U(0,1))",
        "config": {"workload": describe(w), "batch": w.batch, "context": w.n_tokens, "block": 64,
                   "budget_blocks": w.k, "kq": w.kq, "ke": w.ke, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "layers": 1,
                   "step": "nosa_decode_step: selection + attention in one call",
                   "buffer_sets_rotated": main_res["layers"]},
        "step_hbm_gbps": step_gbps,
        "step_hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "step_algorithmic_bytes": by["step"],
        "ms_per_step_repeats": main_res["ms_per_step_repeats"],
        "gpu_span_ms_per_step_repeats": main_res["gpu_span_ms_per_step_repeats"],
        "ms_per_step_two_calls": main_res["ms_per_step_two_calls"],
        "ms_per_step_steady_state": main_res["ms_per_step_steady"],
        "step_ms_median_events": main_res["step_ms_median"],
        "step_ms_p10_p90_events": [main_res["step_ms_p10"], main_res["step_ms_p90"]],
        "roofline": kernel_roofline(args.config, main_res),
        "two_call_attention": {
            "kernels": "nosa_sparse_decode call: decode_mfma_kernel + combine_kernel (split-K merge)",
            "avg_call_ms": main_res["decode_ms_mean"], "algorithmic_bytes": by["decode"],
            "achieved_gbps": by["decode"] / dec_s / 1e9},
        "select_call": {"avg_call_ms": main_res["select_ms_mean"], "algorithmic_bytes": by["select"],
                        "achieved_gbps": by["select"] / (main_res["select_ms_mean"] * 1e-3) / 1e9},
    }
    results = {args.config: main_res}
    also = {}
    for cfg in [c for c in args.also.split(",") if c]:
        r = run_resident(cfg, args.steps, args.warmup)
        results[cfg] = r
        b2 = r["bytes"]
        also[cfg] = {
            "workload": describe(r["workload"]), "tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"],
            "ms_per_step_repeats": r["ms_per_step_repeats"],
            "gpu_span_ms_per_step_repeats": r["gpu_span_ms_per_step_repeats"],
            "ms_per_step_two_calls": r["ms_per_step_two_calls"],
            "ms_per_step_steady_state": r["ms_per_step_steady"],
            "step_hbm_gbps": b2["step"] / (r["ms_per_step"] * 1e-3) / 1e9,
            "step_hbm_frac": b2["step"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "step_ms_median_events": r["step_ms_median"],
            "step_events_gbps": b2["step"] / (r["step_ms_median"] * 1e-3) / 1e9,
            "roofline": kernel_roofline(cfg, r),
            "two_call_decode_gbps": b2["decode"] / (r["decode_ms_mean"] * 1e-3) / 1e9,
        }
    if also:
        line["also"] = also
    link = None
    if not args.no_offload:
        line["offload"] = run_offload("C4")
        link = measure_link_peak()
        line["offload"]["link_peak_gbps_sdma"] = link
        # the eviction dynamics: one block arriving per step, and the pages' 16 + 48 split
        line["offload"]["variants"] = {cfg: run_offload(cfg, full=False) for cfg in ("C4S", "C4P", "C4PS")}
    if not args.no_transfer:
        line["transfer_granularity"] = run_transfer()
        line["transfer_granularity"]["link_peak_gbps_sdma"] = link if link is not None else measure_link_peak()
    if not args.no_cpu_baseline:
        # the oracle leg: the timed outputs of every resident workload against the oracle (a mismatch
        # ends the run without a result line), then the oracle's own timing on the headline workload
        checks = {cfg: check_step_outputs(cfg, r) for cfg, r in results.items()}
        line["checked"] = checks[args.config]
        if also:
            for cfg in also:
                also[cfg]["checked"] = checks[cfg]
        line["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
