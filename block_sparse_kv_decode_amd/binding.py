"""Thin ctypes binding of ``libnosa.so`` (the C ABI in ``include/nosa.h``).

Argument marshalling only: every function takes device tensors (anything with
``data_ptr()``), plain integers for pointers, or ``None`` for NULL, forwards them to the
C entry point of the same name, and raises :class:`NosaError` on a non-zero status.  All
work runs in the library's HIP kernels; there is no fallback path.

Arguments that may live in pinned host memory (the offloaded KV pool) are passed to the library
as device addresses.  A plain integer is taken to be one already (``host_map`` of the tensor,
resolved once: the form for hot loops and graph capture); a CPU tensor is mapped on the spot with
``nosa_host_map``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Any, Optional

# torch is imported before the library is opened, so that libnosa.so binds to the HIP runtime
# torch has already loaded.  Opened first, it would load the system HIP runtime, and torch would
# then load its own bundled copy: two runtimes in one process, each blind to the other's
# allocations and streams.
import torch  # noqa: F401,E402

_PKG = os.path.dirname(os.path.abspath(__file__))
# NOSA_LIBRARY selects another build of the same library (e.g. an experimental variant).
LIB_PATH = os.environ.get("NOSA_LIBRARY") or os.path.join(_PKG, "libnosa.so")

NOSA_OK, NOSA_EINVAL, NOSA_EUNSUPPORTED, NOSA_ECAPACITY, NOSA_EHIP = 0, -1, -2, -3, -4
NOSA_F32, NOSA_BF16 = 0, 1

EXPORTED = (
    "nosa_last_error", "nosa_version", "nosa_workspace_bytes", "nosa_pool_keys", "nosa_append_kv",
    "nosa_block_scores", "nosa_select", "nosa_cache_update", "nosa_sparse_decode", "nosa_offload_decode",
    "nosa_gather_units", "nosa_decode_step", "nosa_host_map", "nosa_profile_next_kernel",
    "nosa_profile_last_kernel", "nosa_decode_step_noalloc", "nosa_offload_step",
)


class NosaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("nosa error %d: %s" % (code, message))
        self.code = code


class NosaShape(ctypes.Structure):
    """Mirror of ``nosa_shape``."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "block_size", "sub_block_size", "n_blocks",
        "n_blocks_max", "kq", "ke", "cache_slots", "dtype", "decode_splits", "select_parts", "sink_blocks",
        "window_blocks")]

    def copy(self, **changes) -> "NosaShape":
        s = NosaShape()
        ctypes.pointer(s)[0] = self
        for k, v in changes.items():
            setattr(s, k, int(v))
        return s

    def __repr__(self) -> str:
        return "NosaShape(%s)" % ", ".join("%s=%d" % (n, getattr(self, n)) for n, _ in self._fields_)


def make_shape(*, batch, n_q_heads, n_kv_heads, head_dim, n_blocks, kq, ke, n_blocks_max=None,
               block_size=64, sub_block_size=32, cache_slots=0, dtype=NOSA_BF16, decode_splits=0,
               select_parts=0, sink_blocks=0, window_blocks=0) -> NosaShape:
    s = NosaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = batch, n_q_heads, n_kv_heads, head_dim
    s.block_size, s.sub_block_size, s.n_blocks = block_size, sub_block_size, n_blocks
    s.n_blocks_max = n_blocks if n_blocks_max is None else n_blocks_max
    s.kq, s.ke, s.cache_slots, s.dtype = kq, ke, cache_slots, dtype
    s.decode_splits, s.select_parts = decode_splits, select_parts
    s.sink_blocks, s.window_blocks = sink_blocks, window_blocks
    return s


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnosa.so is not built (%s); run `python block_sparse_kv_decode_amd/build.py` "
                          "or __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SP = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(NosaShape)
    L.nosa_last_error.restype = ctypes.c_char_p
    L.nosa_last_error.argtypes = []
    L.nosa_version.restype = ctypes.c_char_p
    L.nosa_version.argtypes = []
    L.nosa_workspace_bytes.restype = ctypes.c_size_t
    L.nosa_workspace_bytes.argtypes = [SP]
    L.nosa_pool_keys.restype = ctypes.c_int
    L.nosa_pool_keys.argtypes = [SP, P, I32, I32, P, P]
    L.nosa_append_kv.restype = ctypes.c_int
    L.nosa_append_kv.argtypes = [SP, P, P, P, P, P, P, P, P]
    L.nosa_block_scores.restype = ctypes.c_int
    L.nosa_block_scores.argtypes = [SP, P, P, P, P, P]
    L.nosa_select.restype = ctypes.c_int
    L.nosa_select.argtypes = [SP, P, P, P, I32, P, P, P, P]
    L.nosa_cache_update.restype = ctypes.c_int
    L.nosa_cache_update.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P]
    L.nosa_decode_step.restype = ctypes.c_int
    L.nosa_decode_step.argtypes = [SP, P, P, P, I32, P, P, P, P, I32, ctypes.c_float, P, P, P]
    L.nosa_gather_units.restype = ctypes.c_int
    L.nosa_gather_units.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int64, P, P, ctypes.c_int64, P]
    L.nosa_offload_decode.restype = ctypes.c_int
    L.nosa_offload_decode.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P]
    L.nosa_offload_step.restype = ctypes.c_int
    L.nosa_offload_step.argtypes = [SP, P, P, P, I32, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P]
    L.nosa_sparse_decode.restype = ctypes.c_int
    L.nosa_sparse_decode.argtypes = [SP, P, P, P, I32, P, ctypes.c_float, P, P, P]
    L.nosa_host_map.restype = ctypes.c_int
    L.nosa_host_map.argtypes = [P, ctypes.POINTER(ctypes.c_void_p)]
    L.nosa_profile_next_kernel.restype = ctypes.c_int
    L.nosa_profile_next_kernel.argtypes = [P, P]
    L.nosa_profile_last_kernel.restype = ctypes.c_char_p
    L.nosa_profile_last_kernel.argtypes = []
    L.nosa_decode_step_noalloc.restype = ctypes.c_int
    L.nosa_decode_step_noalloc.argtypes = [SP, P, P, P, I32, P, P, P, P, I32, ctypes.c_float, P, P]
    return L


lib = _load()


def _p(x: Any) -> Optional[int]:
    """Pointer of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def nosa_host_map(x: Any) -> int:
    """Device address of a buffer (device memory as is; pinned host memory: its device mapping)."""
    out = ctypes.c_void_p()
    _check(lib.nosa_host_map(_p(x), ctypes.byref(out)))
    return int(out.value)


def host_map(x: Any) -> int:
    """Alias of nosa_host_map: resolve a host pool's device address once, outside hot loops."""
    return nosa_host_map(x)


def _dp(x: Any) -> Optional[int]:
    """Device address of a buffer argument that may be pinned host memory: ints and None as given,
    device tensors by data_ptr, CPU tensors through nosa_host_map."""
    if x is None or isinstance(x, int):
        return x
    if getattr(x, "is_cuda", True):
        return int(x.data_ptr())
    return nosa_host_map(x)


def nosa_profile_next_kernel(start: Any, stop: Any) -> None:
    """Arm two HIP events (handles as ints, or None) for the next decode call on this thread."""
    _check(lib.nosa_profile_next_kernel(start, stop))


def nosa_profile_last_kernel() -> str:
    """Kernel the last armed decode call timed (see nosa_profile_next_kernel)."""
    return lib.nosa_profile_last_kernel().decode()


def _stream(s: Any) -> Optional[int]:
    """HIP stream handle: None -> torch's current stream on the current device; int -> as is."""
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(rc: int) -> None:
    if rc != NOSA_OK:
        raise NosaError(rc, lib.nosa_last_error().decode(errors="replace"))


def nosa_last_error() -> str:
    return lib.nosa_last_error().decode(errors="replace")


def nosa_version() -> str:
    return lib.nosa_version().decode()


def nosa_workspace_bytes(shape: NosaShape) -> int:
    n = int(lib.nosa_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise NosaError(NOSA_EINVAL, nosa_last_error())
    return n


def nosa_pool_keys(shape, k, first_block, n_new, pooled_k, stream=None) -> None:
    _check(lib.nosa_pool_keys(ctypes.byref(shape), _p(k), int(first_block), int(n_new), _p(pooled_k),
                              _stream(stream)))


def nosa_append_kv(shape, k_new, v_new, positions, k_store, v_store, pool_acc, pooled_k, stream=None) -> None:
    _check(lib.nosa_append_kv(ctypes.byref(shape), _p(k_new), _p(v_new), _p(positions), _dp(k_store), _dp(v_store),
                              _p(pool_acc), _p(pooled_k), _stream(stream)))


def nosa_block_scores(shape, q, pooled_k, scores, ws, stream=None) -> None:
    _check(lib.nosa_block_scores(ctypes.byref(shape), _p(q), _p(pooled_k), _p(scores), _p(ws), _stream(stream)))


def nosa_select(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, ws, stream=None) -> None:
    _check(lib.nosa_select(ctypes.byref(shape), _p(q), _p(pooled_k), _p(evict), int(n_blocks_prev),
                           _p(agn_state), _p(selected), _p(ws), _stream(stream)))


def nosa_cache_update(shape, selected, slot_of_block, block_of_slot, block_table, miss_cnt, miss_list,
                      host_k, host_v, cache_k, cache_v, compute=None, copy=None) -> None:
    cs = _stream(compute)
    cp = cs if copy is None else _stream(copy)
    _check(lib.nosa_cache_update(ctypes.byref(shape), _p(selected), _p(slot_of_block), _p(block_of_slot),
                                 _p(block_table), _p(miss_cnt), _p(miss_list), _dp(host_k), _dp(host_v),
                                 _p(cache_k), _p(cache_v), cs, cp))


def nosa_sparse_decode(shape, q, k_store, v_store, store_blocks, block_table, softmax_scale, out, ws,
                       stream=None) -> None:
    _check(lib.nosa_sparse_decode(ctypes.byref(shape), _p(q), _p(k_store), _p(v_store), int(store_blocks),
                                  _p(block_table), float(softmax_scale), _p(out), _p(ws), _stream(stream)))


def workspace(shape: NosaShape, device=None):
    """Zero-filled device workspace of nosa_workspace_bytes(shape) bytes (a torch uint8 tensor)."""
    import torch
    return torch.zeros(nosa_workspace_bytes(shape), dtype=torch.uint8, device=device or "cuda")


def nosa_offload_decode(shape, q, selected, slot_of_block, block_of_slot, block_table, miss_cnt, miss_list,
                        host_k, host_v, cache_k, cache_v, softmax_scale, out, ws, compute=None, copy=None) -> None:
    """copy=None runs everything on the compute stream (bf16: the gather of the misses and the attention
    over the hits in one launch); a second stream runs the gather there instead."""
    cs = _stream(compute)
    cp = cs if copy is None else _stream(copy)
    _check(lib.nosa_offload_decode(ctypes.byref(shape), _p(q), _p(selected), _p(slot_of_block), _p(block_of_slot),
                                   _p(block_table), _p(miss_cnt), _p(miss_list), _dp(host_k), _dp(host_v),
                                   _p(cache_k), _p(cache_v), ctypes.c_float(softmax_scale), _p(out), _p(ws), cs, cp))


def nosa_gather_units(src, src_units, dst, dst_units, unit_bytes, src_unit, dst_unit, n_units,
                      stream=None) -> None:
    _check(lib.nosa_gather_units(_dp(src), int(src_units), _dp(dst), int(dst_units), int(unit_bytes), _p(src_unit),
                                 _p(dst_unit), int(n_units), _stream(stream)))


def nosa_offload_step(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, slot_of_block, block_of_slot,
                      block_table, miss_cnt, miss_list, host_k, host_v, cache_k, cache_v, softmax_scale, out, ws,
                      compute=None, copy=None) -> None:
    """nosa_select then nosa_offload_decode in one call (streams as for nosa_offload_decode)."""
    cs = _stream(compute)
    cp = cs if copy is None else _stream(copy)
    _check(lib.nosa_offload_step(ctypes.byref(shape), _p(q), _p(pooled_k), _p(evict), int(n_blocks_prev),
                                 _p(agn_state), _p(selected), _p(slot_of_block), _p(block_of_slot), _p(block_table),
                                 _p(miss_cnt), _p(miss_list), _dp(host_k), _dp(host_v), _p(cache_k), _p(cache_v),
                                 ctypes.c_float(softmax_scale), _p(out), _p(ws), cs, cp))


def nosa_decode_step(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, k_store, v_store, store_blocks,
                     softmax_scale, out, ws, stream=None) -> None:
    _check(lib.nosa_decode_step(ctypes.byref(shape), _p(q), _p(pooled_k), _p(evict), int(n_blocks_prev),
                                _p(agn_state), _p(selected), _p(k_store), _p(v_store), int(store_blocks),
                                ctypes.c_float(softmax_scale), _p(out), _p(ws), _stream(stream)))


def nosa_decode_step_noalloc(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, k_store, v_store,
                             store_blocks, softmax_scale, out, stream=None) -> None:
    """nosa_decode_step with the library's fixed per-GPU scratch as its workspace (allocates nothing)."""
    _check(lib.nosa_decode_step_noalloc(ctypes.byref(shape), _p(q), _p(pooled_k), _p(evict), int(n_blocks_prev),
                                        _p(agn_state), _p(selected), _p(k_store), _p(v_store), int(store_blocks),
                                        ctypes.c_float(softmax_scale), _p(out), _stream(stream)))
