"""Python wrapper of the plain CPU oracle (``nosa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by
the benchmark's CPU-baseline leg.  The HIP product path never imports it.

Two builds of the same C source exist.  The default ("f32") accumulates in float32 with
sequential sums, the precision the oracle's contract names; it is the parity reference.  The
"f64" build accumulates in double and serves to bound the f32 build's rounding.  Every function
takes NumPy arrays, widens nothing itself (the C code widens bf16 bit patterns exactly) and
returns arrays of its build's accumulator type; ``precision=`` picks the build per call.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nosa_oracle.c")
_LIBS = {"f32": os.path.join(_HERE, "liboracle.so"), "f64": os.path.join(_HERE, "liboracle_f64.so")}

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile both builds of the oracle with gcc + OpenMP (no HIP, no fast-math); returns the
    path of the default (f32) build."""
    for prec, path in _LIBS.items():
        if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            tmp = path + ".tmp%d" % os.getpid()
            cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                   *(["-DORACLE_F64"] if prec == "f64" else []), _SRC, "-o", tmp, "-lm"]
            subprocess.run(cmd, check=True)
            os.replace(tmp, path)
    return _LIBS["f32"]


_libs = {}


def lib(precision: Optional[str] = None) -> ctypes.CDLL:
    """The oracle library of one build ("f32", the default, or "f64").  NOSA_ORACLE_LIBRARY names
    another build of the same source for the default (the mutation test points it at deliberately
    broken copies to show that the pins catch them)."""
    key = precision or "default"
    if key not in _libs:
        path = os.environ.get("NOSA_ORACLE_LIBRARY") if precision is None else None
        if not path:
            path = _LIBS[precision or "f32"]
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_pool_keys.argtypes = [I64, I64, I, I, P, I, P]
        L.oracle_block_scores.argtypes = [I, I, I, I, I, I, P, I, P, I64, P]
        L.oracle_select.argtypes = [I64, I, I, I, I, P, P, I64, P, P, P]
        L.oracle_select_sw.argtypes = [I64, I, I, I, I, I, I, P, P, I64, P, P, P]
        L.oracle_cache_step.argtypes = [I64, I, I, I, P, P, P, P, P, P]
        L.oracle_gather.argtypes = [I64, I, I, I, I64, P, P, P, P]
        L.oracle_attention.argtypes = [I, I, I, I, I, I, I, P, I, P, P, I, P, D, P]
        L.oracle_attention_masked.argtypes = [I, I, I, I, I, I, I, P, I, P, P, I, P, D, P]
        L.oracle_locality.argtypes = [I64, I, I, P, P, P]
        L.oracle_set_threads.argtypes = [I]
        L.oracle_get_threads.restype = I
        L.oracle_acc_bits.restype = I
        _libs[key] = L
    return _libs[key]


def acc_dtype(precision: Optional[str] = None):
    """NumPy type of the accumulator of a build."""
    return np.float64 if lib(precision).oracle_acc_bits() == 64 else np.float32


def rounding_eps(precision: Optional[str] = None) -> float:
    """Unit roundoff of a build's accumulator (2^-24 or 2^-53)."""
    return float(np.finfo(acc_dtype(precision)).eps) / 2


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError("unsupported oracle input dtype %s" % a.dtype)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its input (code %d)" % (what, rc))


def set_threads(n: int, precision: Optional[str] = None) -> None:
    lib(precision).oracle_set_threads(int(n))


def get_threads(precision: Optional[str] = None) -> int:
    return int(lib(precision).oracle_get_threads())


def pool_keys(k: np.ndarray, sbs: int, n_blocks: Optional[int] = None, precision: Optional[str] = None) -> np.ndarray:
    """k: [B, Hkv, nb, bs, d] (bf16 bits / f32 / f64) -> Kp [B, Hkv, n_blocks*bs/sbs, d]."""
    B, Hkv, nb, bs, d = k.shape
    if n_blocks is None:
        n_blocks = nb
    kk = np.ascontiguousarray(k[:, :, :n_blocks])
    n_tok = n_blocks * bs
    out = np.empty((B, Hkv, n_tok // sbs, d), dtype=acc_dtype(precision))
    _check(lib(precision).oracle_pool_keys(B * Hkv, n_tok, d, sbs, _ptr(kk), _dtype_code(kk), _ptr(out)),
           "pool_keys")
    return out


def block_scores(q: np.ndarray, kp: np.ndarray, n_blocks: int, spb: int, precision: Optional[str] = None) -> np.ndarray:
    """q: [B, Hq, d]; kp: [B, Hkv, nsub, d] (converted to the build's type) -> s [B, Hkv, n_blocks]."""
    B, Hq, d = q.shape
    _, Hkv, nsub, _ = kp.shape
    at = acc_dtype(precision)
    q = np.ascontiguousarray(q)
    kp = np.ascontiguousarray(kp, dtype=at)
    s = np.empty((B, Hkv, n_blocks), dtype=at)
    _check(lib(precision).oracle_block_scores(B, Hq, Hkv, d, n_blocks, spb, _ptr(q), _dtype_code(q), _ptr(kp),
                                              nsub, _ptr(s)), "block_scores")
    return s


def select(s: np.ndarray, evict: np.ndarray, kq: int, ke: int, n_prev: int = 0,
           agn_state: Optional[np.ndarray] = None, n_sink: int = 0,
           n_window: int = 0, precision: Optional[str] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """s: [B, Hkv, n_blocks] block scores (converted to the build's type); evict: [B, Hkv, >=n_blocks]
    float32.

    n_sink / n_window: blocks at the start / end of the visible context that always belong to
    the query-agnostic subset.  Returns (selected [B,Hkv,k] int32 ascending, agn_state
    [B,Hkv,ke] int32 ascending, is_agn [B,Hkv,k] bool)."""
    B, Hkv, n = s.shape
    k = kq + ke
    s = np.ascontiguousarray(s, dtype=acc_dtype(precision))
    ev = np.ascontiguousarray(evict, dtype=np.float32)
    st = np.zeros((B, Hkv, ke), dtype=np.int32) if agn_state is None else \
        np.ascontiguousarray(agn_state, dtype=np.int32).copy()
    sel = np.empty((B, Hkv, k), dtype=np.int32)
    isa = np.empty((B, Hkv, k), dtype=np.uint8)
    _check(lib(precision).oracle_select_sw(B * Hkv, n, kq, ke, n_sink, n_window, n_prev, _ptr(s), _ptr(ev), ev.shape[-1],
                                  _ptr(st) if ke > 0 else None, _ptr(sel), _ptr(isa)), "select")
    return sel, st, isa.astype(bool)


def cache_step(selected: np.ndarray, slot_of_block: np.ndarray, block_of_slot: np.ndarray):
    """One cache step; updates the two maps in place.

    Returns (table [..,k] int32, miss_cnt [..] int32, miss_list [..,k,2] int32)."""
    lead = selected.shape[:-1]
    k = selected.shape[-1]
    R = int(np.prod(lead))
    C = block_of_slot.shape[-1]
    nbmax = slot_of_block.shape[-1]
    sel = np.ascontiguousarray(selected, dtype=np.int32)
    assert slot_of_block.flags["C_CONTIGUOUS"] and slot_of_block.dtype == np.int32
    assert block_of_slot.flags["C_CONTIGUOUS"] and block_of_slot.dtype == np.int32
    table = np.full(lead + (k,), -1, dtype=np.int32)
    mcnt = np.zeros(lead, dtype=np.int32)
    mlist = np.full(lead + (k, 2), -1, dtype=np.int32)
    _check(lib().oracle_cache_step(R, k, C, nbmax, _ptr(sel), _ptr(slot_of_block), _ptr(block_of_slot),
                                   _ptr(table), _ptr(mcnt), _ptr(mlist)), "cache_step")
    return table, mcnt, mlist


def gather(miss_cnt: np.ndarray, miss_list: np.ndarray, host: np.ndarray, cache: np.ndarray) -> None:
    """Copy missed blocks host[..., blk, ...] -> cache[..., slot, ...] in place.

    host: [B, Hkv, nbmax, bs, d]; cache: [B, Hkv, C, bs, d] (any dtype, same for both)."""
    B, Hkv, nbmax = host.shape[:3]
    C = cache.shape[2]
    k = miss_list.shape[-2]
    blk_bytes = int(np.prod(host.shape[3:])) * host.itemsize
    assert host.flags["C_CONTIGUOUS"] and cache.flags["C_CONTIGUOUS"] and host.dtype == cache.dtype
    mc = np.ascontiguousarray(miss_cnt, dtype=np.int32)
    ml = np.ascontiguousarray(miss_list, dtype=np.int32)
    _check(lib().oracle_gather(B * Hkv, k, C, nbmax, blk_bytes, _ptr(mc), _ptr(ml), _ptr(host), _ptr(cache)),
           "gather")


def attention(q: np.ndarray, k_store: np.ndarray, v_store: np.ndarray, table: np.ndarray,
              scale: Optional[float] = None, precision: Optional[str] = None) -> np.ndarray:
    """Gather-form sparse attention. q: [B,Hq,d]; stores: [B,Hkv,nstore,bs,d]; table: [B,Hkv,k]."""
    B, Hq, d = q.shape
    _, Hkv, nstore, bs, _ = k_store.shape
    k = table.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    q = np.ascontiguousarray(q)
    assert k_store.dtype == v_store.dtype
    ks = np.ascontiguousarray(k_store)
    vs = np.ascontiguousarray(v_store)
    tb = np.ascontiguousarray(table, dtype=np.int32)
    out = np.empty((B, Hq, d), dtype=acc_dtype(precision))
    _check(lib(precision).oracle_attention(B, Hq, Hkv, d, bs, k, nstore, _ptr(q), _dtype_code(q), _ptr(ks), _ptr(vs),
                                  _dtype_code(ks), _ptr(tb), float(scale), _ptr(out)), "attention")
    return out


def attention_masked(q: np.ndarray, k_store: np.ndarray, v_store: np.ndarray, mask: np.ndarray,
                     scale: Optional[float] = None, precision: Optional[str] = None) -> np.ndarray:
    """Masked-dense form. mask: [B, Hkv, n_blocks] (nonzero = attend the block)."""
    B, Hq, d = q.shape
    _, Hkv, nstore, bs, _ = k_store.shape
    n_blocks = mask.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    q = np.ascontiguousarray(q)
    ks = np.ascontiguousarray(k_store)
    vs = np.ascontiguousarray(v_store)
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    out = np.empty((B, Hq, d), dtype=acc_dtype(precision))
    _check(lib(precision).oracle_attention_masked(B, Hq, Hkv, d, bs, n_blocks, nstore, _ptr(q), _dtype_code(q), _ptr(ks),
                                         _ptr(vs), _dtype_code(ks), _ptr(m), float(scale), _ptr(out)),
           "attention_masked")
    return out


def append_kv(k_store: np.ndarray, v_store: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              positions: np.ndarray) -> None:
    """Decode append, in place ([P1] paperlayer.ai summary §3.1, pooled keys kept beside the cache;
    [P4] gist.science technical summary, Method 1, blocks arriving under strict eviction).

    stores: [B, Hkv, nbmax, bs, d]; k_new, v_new: [B, Hkv, d]; positions: [B] token index of the
    new token, or outside [0, nbmax * bs) to leave sequence b unchanged.  Token p of a sequence is
    token p % bs of block p // bs.  The pooled key of a sub-block is then ``pool_keys`` of the
    store once its last token has been written."""
    B, Hkv, nbmax, bs, d = k_store.shape
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= nbmax * bs:
            continue
        k_store[b, :, p // bs, p % bs, :] = k_new[b]
        v_store[b, :, p // bs, p % bs, :] = v_new[b]


def gather_units(src: np.ndarray, dst: np.ndarray, unit_bytes: int, src_unit: np.ndarray,
                 dst_unit: np.ndarray) -> None:
    """Transfer at a chosen granularity, in place ([P1] paperlayer.ai summary §3.2, block-wise
    against element-wise communication).  src and dst are viewed as arrays of unit_bytes-byte
    units; for each pair u, unit src_unit[u] of src is copied to unit dst_unit[u] of dst, and a pair
    with either index outside its buffer is skipped."""
    s8 = np.ascontiguousarray(src).view(np.uint8).reshape(-1)
    assert dst.flags["C_CONTIGUOUS"]
    d8 = dst.view(np.uint8).reshape(-1)
    ns, nd = s8.size // unit_bytes, d8.size // unit_bytes
    for su, du in zip(np.asarray(src_unit).tolist(), np.asarray(dst_unit).tolist()):
        if 0 <= su < ns and 0 <= du < nd:
            d8[du * unit_bytes:(du + 1) * unit_bytes] = s8[su * unit_bytes:(su + 1) * unit_bytes]


def locality(prev: np.ndarray, cur: np.ndarray, nbmax: int) -> np.ndarray:
    """gamma per row = |prev ∩ cur| / k."""
    k = cur.shape[-1]
    lead = cur.shape[:-1]
    R = int(np.prod(lead))
    p = np.ascontiguousarray(prev, dtype=np.int32)
    c = np.ascontiguousarray(cur, dtype=np.int32)
    g = np.empty(lead, dtype=np.float64)
    _check(lib().oracle_locality(R, k, nbmax, _ptr(p), _ptr(c), _ptr(g)), "locality")
    return g


def decode_step(q: np.ndarray, kp: np.ndarray, evict: np.ndarray, k_store: np.ndarray, v_store: np.ndarray,
                n_blocks: int, kq: int, ke: int, spb: int, n_prev: int = 0,
                agn_state: Optional[np.ndarray] = None, n_sink: int = 0, n_window: int = 0,
                precision: Optional[str] = None) -> dict:
    """One GPU-resident decode step in the pages' order: scores, selection, attention."""
    s = block_scores(q, kp, n_blocks, spb, precision)
    sel, st, isa = select(s, evict, kq, ke, n_prev, agn_state, n_sink, n_window, precision)
    out = attention(q, k_store, v_store, sel, precision=precision)
    return {"scores": s, "selected": sel, "agn_state": st, "is_agn": isa, "out": out}
