"""The C-ABI library loads on a machine without a GPU, exports every entry point the header
declares, and rejects malformed calls on the host before any HIP call."""

import os
import re
import subprocess

import pytest

import block_sparse_kv_decode_amd as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nosa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nosa_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert set(names) == set(N.EXPORTED), names
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (nosa_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(N.lib, n)
    # binding exposes the same names
    for n in names:
        assert callable(getattr(N, n))


def _good(**kw):
    base = dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, n_blocks=256, kq=32, ke=32, cache_slots=64)
    base.update(kw)
    return N.make_shape(**base)


def test_workspace_bytes():
    s = _good()
    n = N.nosa_workspace_bytes(s)
    assert n > 0 and n % 256 == 0
    # the block score buffer alone needs rows * n_blocks_max floats
    assert n >= 16 * 8 * 256 * 4
    assert N.nosa_workspace_bytes(_good(decode_splits=8)) > N.nosa_workspace_bytes(_good(decode_splits=1))


BAD = [
    (dict(n_q_heads=30), N.NOSA_EINVAL),                    # Hq not a multiple of Hkv
    (dict(n_q_heads=48, n_kv_heads=3), N.NOSA_EUNSUPPORTED),  # G = 16
    (dict(head_dim=96), N.NOSA_EUNSUPPORTED),
    (dict(block_size=32), N.NOSA_EUNSUPPORTED),
    (dict(sub_block_size=24), N.NOSA_EUNSUPPORTED),
    (dict(dtype=7), N.NOSA_EUNSUPPORTED),
    (dict(kq=200, ke=100), N.NOSA_EINVAL),                   # budget above visible blocks
    (dict(kq=0, ke=0), N.NOSA_EINVAL),
    (dict(kq=-1), N.NOSA_EINVAL),
    (dict(n_blocks=300, n_blocks_max=256), N.NOSA_EINVAL),
    (dict(n_blocks=0), N.NOSA_EINVAL),
    (dict(n_blocks_max=20000, n_blocks=256), N.NOSA_EUNSUPPORTED),
    (dict(batch=0), N.NOSA_EINVAL),
    (dict(decode_splits=-2), N.NOSA_EINVAL),
    (dict(sink_blocks=-1), N.NOSA_EINVAL),
    (dict(sink_blocks=1, window_blocks=32), N.NOSA_EINVAL),   # sink + window > ke
    (dict(kq=1, ke=8, window_blocks=8, n_blocks=9, n_blocks_max=9, sink_blocks=1), N.NOSA_EINVAL),
    (dict(kq=2**31 - 1, ke=1), N.NOSA_EINVAL),                      # kq + ke overflows int32
    (dict(kq=2**31 - 1, ke=2**31 - 1), N.NOSA_EINVAL),
    (dict(sink_blocks=2**31 - 1, window_blocks=2**31 - 1), N.NOSA_EINVAL),   # sink + window overflows
]


@pytest.mark.parametrize("kw,code", BAD)
def test_invalid_shapes_rejected_on_host(kw, code):
    s = _good(**kw)
    with pytest.raises(N.NosaError) as ei:
        N.nosa_select(s, 16, 16, 16, 0, 16, 16, 256, stream=0)
    assert ei.value.code == code
    assert N.nosa_last_error() != ""
    with pytest.raises(N.NosaError) as ei:
        N.nosa_sparse_decode(s, 16, 16, 16, 256, 16, 0.1, 16, 256, stream=0)
    assert ei.value.code == code
    assert N.lib.nosa_workspace_bytes(s) == 0


def test_invalid_pointers_rejected_on_host():
    s = _good()
    cases = [
        lambda: N.nosa_select(s, None, 16, 16, 0, 16, 16, 256, stream=0),
        lambda: N.nosa_select(s, 8, 16, 16, 0, 16, 16, 256, stream=0),          # q misaligned
        lambda: N.nosa_select(s, 16, 16, 16, 0, 16, 16, 128, stream=0),         # ws misaligned
        lambda: N.nosa_select(s, 16, 16, 16, 300, 16, 16, 256, stream=0),       # n_blocks_prev > n_blocks
        lambda: N.nosa_select(s, 16, 16, 16, -1, 16, 16, 256, stream=0),
        lambda: N.nosa_select(s.copy(sink_blocks=1, window_blocks=16), 16, 16, 16, 10, 16, 16, 256, stream=0),
        lambda: N.nosa_sparse_decode(s, 16, 16, 16, 0, 16, 0.1, 16, 256, stream=0),    # store_blocks 0
        lambda: N.nosa_sparse_decode(s, 16, 16, 16, 256, 16, -1.0, 16, 256, stream=0), # bad scale
        lambda: N.nosa_sparse_decode(s, 16, 16, 16, 256, 16, float("nan"), 16, 256, stream=0),
        lambda: N.nosa_sparse_decode(s, 16, 16, 16, 256, 16, float("inf"), 16, 256, stream=0),
        lambda: N.nosa_decode_step(s, 16, 16, 16, 0, 16, 16, 16, 16, 256, float("inf"), 16, 256, stream=0),
        lambda: N.nosa_sparse_decode(s, 16, 16, 16, 256, None, 0.1, 16, 256, stream=0),
        lambda: N.nosa_pool_keys(s, 16, 250, 10, 16, stream=0),                 # past n_blocks_max
        lambda: N.nosa_pool_keys(s, 16, -1, 1, 16, stream=0),
        lambda: N.nosa_block_scores(s, 16, 16, None, 256, stream=0),
    ]
    for f in cases:
        with pytest.raises(N.NosaError) as ei:
            f()
        assert ei.value.code == N.NOSA_EINVAL, N.nosa_last_error()


def test_cache_update_rejects_small_cache_and_null():
    s = _good(cache_slots=10)
    args = [16] * 10
    with pytest.raises(N.NosaError) as ei:
        N.nosa_cache_update(s, *args, compute=0, copy=0)
    assert ei.value.code == N.NOSA_ECAPACITY
    s = _good()
    with pytest.raises(N.NosaError) as ei:
        N.nosa_cache_update(s, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, compute=0, copy=0)
    assert ei.value.code == N.NOSA_EINVAL


def test_pool_keys_zero_blocks_is_a_noop():
    N.nosa_pool_keys(_good(), 16, 5, 0, 16, stream=0)   # validates, launches nothing


def test_append_rejects_bad_pointers_on_host():
    s = _good()
    with pytest.raises(N.NosaError) as ei:
        N.nosa_append_kv(s, 16, 16, None, 16, 16, 16, 16, stream=0)
    assert ei.value.code == N.NOSA_EINVAL
    with pytest.raises(N.NosaError) as ei:
        N.nosa_append_kv(s, 16, 8, 16, 16, 16, 16, 16, stream=0)      # v_new misaligned
    assert ei.value.code == N.NOSA_EINVAL
    with pytest.raises(N.NosaError) as ei:
        N.nosa_append_kv(_good(head_dim=96), 16, 16, 16, 16, 16, 16, 16, stream=0)
    assert ei.value.code == N.NOSA_EUNSUPPORTED


def test_one_hip_runtime_in_the_process():
    # The library shares torch's HIP runtime: importing the package (which imports torch first)
    # maps exactly one libamdhip64 into the process.
    code = ("import block_sparse_kv_decode_amd, torch\n"
            "m = sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l})\n"
            "print(len(m)); print(m)\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, check=True, cwd=ROOT).stdout
    assert out.splitlines()[0] == "1", out


def test_offload_decode_rejects_on_host():
    s = _good(cache_slots=10)
    args = [16] * 11
    with pytest.raises(N.NosaError) as ei:
        N.nosa_offload_decode(s, 16, *args[:10], 0.1, 16, 256, compute=0, copy=0)
    assert ei.value.code == N.NOSA_ECAPACITY
    s = _good()
    with pytest.raises(N.NosaError) as ei:      # miss_list NULL
        N.nosa_offload_decode(s, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, 16, 0.1, 16, 256, compute=0, copy=0)
    assert ei.value.code == N.NOSA_EINVAL
    with pytest.raises(N.NosaError) as ei:      # bad scale
        N.nosa_offload_decode(s, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 0.0, 16, 256, compute=0, copy=0)
    assert ei.value.code == N.NOSA_EINVAL
    # the one-call offloaded step validates the cache, decode and selection arguments before any launch
    with pytest.raises(N.NosaError) as ei:      # cache below the budget
        N.nosa_offload_step(_good(cache_slots=10), 16, 16, 16, 0, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 0.1, 16,
                            256, compute=0, copy=0)
    assert ei.value.code == N.NOSA_ECAPACITY
    with pytest.raises(N.NosaError) as ei:      # miss_list NULL
        N.nosa_offload_step(s, 16, 16, 16, 0, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, 16, 0.1, 16, 256, compute=0,
                            copy=0)
    assert ei.value.code == N.NOSA_EINVAL
    with pytest.raises(N.NosaError) as ei:      # pooled keys NULL
        N.nosa_offload_step(s, 16, None, 16, 0, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 0.1, 16, 256, compute=0,
                            copy=0)
    assert ei.value.code == N.NOSA_EINVAL
    with pytest.raises(N.NosaError) as ei:      # n_blocks_prev beyond n_blocks
        N.nosa_offload_step(s, 16, 16, 16, s.n_blocks + 1, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 0.1, 16, 256,
                            compute=0, copy=0)
    assert ei.value.code == N.NOSA_EINVAL
    # the workspace grows by the hit table and the second set of partial slots when a cache is set
    assert N.nosa_workspace_bytes(_good(cache_slots=64)) > N.nosa_workspace_bytes(_good(cache_slots=0))


def test_gather_units_rejects_on_host():
    for ub in (0, 8, 24, 1 << 21):
        with pytest.raises(N.NosaError) as ei:
            N.nosa_gather_units(16, 4, 16, 4, ub, 16, 16, 1, stream=0)
        assert ei.value.code == N.NOSA_EINVAL
    with pytest.raises(N.NosaError):
        N.nosa_gather_units(16, 4, 16, 4, 256, 16, 16, -1, stream=0)
    with pytest.raises(N.NosaError):
        N.nosa_gather_units(None, 4, 16, 4, 256, 16, 16, 1, stream=0)
    with pytest.raises(N.NosaError):
        N.nosa_gather_units(16, 4, 8, 4, 256, 16, 16, 1, stream=0)        # dst misaligned
    N.nosa_gather_units(None, 0, None, 0, 256, None, None, 0, stream=0)   # zero units: no-op


def test_rows_limit_rejected_on_host():
    with pytest.raises(N.NosaError) as ei:
        N.nosa_select(_good(batch=10000, n_kv_heads=8, n_q_heads=32), 16, 16, 16, 0, 16, 16, 256, stream=0)
    assert ei.value.code == N.NOSA_EUNSUPPORTED


def test_decode_step_rejects_a_store_smaller_than_the_visible_blocks():
    # Every selected id names a visible block, so a resident store of fewer blocks would let the
    # kernels skip part of the selection: rejected on the host.
    s = _good()
    with pytest.raises(N.NosaError) as ei:
        N.nosa_decode_step(s, 16, 16, 16, 0, 16, 16, 16, 16, 255, 0.1, 16, 256, stream=0)
    assert ei.value.code == N.NOSA_EINVAL
    assert "store_blocks" in N.nosa_last_error()


def test_host_map_and_profile_hook_validate_on_host():
    import ctypes
    out = ctypes.c_void_p(123)
    assert N.lib.nosa_host_map(None, ctypes.byref(out)) == N.NOSA_EINVAL
    assert out.value is None
    assert N.lib.nosa_host_map(16, None) == N.NOSA_EINVAL
    # the profiling hook wants both events or neither
    assert N.lib.nosa_profile_next_kernel(16, None) == N.NOSA_EINVAL
    assert N.lib.nosa_profile_next_kernel(None, 16) == N.NOSA_EINVAL
    assert N.lib.nosa_profile_next_kernel(None, None) == N.NOSA_OK
    # an armed pair is consumed by the next decode call even when that call is rejected, so a
    # failed call leaves nothing armed for a later one
    assert N.lib.nosa_profile_next_kernel(16, 32) == N.NOSA_OK
    with pytest.raises(N.NosaError):
        N.nosa_decode_step(_good(), 16, 16, 16, 0, 16, 16, 16, 16, 0, 0.1, 16, 256, stream=0)


def test_noalloc_step_validates_on_host():
    # a shape whose workspace exceeds the fixed scratch, and an invalid shape, are both rejected
    # before any HIP call
    big = N.make_shape(batch=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, n_blocks=2048, kq=32, ke=32)
    with pytest.raises(N.NosaError) as ei:
        N.nosa_decode_step_noalloc(big, 16, 16, 16, 0, 16, 16, 16, 16, 2048, 0.1, 16, stream=0)
    assert ei.value.code == N.NOSA_ECAPACITY
    with pytest.raises(N.NosaError) as ei:
        N.nosa_decode_step_noalloc(_good(head_dim=96), 16, 16, 16, 0, 16, 16, 16, 16, 256, 0.1, 16, stream=0)
    assert ei.value.code == N.NOSA_EUNSUPPORTED
