"""NOSA decode-step hot path on AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libnosa.so`` (C ABI: ``include/nosa.h``); this package
is its thin Python binding.  Importing it fails loudly when the library is not built.
"""

from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, NOSA_BF16, NOSA_EHIP, NOSA_EINVAL, NOSA_ECAPACITY, NOSA_EUNSUPPORTED, NOSA_F32,
    NOSA_OK, NosaError, NosaShape, lib, make_shape, nosa_block_scores, nosa_cache_update,
    nosa_last_error, nosa_pool_keys, nosa_append_kv, nosa_select, nosa_sparse_decode, nosa_version,
    nosa_offload_decode, nosa_gather_units, nosa_decode_step, nosa_host_map, host_map, nosa_profile_next_kernel,
    nosa_profile_last_kernel, nosa_decode_step_noalloc, nosa_offload_step,
    nosa_workspace_bytes, workspace,
)
