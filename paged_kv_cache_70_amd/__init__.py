"""Paged KV-cache write, paged decode and paged prefill attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libpaged_kv.so`` (C ABI in
``include/paged_kv.h``); :mod:`paged_kv_cache_70_amd.api` marshals torch
tensors into it.  Build the library with ``python -m paged_kv_cache_70_amd.build``.
"""
from .api import (  # noqa: F401
    NOALLOC_SCRATCH_BYTES,
    CacheDesc,
    PaError,
    CHECK_CONTEXT_RANGE,
    CHECK_QUERY_RANGE,
    CHECK_SLOT_DUPLICATE,
    CHECK_SLOT_RANGE,
    CHECK_TABLE_RANGE,
    abi_version,
    cache_desc,
    check_decode,
    check_prefill,
    check_write,
    decode,
    decode_append,
    decode_merge,
    decode_noalloc,
    decode_partials_shared_prefix,
    decode_shared_prefix,
    decode_partials,
    library_path,
    load_library,
    measure_mfma,
    measure_read,
    new_append_workspace,
    new_workspace,
    partition_size,
    prefill,
    prefill_workspace,
    status_string,
    workspace_bytes,
    write_kv,
)
from .block_manager import BlockManager, BlockManagerError  # noqa: F401,E402
