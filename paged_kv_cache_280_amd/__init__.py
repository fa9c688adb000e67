"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The computation lives in the HIP library ``libpkv.so`` (C ABI in
``include/pkv.h``); this package is its thin Python binding plus host-side
helpers (byte accounting, the block manager).
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    PkvError,
    CHECK_KINDS,
    abi_version,
    check_batch,
    copy_blocks,
    kv_append,
    kv_append_fp8,
    load_library,
    new_multi_workspace,
    new_workspace,
    paged_attn_decode,
    paged_attn_decode_append,
    paged_attn_decode_fp8,
    paged_attn_decode_noalloc,
    paged_attn_decode_shared,
    paged_attn_decode_shared_workspace_bytes,
    paged_attn_decode_workspace_bytes,
    paged_attn_multi,
    paged_attn_multi_workspace_bytes,
    pools_ok,
    status_string,
)
