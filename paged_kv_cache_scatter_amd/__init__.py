"""Paged KV cache write and paged decode attention for AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of ``libpkv.so``
(``include/pkv.h``); this package is the thin ctypes binding over it.
"""

from ._binding import (  # noqa: F401
    BF16,
    EXPORTS,
    F32,
    NOALLOC_SCRATCH_BYTES,
    LIB_PATH,
    PkvError,
    PreparedCall,
    PoolDesc,
    SCHEDULES,
    VALIDATE_FIELDS,
    abi_version,
    block_bytes,
    decode,
    decode_shared,
    decode_shared_workspace_bytes,
    decode_step,
    decode_step_noalloc,
    decode_partition,
    decode_schedule,
    decode_workspace_bytes,
    debug_enabled,
    load,
    plan_pool,
    pool_desc,
    prepare_decode,
    prepare_decode_step,
    prefill,
    slot_mapping,
    validate,
    write,
)
