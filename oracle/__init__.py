"""CPU oracle for paged KV writes and paged attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never calls it, and it
never calls the HIP library.
"""

from .pkv_oracle import (  # noqa: F401
    attention,
    bf16_bits_from_f64,
    combine_partials,
    decode,
    decode_one,
    index_errors,
    prefill,
    prefill_one,
    slot_mapping,
    split_partials,
    storage_to_f64,
    token_rows,
    write,
)
