"""Plain CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  It shares no code with the HIP library in
``paged_kv_cache_388_amd`` and imports nothing from it.

Every function is pinned by ``tests/test_oracle_pins.py`` against values the
pages print, closed forms, invariants the pages state and brute force on tiny
inputs.  No function in this package is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    DTYPES,
    blocks_for_tokens,
    copy_blocks,
    decode_attention,
    gather_context,
    kv_bytes_per_token,
    kv_append,
    last_block_fill,
    mean_tail_waste,
    merge_partitions,
    multi_query_attention,
    partition_states,
    split_decode_attention,
    storage_to_f64,
    swap_in,
    swap_out,
)
