"""CPU fp64 oracle for the paged decode path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does.
"""
from .paged_attention import (  # noqa: F401
    BLOCK_SIZE,
    reshape_and_cache,
    copy_blocks,
    swap_blocks,
    decode,
    decode_step,
    gather_sequence,
    attention_one_query,
    logical_k_blocks,
    logical_v_blocks,
    kv_bytes_per_token,
)
from .chunked_prefill import prefill, prefill_flops  # noqa: F401
