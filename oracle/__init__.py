"""CPU oracle for the paged decode path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  The product package never imports it.
"""

from .paged_attention import (  # noqa: F401
    attention_weights,
    block_copy,
    brute_force_decode,
    cache_append,
    decode,
    decode_one,
    gather_head,
    gather_head_fast,
    merge_partition_states,
    partition_state,
    slot_of,
    slots_for_positions,
    swap_blocks,
    token_location,
)
