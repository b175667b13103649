"""CPU fp64 oracle for generalized paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  It shares no code with the HIP path.
"""
from .block_manager_ref import BlockManagerRef, copy_blocks_ref, swap_blocks_ref
from .paged_ref import (BLOCK_SIZE, attention_blockwise_ref, attention_ref,
                        attention_ref_sample, attention_split_merge_ref, bits_to_f64,
                        gather_keys_values, internal_fragmentation, kv_bytes_per_token,
                        kv_cache_elements, kv_write_ref, merge_partitions, num_blocks,
                        partition_state)

__all__ = ["BLOCK_SIZE", "BlockManagerRef", "copy_blocks_ref", "swap_blocks_ref", "attention_blockwise_ref", "attention_ref", "attention_ref_sample",
           "attention_split_merge_ref", "bits_to_f64", "gather_keys_values",
           "internal_fragmentation", "kv_bytes_per_token", "kv_cache_elements", "kv_write_ref",
           "merge_partitions", "num_blocks", "partition_state"]
