"""fp64 CPU oracle for factorized sparse self-attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the HIP
library under ``factorized_sparse_self_amd/`` and neither imports the other.
"""
from .sparse_attention import (DENSE, FIXED, FIXED_R1, FIXED_UNION, STRIDED, STRIDED_UNION,
                               UNION_BASE, backward, backward_dkdv_keys, backward_dq_rows, forward,
                               forward_rows, head_kind, in_key_set, key_set, pair_count,
                               part_key_set, queries_of_key, summary_offsets)
from .block_layout import block_layout, kernel_maps

__all__ = [
    "STRIDED", "FIXED", "FIXED_R1", "DENSE", "STRIDED_UNION", "FIXED_UNION", "UNION_BASE",
    "head_kind", "key_set", "part_key_set", "in_key_set",
    "queries_of_key", "forward", "forward_rows", "backward", "backward_dq_rows",
    "backward_dkdv_keys", "pair_count", "block_layout", "kernel_maps", "summary_offsets",
]
