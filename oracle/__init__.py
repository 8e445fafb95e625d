"""fp64 CPU oracle for factorized sparse self-attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the HIP
library under ``factorized_sparse_self_amd/`` and neither imports the other.
"""
from .sparse_attention import (DENSE, FIXED, FIXED_R1, STRIDED, backward, backward_dkdv_keys,
                               backward_dq_rows, forward, forward_rows, head_kind, in_key_set,
                               key_set, pair_count, queries_of_key)
from .block_layout import block_layout, kernel_maps

__all__ = [
    "STRIDED", "FIXED", "FIXED_R1", "DENSE", "head_kind", "key_set", "in_key_set",
    "queries_of_key", "forward", "forward_rows", "backward", "backward_dq_rows",
    "backward_dkdv_keys", "pair_count", "block_layout", "kernel_maps",
]
