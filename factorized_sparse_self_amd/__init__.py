"""Factorized sparse causal self-attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libst.so`` (hand-written HIP kernels behind the C ABI of
``include/st.h``); this package is its thin Python binding.  Importing the
package does not load the library; the first call does, and raises if it has
not been built (``python -m factorized_sparse_self_amd.build``).
"""
from ._lib import (EXPORTED, KERNEL_NAMES, ST_DENSE, ST_FIXED, ST_FIXED_R1, ST_FIXED_UNION, ST_STRIDED,
                   ST_STRIDED_UNION, StError,
                   lib, sparse_attention, st_block_size, st_layout_build, st_release, st_set_dkdv_keys_per_wave,
                   st_set_fwd_rows_per_wave,
                   st_sparse_attn_bwd, st_sparse_attn_bwd_noalloc, st_sparse_attn_fwd, st_timing_enable,
                   st_timing_read, st_timing_reset)

__all__ = [
    "EXPORTED", "ST_STRIDED", "ST_FIXED", "ST_FIXED_R1", "ST_DENSE", "ST_STRIDED_UNION",
    "ST_FIXED_UNION", "StError", "lib",
    "sparse_attention", "st_block_size", "st_layout_build", "st_release", "st_set_dkdv_keys_per_wave",
    "st_set_fwd_rows_per_wave",
    "st_sparse_attn_bwd", "st_sparse_attn_bwd_noalloc", "st_sparse_attn_fwd", "st_timing_enable", "st_timing_read",
    "st_timing_reset", "KERNEL_NAMES",
]
