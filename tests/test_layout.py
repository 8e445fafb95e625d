"""st_layout_build (C++ host builder) against the oracle's LUT derivation, bit-exact.

The library enumerates block pairs from closed-form per-row key runs; the
oracle counts enumerated (query, key) pairs.  Maps, CSR, CSC, flags, block
counts and total pair counts must agree exactly.  Host code only: no GPU.
"""
import os

import numpy as np
import pytest

import oracle
from factorized_sparse_self_amd import inputs

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "factorized_sparse_self_amd", "libst.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libst.so not built")

CASES = [(w.pattern, w.T, w.l, w.c) for w in inputs.WORKLOADS] + [
    (inputs.STRIDED, 250, 16, 0), (inputs.FIXED, 250, 16, 3), (inputs.FIXED, 333, 20, 20),
    (inputs.STRIDED, 100, 128, 0), (inputs.FIXED, 60, 64, 4), (inputs.FIXED, 1, 1, 1),
    (inputs.STRIDED, 1, 5, 0), (inputs.STRIDED, 129, 1, 0), (inputs.FIXED_R1, 250, 16, 3),
    (inputs.FIXED_R1, 1024, 32, 4), (inputs.DENSE, 300, 16, 0), (inputs.STRIDED, 1000, 96, 0),
    (inputs.STRIDED_UNION, 250, 16, 0), (inputs.STRIDED_UNION, 12288, 128, 0), (inputs.STRIDED_UNION, 129, 1, 0),
    (inputs.STRIDED_UNION, 1, 5, 0), (inputs.STRIDED_UNION, 1000, 96, 0), (inputs.FIXED_UNION, 250, 16, 3),
    (inputs.FIXED_UNION, 12288, 128, 8), (inputs.FIXED_UNION, 333, 20, 20), (inputs.FIXED_UNION, 1, 1, 1),
    # general summary sets (offsets within each l-block)
    (inputs.FIXED, 250, 16, (0, 5, 9)), (inputs.FIXED, 12288, 128, tuple(range(0, 128, 16))),
    (inputs.FIXED, 300, 20, (0, 7, 19)), (inputs.FIXED_R1, 250, 16, (2, 15)), (inputs.FIXED_R1, 300, 20, (0,)),
    (inputs.FIXED_R1, 1000, 96, (1, 2, 50, 95)), (inputs.FIXED_UNION, 256, 32, (0, 31)),
]


@pytest.mark.parametrize("pattern,T,l,c", CASES)
def test_layout_bit_exact(pattern, T, l, c):
    from factorized_sparse_self_amd import st_block_size, st_layout_build
    bs = st_block_size()
    assert bs == 64
    got = st_layout_build(pattern, T, l, c)
    for kind in (0, 1):
        ref = oracle.block_layout(pattern, kind, T, l, c, bs)
        g = got[kind]
        for key in ("n_rows", "n_keys", "n_qb", "n_kb", "nnz"):
            assert g[key] == ref[key], (kind, key)
        assert g["pairs"] == ref["pair_count"], kind
        for key in ("row_pos", "key_pos", "row_ptr", "col_idx", "flags", "col_ptr", "row_idx", "csc_flags"):
            np.testing.assert_array_equal(g[key], ref[key], err_msg=f"kind {kind} {key}")


def test_layout_block_counts_of_the_workloads():
    """Non-empty block pairs at block size 64 for the 12288-long workloads."""
    from factorized_sparse_self_amd import st_layout_build
    strided = st_layout_build(inputs.STRIDED, 12288, 128, 0)
    assert strided[0]["nnz"] == 573 and int(strided[0]["flags"].sum()) == 191
    # strided kind 1: 128 residue classes of 96 positions, packed back to back (four
    # classes fill six row blocks, with 10 block pairs: 1, 2, 2, 1, 2, 2)
    assert strided[1]["n_rows"] == 128 * 96 and strided[1]["nnz"] == 32 * 10
    assert int(strided[1]["flags"].sum()) == 0  # no block is all one class and causal-free
    fixed = st_layout_build(inputs.FIXED, 12288, 128, 8)
    assert fixed[0]["nnz"] == 288 and int(fixed[0]["flags"].sum()) == 96
    assert fixed[1]["nnz"] == 1224 and int(fixed[1]["flags"].sum()) == 1056


def test_explicit_tail_summary_is_the_default_layout():
    from factorized_sparse_self_amd import st_layout_build
    a = st_layout_build(inputs.FIXED_R1, 250, 16, 3)
    b = st_layout_build(inputs.FIXED_R1, 250, 16, (13, 14, 15))
    for kind in (0, 1):
        for key in a[kind]:
            np.testing.assert_array_equal(a[kind][key], b[kind][key])


@pytest.mark.parametrize("args", [(9, 100, 8, 2), (inputs.FIXED, 100, 8, 0), (inputs.FIXED, 100, 8, 9),
                                  (inputs.STRIDED, 0, 8, 0), (inputs.STRIDED, 100, 0, 0),
                                  (inputs.STRIDED, (1 << 24) + 1, 8, 0),
                                  (inputs.FIXED, 100, 8, (3, 2)), (inputs.FIXED, 100, 8, (1, 1)),
                                  (inputs.FIXED, 100, 8, (0, 8)), (inputs.FIXED_R1, 100, 8, (-1,)),
                                  (inputs.STRIDED, 100, 8, (1,)), (inputs.DENSE, 100, 8, (0,))])
def test_layout_rejects_bad_arguments(args):
    from factorized_sparse_self_amd import StError, st_layout_build
    with pytest.raises(StError) as e:
        st_layout_build(*args)
    assert e.value.status == -1
