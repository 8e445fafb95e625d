"""Pins for the oracle's block LUT derivation (CPU only).

``oracle.block_layout`` counts enumerated (query, key) pairs per block.  Here the
same counts come from a dense boolean matrix in kernel coordinates, built with
the membership predicate and summed block-wise by a reshape, and the maps are
checked to be bijections onto the positions they claim.
"""
import numpy as np
import pytest

import oracle
from oracle import DENSE, FIXED, FIXED_R1, FIXED_UNION, STRIDED, STRIDED_UNION, UNION_BASE


def in_part(pattern, kind, t, j, l, c):
    """Membership in the set one LUT covers: the head kind's set, or for merged heads the
    base kind's set, without t itself on the strided pass (the window has it)."""
    if pattern in UNION_BASE:
        base = UNION_BASE[pattern]
        m = oracle.in_key_set(base, kind, t, j, l, c)
        return m & (t != j) if (base == STRIDED and kind == 1) else m
    return oracle.in_key_set(pattern, kind, t, j, l, c)


def brute_force_counts(pattern, kind, T, l, c, bs):
    rows, keys = oracle.kernel_maps(pattern, kind, T, l, c, bs)
    n_qb = -(-len(rows) // bs)
    n_kb = -(-len(keys) // bs)
    rp = np.full(n_qb * bs, -1)
    rp[:len(rows)] = rows
    kp = np.full(n_kb * bs, -1)
    kp[:len(keys)] = keys
    M = in_part(pattern, kind, rp[:, None], kp[None, :], l, c)
    M &= (rp[:, None] >= 0) & (kp[None, :] >= 0)
    return M.reshape(n_qb, bs, n_kb, bs).sum(axis=(1, 3))


CASES = [
    (STRIDED, 256, 16, 0, 16), (STRIDED, 256, 16, 0, 64), (STRIDED, 250, 16, 0, 32),
    (STRIDED, 300, 7, 0, 16), (STRIDED, 100, 128, 0, 64),
    (FIXED, 1024, 32, 4, 64), (FIXED, 250, 16, 3, 16), (FIXED, 333, 20, 20, 32),
    (FIXED, 60, 64, 4, 64), (FIXED_R1, 250, 16, 3, 16), (FIXED_R1, 256, 32, 4, 64),
    (DENSE, 200, 16, 0, 64),
    (STRIDED_UNION, 256, 16, 0, 64), (STRIDED_UNION, 300, 7, 0, 16),
    (FIXED_UNION, 250, 16, 3, 16), (FIXED_UNION, 1024, 32, 4, 64),
    (FIXED, 250, 16, (0, 5, 9), 16), (FIXED_R1, 250, 16, (2, 15), 64), (FIXED_UNION, 256, 32, (0, 31), 64),
    (FIXED, 300, 20, (1, 2, 3, 17), 32),
]


@pytest.mark.parametrize("pattern,T,l,c,bs", CASES)
def test_lut_matches_dense_block_sums(pattern, T, l, c, bs):
    if pattern in UNION_BASE:
        # the two passes of a merged head cover the union exactly once
        total = sum(oracle.block_layout(pattern, kind, T, l, c, bs)["pair_count"] for kind in (0, 1))
        assert total == oracle.pair_count(pattern, 0, T, l, c)
    for kind in (0, 1):
        lay = oracle.block_layout(pattern, kind, T, l, c, bs)
        counts = brute_force_counts(pattern, kind, T, l, c, bs)
        qb, kb = np.nonzero(counts)
        assert lay["nnz"] == len(qb)
        rp = lay["row_ptr"]
        for q in range(lay["n_qb"]):
            sel = qb == q
            assert lay["col_idx"][rp[q]:rp[q + 1]].tolist() == kb[sel].tolist()
            full = (counts[q, kb[sel]] == bs * bs).astype(np.uint8)
            assert lay["flags"][rp[q]:rp[q + 1]].tolist() == full.tolist()
        cp = lay["col_ptr"]
        for k in range(lay["n_kb"]):
            sel = kb == k
            assert lay["row_idx"][cp[k]:cp[k + 1]].tolist() == sorted(qb[sel].tolist())
        if pattern not in UNION_BASE:
            assert lay["pair_count"] == oracle.pair_count(pattern, kind, T, l, c)


@pytest.mark.parametrize("pattern,T,l,c,bs", CASES)
def test_maps_are_bijections(pattern, T, l, c, bs):
    for kind in (0, 1):
        rows, keys = oracle.kernel_maps(pattern, kind, T, l, c, bs)
        real_rows = rows[rows >= 0]
        assert sorted(real_rows.tolist()) == list(range(T))
        real_keys = keys[keys >= 0]
        assert len(set(real_keys.tolist())) == real_keys.size
        attended = set()
        for t in range(T):
            attended |= set(oracle.part_key_set(pattern, kind, t, T, l, c).tolist())
        assert attended <= set(real_keys.tolist())
        if UNION_BASE.get(pattern, pattern) == FIXED and kind == 1:
            nb = -(-T // l)
            offsets = range(l - c, l) if isinstance(c, int) else sorted(c)
            expect = [b * l + o for b in range(nb - 1) for o in offsets]
            assert real_keys.tolist() == expect
        if UNION_BASE.get(pattern, pattern) == STRIDED and kind == 1:
            # within a class the run is in increasing position order, l apart
            n_pad = len(rows) // min(l, T)
            assert n_pad % max(1, bs // 2) == 0 and n_pad - (-(-T // l)) < max(1, bs // 2)
            for r in range(min(l, T)):
                run = rows[r * n_pad:(r + 1) * n_pad]
                run = run[run >= 0]
                assert run.tolist() == list(range(r, T, l))
