"""Pins for the oracle's key sets (CPU only).

The oracle enumerates S(t) from set definitions (ranges and residues).  These
tests hold it against formulations that do not share that arithmetic:

* recursive constructions written from the pages' prose (llm-arch-kb
  "Sparse Transformer", §2 Derivation and the §3 mask sketch; nlp-lineage,
  "The idea"): the window slides by one position per query, the strided set
  of t is {t} plus the strided set of t - l, the own-block set restarts at each
  block start, and the summary set grows by one block's summary offsets at
  each block start;
* the per-query key counts and the cost bounds that §2 prints;
* causality and two-hop reachability (§2 "Two-hop reachability").
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (DENSE, FIXED, FIXED_R1, FIXED_UNION, STRIDED, STRIDED_UNION, UNION_BASE,
                    in_key_set, key_set, pair_count, part_key_set, queries_of_key)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def recursive_sets(pattern, T, l, c):
    """Per-query key sets (kind 0, kind 1) built position by position from the prose.
    ``c``: the summary set's size (its last c offsets) or its offsets."""
    summary = set(range(l - c, l)) if isinstance(c, int) else set(c)
    k0, k1 = [], []
    for t in range(T):
        blk_start = (t // l) * l
        if pattern == STRIDED:
            # the most recent l positions: previous window, plus t, minus what fell out
            prev = k0[t - 1] if t else set()
            k0.append((prev | {t}) - {t - l})
            # every l-th position going back from t: t together with the set of t - l
            k1.append({t} | (k1[t - l] if t >= l else set()))
        elif pattern in (FIXED, FIXED_R1):
            # own block: restarts at each block boundary
            k0.append({t} | (k0[t - 1] if t != blk_start else set()))
            if pattern == FIXED:
                # earlier blocks' summary keys: at a block start, add the previous block's
                if t == 0:
                    k1.append(set())
                elif t == blk_start:
                    pb = blk_start - l
                    k1.append(k1[t - 1] | {pb + o for o in summary})
                else:
                    k1.append(set(k1[t - 1]))
            else:
                # summary keys of any block up to and including t's own, not past t
                k1.append((k1[t - 1] if t else set()) | ({t} if (t % l) in summary else set()))
        elif pattern == DENSE:
            k0.append({t} | (k0[t - 1] if t else set()))
            k1.append(set(k0[t]))
    return k0, k1


CASES = [
    (STRIDED, 64, 8, 0), (STRIDED, 50, 7, 0), (STRIDED, 20, 32, 0), (STRIDED, 33, 1, 0),
    (FIXED, 64, 8, 2), (FIXED, 50, 7, 3), (FIXED, 40, 8, 8), (FIXED, 20, 32, 4), (FIXED, 37, 5, 1),
    (FIXED_R1, 64, 8, 2), (FIXED_R1, 50, 7, 3), (FIXED_R1, 41, 8, 8),
    (DENSE, 30, 4, 0),
]
# general summary sets S (llm-arch-kb §2 Pattern B): given as offsets
SIGMA_CASES = [
    (FIXED, 64, 8, (0, 5)), (FIXED, 50, 7, (2,)), (FIXED, 40, 8, (0, 1, 2, 3, 4, 5, 6, 7)),
    (FIXED, 37, 5, (0, 4)), (FIXED_R1, 64, 8, (1, 3, 6)), (FIXED_R1, 41, 8, (0, 7)),
    (FIXED_R1, 50, 7, (3,)),
]


@pytest.mark.parametrize("pattern,T,l,c", CASES + SIGMA_CASES)
def test_key_sets_match_recursive_construction(pattern, T, l, c):
    k0, k1 = recursive_sets(pattern, T, l, c)
    for t in range(T):
        assert key_set(pattern, 0, t, T, l, c).tolist() == sorted(k0[t]), (t, 0)
        assert key_set(pattern, 1, t, T, l, c).tolist() == sorted(k1[t]), (t, 1)


# merged heads: every head attends the union of the pattern's two sets
UNION_CASES = [
    (STRIDED_UNION, 64, 8, 0), (STRIDED_UNION, 50, 7, 0), (STRIDED_UNION, 20, 32, 0), (STRIDED_UNION, 33, 1, 0),
    (FIXED_UNION, 64, 8, 2), (FIXED_UNION, 50, 7, 3), (FIXED_UNION, 40, 8, 8), (FIXED_UNION, 37, 5, 1),
    (FIXED_UNION, 64, 8, (0, 5)), (FIXED_UNION, 37, 5, (2,)),
]


@pytest.mark.parametrize("pattern,T,l,c", UNION_CASES)
def test_union_sets_match_recursive_construction(pattern, T, l, c):
    k0, k1 = recursive_sets(UNION_BASE[pattern], T, l, c)
    for t in range(T):
        for h in (0, 1):
            assert key_set(pattern, h, t, T, l, c).tolist() == sorted(k0[t] | k1[t]), (t, h)


@pytest.mark.parametrize("pattern,T,l,c", UNION_CASES)
def test_union_parts_split_the_union_disjointly(pattern, T, l, c):
    """The two passes of a merged head: part 0 is the local / own-block set, part 1 the
    strided set without t (already in the window) or the summary set; disjoint, and
    together the union."""
    k0, k1 = recursive_sets(UNION_BASE[pattern], T, l, c)
    for t in range(T):
        p0 = set(part_key_set(pattern, 0, t, T, l, c).tolist())
        p1 = set(part_key_set(pattern, 1, t, T, l, c).tolist())
        assert p0 == k0[t]
        assert p1 == (k1[t] - {t} if pattern == STRIDED_UNION else k1[t])
        assert not (p0 & p1)
        assert p0 | p1 == set(key_set(pattern, 0, t, T, l, c).tolist())


@pytest.mark.parametrize("T,l", [(256, 16), (250, 16), (1000, 31), (64, 64), (10, 16)])
def test_strided_union_counts_closed_form(T, l):
    """|A1 u A2| = min(l, t+1) + floor(t/l): the page's l + ceil(i/l) - 1, i = t+1, once t >= l-1."""
    for t in range(T):
        n = len(key_set(STRIDED_UNION, 0, t, T, l, 0))
        assert n == min(l, t + 1) + t // l
        if t >= l - 1:
            assert n == l + math.ceil((t + 1) / l) - 1


@pytest.mark.parametrize("T,l,c", [(256, 16, 4), (250, 16, 3), (1024, 32, 4), (96, 8, 8), (12, 16, 2)])
def test_fixed_union_counts_closed_form(T, l, c):
    """|B1 u B2| = (t mod l) + 1 + c*floor(t/l), within the page's bound l + c*ceil(i/l)."""
    for t in range(T):
        n = len(key_set(FIXED_UNION, 0, t, T, l, c))
        assert n == t % l + 1 + c * (t // l)
        assert n <= l + c * math.ceil((t + 1) / l)


@pytest.mark.parametrize("pattern,T,l,c", CASES + SIGMA_CASES + UNION_CASES)
def test_membership_predicate_agrees_with_enumeration(pattern, T, l, c):
    tt, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    for kind in (0, 1):
        dense = in_key_set(pattern, kind, tt, jj, l, c)
        for t in range(T):
            assert np.nonzero(dense[t])[0].tolist() == key_set(pattern, kind, t, T, l, c).tolist()
        for j in range(T):
            assert queries_of_key(pattern, kind, j, T, l, c).tolist() == np.nonzero(dense[:, j])[0].tolist()


def test_fixed_readings_union_equals_mask_sketch_union():
    """The mask sketch admits own-block summary keys; B1 already covers them, so the union
    of the two heads is the same under both readings of the summary head."""
    T, l, c = 70, 8, 3
    for t in range(T):
        u2 = set(key_set(FIXED, 0, t, T, l, c)) | set(key_set(FIXED, 1, t, T, l, c))
        u1 = set(key_set(FIXED_R1, 0, t, T, l, c)) | set(key_set(FIXED_R1, 1, t, T, l, c))
        assert u1 == u2


@pytest.mark.parametrize("T,l", [(256, 16), (250, 16), (1000, 31), (64, 64), (10, 16)])
def test_strided_counts_closed_form(T, l):
    """|A1_t| = min(l, t+1), |A2_t| = floor(t/l)+1, and they share exactly t; with i = t+1 the
    page's total |A1|+|A2|-1 ~ l + ceil(i/l) holds exactly as l + ceil(i/l) - 1 once t >= l-1."""
    for t in range(T):
        a1 = set(key_set(STRIDED, 0, t, T, l, 0))
        a2 = set(key_set(STRIDED, 1, t, T, l, 0))
        assert len(a1) == min(l, t + 1)
        assert len(a2) == t // l + 1
        assert a1 & a2 == {t}
        i = t + 1
        if t >= l - 1:
            assert len(a1) + len(a2) - 1 == l + math.ceil(i / l) - 1
        assert len(a1 | a2) <= l + math.ceil(i / l)


@pytest.mark.parametrize("T,l,c", [(256, 16, 4), (250, 16, 3), (1024, 32, 4), (96, 8, 8), (12, 16, 2)])
def test_fixed_counts_closed_form(T, l, c):
    """|B1_t| = (t mod l)+1 and |B2_t| = c*floor(t/l) (disjoint), within the page's
    bound l + c*ceil(i/l), i = t+1."""
    for t in range(T):
        b1 = set(key_set(FIXED, 0, t, T, l, c))
        b2 = set(key_set(FIXED, 1, t, T, l, c))
        assert len(b1) == t % l + 1
        assert len(b2) == c * (t // l)
        assert not (b1 & b2)
        assert len(b1) + len(b2) <= l + c * math.ceil((t + 1) / l)
        r1 = set(key_set(FIXED_R1, 1, t, T, l, c))
        assert len(b1 | r1) == len(b1) + len(b2)


@pytest.mark.parametrize("pattern,T,l,c", CASES + UNION_CASES)
def test_causality(pattern, T, l, c):
    for kind in (0, 1):
        for t in range(T):
            S = key_set(pattern, kind, t, T, l, c)
            assert (S <= t).all() and (S >= 0).all()
            assert len(set(S.tolist())) == S.size


@pytest.mark.parametrize("pattern,T,l,c", [(STRIDED, 256, 16, 0), (STRIDED, 250, 16, 0),
                                           (STRIDED, 100, 7, 0), (FIXED, 256, 16, 4),
                                           (FIXED, 250, 16, 3), (FIXED, 100, 7, 1),
                                           (FIXED_R1, 100, 7, 2)])
def test_two_hop_reachability(pattern, T, l, c):
    """Every k <= i is reached from i within two hops: directly through the local head, or
    through the strided / summary head to some j0 whose local head holds k."""
    local = [set(key_set(pattern, 0, t, T, l, c)) for t in range(T)]
    far = [set(key_set(pattern, 1, t, T, l, c)) for t in range(T)]
    for i in range(T):
        reach = set(local[i]) | far[i]
        for j0 in far[i]:
            reach |= local[j0]
        assert reach == set(range(i + 1)), i


def test_two_hop_explicit_hop_strided():
    """The hop the derivation intends: j0 = i - l*floor((i-k)/l) is in A2(i) and k is in A1(j0)."""
    T, l = 300, 12
    for i in range(T):
        a2 = set(key_set(STRIDED, 1, i, T, l, 0))
        for k in range(i + 1):
            j0 = i - l * ((i - k) // l)
            assert j0 in a2 and k in set(key_set(STRIDED, 0, j0, T, l, 0))


@pytest.mark.parametrize("T,l,c", [(256, 16, 4), (12288, 128, 8), (1024, 32, 4), (4096, 64, 1)])
def test_total_pair_counts(T, l, c):
    """Totals for T = n*l: A1 l(l+1)/2 + (T-l)l; A2 l*n(n+1)/2; B1 n*l(l+1)/2; B2 c*l*n(n-1)/2."""
    n = T // l
    assert T == n * l
    assert pair_count(STRIDED, 0, T, l, c) == l * (l + 1) // 2 + (T - l) * l
    assert pair_count(STRIDED, 1, T, l, c) == l * n * (n + 1) // 2
    assert pair_count(FIXED, 0, T, l, c) == n * l * (l + 1) // 2
    assert pair_count(FIXED, 1, T, l, c) == c * l * n * (n - 1) // 2


def test_page_cost_figures():
    """The §1 and §2 cost statements of llm-arch-kb "Sparse Transformer", stored with their
    citation in tests/golden/page_cost_figures.json."""
    with open(os.path.join(GOLDEN, "page_cost_figures.json")) as f:
        g = json.load(f)
    T = g["premise"]["T"]
    # dense logits per head per layer ~ 1.5e8 and ~36e9 per forward at 8 heads x 30 layers
    assert abs(T * T / g["premise"]["dense_logits_per_head_layer"] - 1) < 0.01
    per_fwd = T * T * g["premise"]["heads"] * g["premise"]["layers"]
    assert abs(per_fwd / g["premise"]["dense_logits_per_forward"] - 1) < 0.01
    # strided union total ~ T*l + T^2/(2l); fixed union total <= sum_i (l + c*ceil(i/l))
    for case in g["strided_cost"]:
        T, l = case["T"], case["l"]
        union = pair_count(STRIDED, 0, T, l, 0) + pair_count(STRIDED, 1, T, l, 0) - T
        approx = T * l + T * T / (2 * l)
        assert abs(union / approx - 1) < case["rel_tol"], (union, approx)
    for case in g["fixed_cost"]:
        T, l, c = case["T"], case["l"], case["c"]
        union = pair_count(FIXED, 0, T, l, c) + pair_count(FIXED, 1, T, l, c)
        bound = sum(l + c * math.ceil(i / l) for i in range(1, T + 1))
        assert case["min_fraction_of_bound"] * bound <= union <= bound


def test_summary_offsets_default_and_explicit_agree():
    """An integer c is the last c offsets; the same offsets given explicitly (in any
    order) give the same sets, and invalid offsets are refused."""
    from oracle import summary_offsets
    assert summary_offsets(8, 3).tolist() == [5, 6, 7]
    for pattern in (FIXED, FIXED_R1, FIXED_UNION):
        for t in range(50):
            for kind in (0, 1):
                assert (key_set(pattern, kind, t, 50, 8, 3).tolist()
                        == key_set(pattern, kind, t, 50, 8, (7, 5, 6)).tolist())
    for bad in ((8,), (-1,), (2, 2), ()):
        with pytest.raises(ValueError):
            summary_offsets(8, bad)


@pytest.mark.parametrize("T,l,S", [(64, 8, (0, 5)), (50, 7, (2,)), (41, 8, (0, 7)), (100, 16, (1, 4, 9))])
def test_general_summary_counts(T, l, S):
    """|B2(t)| = |S| * floor(t/l) under FIXED, plus #{s in S : s <= t mod l} under FIXED_R1."""
    for t in range(T):
        assert len(key_set(FIXED, 1, t, T, l, S)) == len(S) * (t // l)
        own = sum(1 for s in S if s <= t % l)
        assert len(key_set(FIXED_R1, 1, t, T, l, S)) == len(S) * (t // l) + own
