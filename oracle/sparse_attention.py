"""fp64 CPU oracle for factorized sparse causal self-attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and must never be used as a fallback for it.

What it computes is the plain definition, written out with an explicit
per-row gather over the key set S(t) and numpy fp64 arithmetic:

* The patterns.  llm-arch-kb "Sparse Transformer", §2 Derivation (Pattern A --
  strided, Pattern B -- fixed) and §3 Reference implementation (the mask
  sketch); nlp-lineage milestone page on the Sparse Transformer, section
  "The idea" (each pattern is split over two heads).
* The attention.  nlp-lineage, "The notation": a softmax of the scaled dot
  products q_t . k_j / sqrt(d) over j in S(t), weighting v_j; llm-arch-kb §2
  ("Sparse attention as an unnormalized form"): keys outside S(t) carry no
  probability mass.
* The backward.  The exact gradient of <dO, O> with respect to q, k and v; the
  attention weights are rebuilt from q, k and the row log-sum-exp, as the
  pages' recomputation strategy does (nlp-lineage, "The idea", recomputation).

Readings taken where the pages are silent, garbled or at odds (each is also
listed in the design notes):

R-heads   Factorised heads: head h uses sub-pattern ``h % 2``; kind 0 is the
          local / own-block set, kind 1 the strided / summary set.
R-self    The local window and the strided set both contain t itself
          (window [t-l+1, t]; strided t, t-l, t-2l, ...).
R-summary The summary set is a fixed set S of offsets within each l-block
          (llm-arch-kb §2, Pattern B; the §3 sketch takes it as an argument).
          Everywhere a pattern takes ``c``, ``c`` is either the count |S| with
          S the last c offsets (nlp-lineage, "The idea": summary positions at
          the end of each block) or the offsets of S themselves (a sequence).
          Fixed kind 1 (pattern FIXED) uses summary keys of strictly earlier
          blocks only.  FIXED_R1 also admits own-block summary keys j <= t,
          which is what the mask sketch's loop over ``block + 1`` blocks does.
R-empty   A row with an empty key set (fixed kind 1, first block) has O = 0 and
          lse = -inf, and contributes nothing to any gradient.
R-scale   d is the head dimension D; lse is the natural log of the sum of
          exp(scaled logits).
R-index   Positions are 0-based; T need not be a multiple of l.
DENSE     Full causal attention S(t) = {j <= t} (nlp-lineage, "The notation"),
          used as the dense comparator and as a special case.
UNION     Merged heads (STRIDED_UNION, FIXED_UNION): every head attends the
          union of the pattern's two sets, as llm-arch-kb §2 states each
          pattern and as its §3 mask sketch builds one mask from both loops.
          For the fixed pattern the union is the same under either summary
          reading (own-block summary keys <= t are already in the own block).

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (mask description, closed-form counts, causality,
two-hop reachability, torch SDPA in fp64 with autograd, finite differences,
single-key rows).
"""
from __future__ import annotations

import math

import numpy as np

STRIDED, FIXED, FIXED_R1, DENSE, STRIDED_UNION, FIXED_UNION = 0, 1, 2, 3, 4, 5
UNION_BASE = {STRIDED_UNION: STRIDED, FIXED_UNION: FIXED}


def head_kind(h: int) -> int:
    """Sub-pattern used by head h (reading R-heads)."""
    return h % 2


def summary_offsets(l: int, c) -> np.ndarray:
    """The summary set S as sorted offsets in [0, l) (reading R-summary): the
    last ``c`` offsets for an integer ``c``, else the given offsets."""
    if isinstance(c, (int, np.integer)):
        return np.arange(l - int(c), l, dtype=np.int64)
    S = np.asarray(sorted(int(o) for o in c), dtype=np.int64)
    if S.size == 0 or S[0] < 0 or S[-1] >= l or np.unique(S).size != S.size:
        raise ValueError("summary offsets must be distinct and in [0, l)")
    return S


# --------------------------------------------------------------------------
# Key sets
# --------------------------------------------------------------------------

def key_set(pattern: int, kind: int, t: int, T: int, l: int, c: int) -> np.ndarray:
    """Sorted key positions S(t) of one query, enumerated from the set definitions.

    llm-arch-kb §2 Derivation: Pattern A (strided) = A1 (the last l positions)
    and A2 (every l-th position counting back from t); Pattern B (fixed) = B1
    (the l-block holding t, up to t) and B2 (the summary offsets of the
    blocks before t's block).
    """
    if not 0 <= t < T:
        raise ValueError("query position out of range")
    if pattern in UNION_BASE:
        # merged heads: the union of both sets, whatever the head (reading UNION)
        base = UNION_BASE[pattern]
        return np.union1d(key_set(base, 0, t, T, l, c), key_set(base, 1, t, T, l, c))
    if pattern == STRIDED:
        if kind == 0:
            return np.arange(max(0, t - l + 1), t + 1, dtype=np.int64)
        return np.arange(t % l, t + 1, l, dtype=np.int64)
    if pattern in (FIXED, FIXED_R1):
        blk = t // l
        if kind == 0:
            return np.arange(blk * l, t + 1, dtype=np.int64)
        last_block = blk - 1 if pattern == FIXED else blk
        # the summary offsets of blocks 0 .. last_block, block by block
        starts = np.arange(last_block + 1, dtype=np.int64)[:, None] * l
        keys = (starts + summary_offsets(l, c)[None, :]).ravel()
        return keys[keys <= t]
    if pattern == DENSE:
        return np.arange(0, t + 1, dtype=np.int64)
    raise ValueError(f"unknown pattern {pattern}")


def in_key_set(pattern: int, kind: int, t, j, l: int, c: int) -> np.ndarray:
    """Membership test j in S(t), elementwise with numpy broadcasting.

    The same sets as :func:`key_set`, stated as predicates; used to find every
    query that attends a given key (for dk / dv at sampled keys).
    """
    t = np.asarray(t, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    if pattern in UNION_BASE:
        base = UNION_BASE[pattern]
        return in_key_set(base, 0, t, j, l, c) | in_key_set(base, 1, t, j, l, c)
    causal = (j >= 0) & (j <= t)
    if pattern == STRIDED:
        if kind == 0:
            return causal & (t - j < l)
        return causal & ((t - j) % l == 0)
    if pattern in (FIXED, FIXED_R1):
        if kind == 0:
            return causal & (j // l == t // l)
        summary = np.isin(j % l, summary_offsets(l, c))
        if pattern == FIXED:
            return (j >= 0) & summary & (j // l < t // l)
        return causal & summary
    if pattern == DENSE:
        return causal
    raise ValueError(f"unknown pattern {pattern}")


def part_key_set(pattern: int, part: int, t: int, T: int, l: int, c: int) -> np.ndarray:
    """The part (0 or 1) of S(t) that one head kind, or one pass over a merged
    head, covers.

    Factorised patterns: the set of head kind ``part``.  Merged heads: the two
    sets of the base pattern made disjoint, so that the union splits into two
    parts whose softmaxes merge exactly by their log-sum-exps.  The strided
    set loses t itself (already in the local window); the fixed sets are
    disjoint already (own block vs earlier blocks).
    """
    if pattern in UNION_BASE:
        base = UNION_BASE[pattern]
        S = key_set(base, part, t, T, l, c)
        return S[S != t] if (base == STRIDED and part == 1) else S
    return key_set(pattern, part, t, T, l, c)


def queries_of_key(pattern: int, kind: int, j: int, T: int, l: int, c: int) -> np.ndarray:
    """Every query position t whose key set holds j."""
    t = np.arange(T, dtype=np.int64)
    return np.nonzero(in_key_set(pattern, kind, t, j, l, c))[0]


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def _attend_row(qt: np.ndarray, Ks: np.ndarray, Vs: np.ndarray, scale: float):
    """One query over its gathered keys: (o, lse, p) in fp64 (nlp-lineage, "The notation")."""
    s = (Ks @ qt) * scale
    m = s.max()
    lse = m + math.log(np.exp(s - m).sum())
    p = np.exp(s - lse)
    return p @ Vs, lse, p


def _heads(H, heads):
    return range(H) if heads is None else [int(h) for h in heads]


def forward_rows(q, k, v, pattern, l, c, rows=None, heads=None):
    """Attention output and row log-sum-exp for the given query positions.

    q, k, v: float64 arrays [B, H, T, D].  ``rows`` is an iterable of query
    positions (all positions when None); ``heads`` restricts the heads that
    are computed (the others stay 0 / -inf).  Returns (O [B, H, R, D],
    lse [B, H, R]).  Empty key sets give O = 0, lse = -inf (reading R-empty).
    """
    B, H, T, D = q.shape
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = 1.0 / math.sqrt(D)
    O = np.zeros((B, H, len(rows), D), dtype=np.float64)
    lse = np.full((B, H, len(rows)), -np.inf, dtype=np.float64)
    for h in _heads(H, heads):
        kind = head_kind(h)
        for ri, t in enumerate(rows):
            S = key_set(pattern, kind, int(t), T, l, c)
            if S.size == 0:
                continue
            for b in range(B):
                o, m, _ = _attend_row(q[b, h, t], k[b, h, S], v[b, h, S], scale)
                O[b, h, ri] = o
                lse[b, h, ri] = m
    return O, lse


def forward(q, k, v, pattern, l, c):
    """Full forward: O [B, H, T, D] and lse [B, H, T]."""
    return forward_rows(q, k, v, pattern, l, c, None)


# --------------------------------------------------------------------------
# Backward (weights recomputed from q, k and lse)
# --------------------------------------------------------------------------

def _given_or_forward(q, k, v, pattern, l, c, O, lse):
    """The forward's output and lse as a backward receives them; exact when not given."""
    if O is None or lse is None:
        O2, lse2 = forward(q, k, v, pattern, l, c)
        O = O2 if O is None else O
        lse = lse2 if lse is None else lse
    return O, lse


def backward(q, k, v, dO, pattern, l, c, O=None, lse=None):
    """Gradients (dq, dk, dv) of L = <dO, O>, all float64 [B, H, T, D].

    For each query t with keys S(t): p_j = exp(s_j - lse_t) is recomputed,
    Delta_t = dO_t . O_t, dp_j = dO_t . v_j, ds_j = p_j (dp_j - Delta_t); then
    dv_j += p_j dO_t, dq_t = sum_j ds_j k_j / sqrt(D), dk_j += ds_j q_t / sqrt(D).
    O [B, H, T, D] and lse [B, H, T] are the forward results the backward
    receives (nlp-lineage, "The idea": the weights are rebuilt from the stored
    row statistics); when not given they are computed exactly here.
    """
    B, H, T, D = q.shape
    scale = 1.0 / math.sqrt(D)
    O, lse = _given_or_forward(q, k, v, pattern, l, c, O, lse)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(H):
        kind = head_kind(h)
        for t in range(T):
            S = key_set(pattern, kind, t, T, l, c)
            if S.size == 0:
                continue
            for b in range(B):
                s = (k[b, h, S] @ q[b, h, t]) * scale
                p = np.exp(s - lse[b, h, t])
                delta = dO[b, h, t] @ O[b, h, t]
                dp = v[b, h, S] @ dO[b, h, t]
                ds = p * (dp - delta)
                dq[b, h, t] = scale * (ds @ k[b, h, S])
                dk[b, h, S] += scale * np.outer(ds, q[b, h, t])
                dv[b, h, S] += np.outer(p, dO[b, h, t])
    return dq, dk, dv


def _row_stats(q, k, v, b, h, t, S, scale, O, lse):
    """(o_t, p over S) of query t: exact, or from the given forward results."""
    if O is None or lse is None:
        o, _, p = _attend_row(q[b, h, t], k[b, h, S], v[b, h, S], scale)
    if O is not None:
        o = np.asarray(O[b, h, t], dtype=np.float64)
    if lse is not None:
        p = np.exp((k[b, h, S] @ q[b, h, t]) * scale - float(lse[b, h, t]))
    return o, p


def backward_dq_rows(q, k, v, dO, pattern, l, c, rows, heads=None, O=None, lse=None):
    """dq at the given query positions only: float64 [B, H, R, D].  O, lse: as in backward
    (full [B, H, T, ...] arrays indexed by position), recomputed per row when not given."""
    B, H, T, D = q.shape
    scale = 1.0 / math.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((B, H, len(rows), D), dtype=np.float64)
    for h in _heads(H, heads):
        kind = head_kind(h)
        for ri, t in enumerate(rows):
            S = key_set(pattern, kind, int(t), T, l, c)
            if S.size == 0:
                continue
            for b in range(B):
                o, p = _row_stats(q, k, v, b, h, int(t), S, scale, O, lse)
                delta = dO[b, h, t] @ o
                dp = v[b, h, S] @ dO[b, h, t]
                ds = p * (dp - delta)
                dq[b, h, ri] = scale * (ds @ k[b, h, S])
    return dq


def backward_dkdv_keys(q, k, v, dO, pattern, l, c, keys, heads=None, O=None, lse=None):
    """dk, dv at the given key positions only: two float64 arrays [B, H, K, D].

    Every query that attends a sampled key is recomputed in full (its own key
    set, softmax and Delta), so the result equals the full backward at j.
    O, lse: as in backward (used for those queries' Delta and weights when given).
    """
    B, H, T, D = q.shape
    scale = 1.0 / math.sqrt(D)
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((B, H, len(keys), D), dtype=np.float64)
    dv = np.zeros((B, H, len(keys), D), dtype=np.float64)
    for h in _heads(H, heads):
        kind = head_kind(h)
        for ki, j in enumerate(keys):
            for t in queries_of_key(pattern, kind, int(j), T, l, c):
                S = key_set(pattern, kind, int(t), T, l, c)
                pos = int(np.searchsorted(S, j))
                for b in range(B):
                    o, p = _row_stats(q, k, v, b, h, int(t), S, scale, O, lse)
                    delta = dO[b, h, t] @ o
                    dp_j = v[b, h, j] @ dO[b, h, t]
                    ds_j = p[pos] * (dp_j - delta)
                    dk[b, h, ki] += scale * ds_j * q[b, h, t]
                    dv[b, h, ki] += p[pos] * dO[b, h, t]
    return dk, dv


# --------------------------------------------------------------------------
# Counting helpers used by the cost accounting
# --------------------------------------------------------------------------

def pair_count(pattern: int, kind: int, T: int, l: int, c: int) -> int:
    """Number of (query, key) pairs of one head of the given kind: sum_t |S(t)|."""
    return int(sum(key_set(pattern, kind, t, T, l, c).size for t in range(T)))
