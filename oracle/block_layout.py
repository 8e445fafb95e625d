"""Oracle derivation of the block look-up tables (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.

The pages state that the per-query key indices are precomputed and that the
attention runs as a block-sparse product over the non-empty blocks only
(llm-arch-kb "Sparse Transformer", §2 "Per-layer cost" and §3 Reference
implementation).  The library does this in its own coordinate system, where
each head kind's rows and keys are re-indexed so that its non-zeros fall into
dense blocks.  This module restates that coordinate system as plain
definitions, enumerates every (query, key) pair from
:func:`oracle.sparse_attention.part_key_set` (the head kind's set, or one
pass's part of a merged head's set), maps both ends into kernel
coordinates and counts the pairs that land in each (row block, key block).

Kernel coordinates for one head kind with block size ``bs``:

* rows: kernel row R holds query position ``row_pos[R]`` (-1 = padding);
* keys: kernel key K holds key position ``key_pos[K]`` (-1 = padding).

The maps:

* identity (strided kind 0, fixed kinds 0, dense): R = t and K = j.
* strided kind 1, residue-major: the positions t = m*l + r of residue class
  r = t mod l become the contiguous run R = r*n_pad + m, with n = ceil(T/l)
  and n_pad = n rounded up to a multiple of ``bs // 2`` (a block then holds
  one class, or the end of one class and the start of the next); rows and
  keys share the map.  The strided set of t is then the class-r prefix
  m' <= m.
* fixed kind 1, compacted summary keys: K = b*c + o holds position
  b*l + S[o], S the sorted summary offsets (c = |S|; for the default set the
  last c offsets, b*l + (l - c) + o).  Under the strictly-earlier-block reading (FIXED) only
  blocks 0 .. nb-2 (nb = ceil(T/l)) appear, since the last block's summary
  keys have no later query; under FIXED_R1 all nb blocks appear and
  positions >= T are padding.  Rows are the identity.

A block pair with count 0 is absent; count == bs*bs is FULL (flag 1, which
also implies every row and key of the pair is real); anything else is PARTIAL
(flag 0).  The CSR lists pairs by (row block, key block), the CSC by
(key block, row block).
"""
from __future__ import annotations

import numpy as np

from .sparse_attention import DENSE, FIXED, FIXED_R1, STRIDED, UNION_BASE, part_key_set, summary_offsets


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def kernel_maps(pattern: int, kind: int, T: int, l: int, c: int, bs: int):
    """(row_pos, key_pos): int64 arrays mapping kernel rows / keys to positions.

    A merged-head pattern's two passes use the maps of its base pattern's two
    kinds."""
    pattern = UNION_BASE.get(pattern, pattern)
    identity = np.arange(T, dtype=np.int64)
    if pattern == STRIDED and kind == 1:
        n = _ceil_div(T, l)
        gran = max(1, bs // 2)
        n_pad = _ceil_div(n, gran) * gran
        n_cls = min(l, T)
        rows = np.full(n_cls * n_pad, -1, dtype=np.int64)
        for r in range(n_cls):
            for m in range(n_pad):
                t = m * l + r
                if t < T:
                    rows[r * n_pad + m] = t
        return rows, rows.copy()
    if pattern in (FIXED, FIXED_R1) and kind == 1:
        nb = _ceil_div(T, l)
        n_blocks = nb - 1 if pattern == FIXED else nb
        S = summary_offsets(l, c)
        keys = []
        for b in range(n_blocks):
            for o in range(len(S)):
                j = b * l + int(S[o])
                keys.append(j if j < T else -1)
        return identity, np.asarray(keys, dtype=np.int64)
    if pattern in (STRIDED, FIXED, FIXED_R1, DENSE):
        return identity, identity.copy()
    raise ValueError(f"unknown pattern {pattern}")


def block_layout(pattern: int, kind: int, T: int, l: int, c: int, bs: int) -> dict:
    """Block LUT of one head kind, derived by counting enumerated pairs."""
    row_pos, key_pos = kernel_maps(pattern, kind, T, l, c, bs)
    key_of_pos = np.full(T, -1, dtype=np.int64)
    real = key_pos >= 0
    key_of_pos[key_pos[real]] = np.nonzero(real)[0]
    n_qb = _ceil_div(len(row_pos), bs)
    n_kb = _ceil_div(len(key_pos), bs)
    counts: dict[tuple[int, int], int] = {}
    for R, t in enumerate(row_pos):
        if t < 0:
            continue
        S = part_key_set(pattern, kind, int(t), T, l, c)
        K = key_of_pos[S]
        if (K < 0).any():
            raise AssertionError("a key of the pattern has no kernel coordinate")
        kbs, n = np.unique(K // bs, return_counts=True)
        qb = R // bs
        for kb, cnt in zip(kbs.tolist(), n.tolist()):
            counts[(qb, kb)] = counts.get((qb, kb), 0) + cnt
    pairs = sorted(counts)
    row_ptr = np.zeros(n_qb + 1, dtype=np.int32)
    for qb, _ in pairs:
        row_ptr[qb + 1] += 1
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    col_idx = np.asarray([kb for _, kb in pairs], dtype=np.int32)
    flags = np.asarray([1 if counts[p] == bs * bs else 0 for p in pairs], dtype=np.uint8)
    pairs_t = sorted(pairs, key=lambda p: (p[1], p[0]))
    col_ptr = np.zeros(n_kb + 1, dtype=np.int32)
    for _, kb in pairs_t:
        col_ptr[kb + 1] += 1
    col_ptr = np.cumsum(col_ptr).astype(np.int32)
    row_idx = np.asarray([qb for qb, _ in pairs_t], dtype=np.int32)
    csc_flags = np.asarray([1 if counts[p] == bs * bs else 0 for p in pairs_t], dtype=np.uint8)
    return {
        "block": bs, "n_rows": len(row_pos), "n_keys": len(key_pos),
        "n_qb": n_qb, "n_kb": n_kb, "nnz": len(pairs),
        "row_pos": row_pos.astype(np.int32), "key_pos": key_pos.astype(np.int32),
        "row_ptr": row_ptr, "col_idx": col_idx, "flags": flags,
        "col_ptr": col_ptr, "row_idx": row_idx, "csc_flags": csc_flags,
        "pair_count": int(sum(counts.values())),
    }
