"""Pins for the oracle's forward and backward values (CPU only).

* torch's scaled_dot_product_attention in fp64 with a dense boolean mask (the
  "masked logits are -inf before the softmax" statement of llm-arch-kb
  "Sparse Transformer", §2) and torch.autograd through it;
* central finite differences of L = <dO, O> in fp64;
* closed-form special cases: single-key rows, l >= T (local head = full causal
  attention), c = l (summary head = every earlier-block key);
* invariants: a constant added to every value shifts O by that constant, and a
  constant added to every key leaves O and dq unchanged.

The dense masks come from the recursive construction in
``test_oracle_sets.recursive_sets``, not from the oracle's own enumeration.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import DENSE, FIXED, FIXED_R1, FIXED_UNION, STRIDED, STRIDED_UNION, UNION_BASE
from tests.test_oracle_sets import recursive_sets


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def dense_masks(pattern, T, l, c, H):
    """One boolean [T, T] mask per head: kind h % 2's set, or the union of both for
    merged-head patterns."""
    k0, k1 = recursive_sets(UNION_BASE.get(pattern, pattern), T, l, c)
    masks = []
    for h in range(H):
        m = np.zeros((T, T), dtype=bool)
        for t in range(T):
            if pattern in UNION_BASE:
                keys = k0[t] | k1[t]
            else:
                keys = k0[t] if h % 2 == 0 else k1[t]
            m[t, sorted(keys)] = True
        masks.append(m)
    return masks


SMALL = [
    (STRIDED, 2, 3, 40, 5, 6, 0), (STRIDED, 1, 2, 33, 8, 4, 0),
    (FIXED, 2, 3, 40, 5, 6, 2), (FIXED, 1, 4, 37, 4, 5, 5),
    (FIXED_R1, 1, 2, 40, 3, 6, 2), (DENSE, 1, 2, 25, 4, 6, 0),
    (STRIDED_UNION, 1, 2, 40, 5, 6, 0), (FIXED_UNION, 2, 2, 37, 4, 5, 2),
    # general summary sets (offsets)
    (FIXED, 2, 3, 40, 5, 6, (0, 3)), (FIXED_R1, 1, 2, 40, 3, 6, (1, 4)), (FIXED_UNION, 1, 2, 37, 4, 5, (0, 2)),
]


@pytest.mark.parametrize("pattern,B,H,T,D,l,c", SMALL)
def test_forward_matches_torch_sdpa(pattern, B, H, T, D, l, c):
    q, k, v = (rand((B, H, T, D), s) for s in (1, 2, 3))
    O, lse = oracle.forward(q, k, v, pattern, l, c)
    masks = dense_masks(pattern, T, l, c, H)
    for h in range(H):
        m = masks[h]
        rows = np.nonzero(m.any(1))[0]
        empty = np.nonzero(~m.any(1))[0]
        qt = torch.from_numpy(q[:, h, rows])
        ref = F.scaled_dot_product_attention(qt, torch.from_numpy(k[:, h]), torch.from_numpy(v[:, h]),
                                             attn_mask=torch.from_numpy(m[rows]))
        np.testing.assert_allclose(O[:, h, rows], ref.numpy(), rtol=0, atol=1e-12)
        logits = (qt @ torch.from_numpy(k[:, h]).transpose(-1, -2)) / math.sqrt(D)
        logits = logits.masked_fill(~torch.from_numpy(m[rows]), -math.inf)
        np.testing.assert_allclose(lse[:, h, rows], torch.logsumexp(logits, -1).numpy(), rtol=0, atol=1e-12)
        assert (O[:, h, empty] == 0).all() and np.isneginf(lse[:, h, empty]).all()


@pytest.mark.parametrize("pattern,B,H,T,D,l,c", SMALL)
def test_backward_matches_torch_autograd(pattern, B, H, T, D, l, c):
    q, k, v, dO = (rand((B, H, T, D), s) for s in (4, 5, 6, 7))
    dq, dk, dv = oracle.backward(q, k, v, dO, pattern, l, c)
    masks = dense_masks(pattern, T, l, c, H)
    for h in range(H):
        m = masks[h]
        rows = np.nonzero(m.any(1))[0]
        qt = torch.from_numpy(q[:, h]).requires_grad_()
        kt = torch.from_numpy(k[:, h]).requires_grad_()
        vt = torch.from_numpy(v[:, h]).requires_grad_()
        out = F.scaled_dot_product_attention(qt[:, rows], kt, vt, attn_mask=torch.from_numpy(m[rows]))
        (out * torch.from_numpy(dO[:, h, rows])).sum().backward()
        np.testing.assert_allclose(dq[:, h], qt.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[:, h], kt.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[:, h], vt.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("pattern,T,l,c", [(STRIDED, 12, 4, 0), (STRIDED, 11, 3, 0),
                                           (FIXED, 12, 4, 2), (FIXED, 13, 3, 1), (FIXED_R1, 12, 4, 2),
                                           (STRIDED_UNION, 11, 3, 0), (FIXED_UNION, 12, 4, 2)])
def test_backward_finite_differences(pattern, T, l, c):
    B, H, D = 1, 2, 3
    q, k, v, dO = (rand((B, H, T, D), s) for s in (8, 9, 10, 11))
    dq, dk, dv = oracle.backward(q, k, v, dO, pattern, l, c)

    def loss(q_, k_, v_):
        O, _ = oracle.forward(q_, k_, v_, pattern, l, c)
        return float((O * dO).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos] = xp
            args_m[pos] = xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(g[idx])) + 1e-8, (name, idx, fd, g[idx])


@pytest.mark.parametrize("pattern,T,l,c", [(STRIDED_UNION, 40, 5, 0), (FIXED_UNION, 40, 5, 2),
                                           (STRIDED_UNION, 9, 16, 0)])
def test_union_is_the_lse_merge_of_its_parts(pattern, T, l, c):
    """Over a union of two disjoint parts, O = (e^lse0 O0 + e^lse1 O1) / (e^lse0 + e^lse1)
    and lse = log(e^lse0 + e^lse1), with O_p, lse_p the softmax over part p alone (an empty
    part has lse = -inf and drops out).  The parts' softmaxes are computed here with torch."""
    B, H, D = 1, 2, 4
    q, k, v = (rand((B, H, T, D), s) for s in (20, 21, 22))
    O, L = oracle.forward(q, k, v, pattern, l, c)
    for h in range(H):
        for t in range(T):
            parts = []
            for part in (0, 1):
                S = torch.from_numpy(oracle.part_key_set(pattern, part, t, T, l, c))
                if len(S) == 0:
                    parts.append((torch.zeros(D, dtype=torch.float64), -math.inf))
                    continue
                s_ = torch.from_numpy(k[0, h])[S] @ torch.from_numpy(q[0, h, t]) / math.sqrt(D)
                parts.append((torch.softmax(s_, 0) @ torch.from_numpy(v[0, h])[S], float(torch.logsumexp(s_, 0))))
            (o0, l0), (o1, l1) = parts
            lse = float(torch.logaddexp(torch.tensor(l0, dtype=torch.float64),
                                        torch.tensor(l1, dtype=torch.float64)))
            merged = math.exp(l0 - lse) * o0 + math.exp(l1 - lse) * o1
            np.testing.assert_allclose(O[0, h, t], merged.numpy(), rtol=0, atol=1e-13)
            assert L[0, h, t] == pytest.approx(lse, abs=1e-13)


def test_single_key_rows_are_exact():
    """A row with one key has p = 1: O_t = v_t and lse_t = q_t.k_t / sqrt(D), exactly."""
    B, H, T, D, l, c = 1, 2, 40, 8, 8, 2
    q, k, v = (rand((B, H, T, D), s) for s in (12, 13, 14))
    for pattern, kind, rows in ((STRIDED, 0, [0]), (STRIDED, 1, list(range(l))),
                                (FIXED, 0, list(range(0, T, l)))):
        O, lse = oracle.forward_rows(q, k, v, pattern, l, c, rows)
        h = kind
        for ri, t in enumerate(rows):
            assert np.array_equal(O[0, h, ri], v[0, h, t])
            assert lse[0, h, ri] == pytest.approx(float(q[0, h, t] @ k[0, h, t]) / math.sqrt(D), abs=1e-14)


def test_long_window_is_full_causal_attention():
    """With l >= T the local head (strided kind 0) and own-block head (fixed kind 0) see every
    earlier key: both equal full causal attention."""
    B, H, T, D = 2, 2, 30, 4
    q, k, v = (rand((B, H, T, D), s) for s in (15, 16, 17))
    Od, Ld = oracle.forward(q, k, v, DENSE, 8, 0)
    for pattern, c in ((STRIDED, 0), (FIXED, 1)):
        O, L = oracle.forward(q, k, v, pattern, T, c)
        np.testing.assert_allclose(O[:, 0], Od[:, 0], atol=1e-13, rtol=0)
        np.testing.assert_allclose(L[:, 0], Ld[:, 0], atol=1e-13, rtol=0)
    causal = np.tril(np.ones((T, T), dtype=bool))
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(causal))
    np.testing.assert_allclose(Od, ref.numpy(), atol=1e-12, rtol=0)


def test_full_summary_set_is_every_earlier_block_key():
    T, l = 24, 4
    for t in range(T):
        S = oracle.key_set(FIXED, 1, t, T, l, l)
        assert S.tolist() == list(range((t // l) * l))


def test_value_shift_and_key_shift_invariants():
    B, H, T, D, l, c = 1, 2, 36, 5, 6, 2
    q, k, v, dO = (rand((B, H, T, D), s) for s in (18, 19, 20, 21))
    u = rand((D,), 22)
    w = rand((D,), 23)
    for pattern in (STRIDED, FIXED):
        O, _ = oracle.forward(q, k, v, pattern, l, c)
        O2, _ = oracle.forward(q, k, v + u, pattern, l, c)
        _, L = oracle.forward(q, k, v, pattern, l, c)
        nonempty = np.isfinite(L)
        np.testing.assert_allclose(O2[nonempty], (O + u)[nonempty], atol=1e-12, rtol=0)
        dq, _, _ = oracle.backward(q, k, v, dO, pattern, l, c)
        dq2, _, _ = oracle.backward(q, k + w, v, dO, pattern, l, c)
        np.testing.assert_allclose(dq2, dq, atol=1e-11, rtol=0)


@pytest.mark.parametrize("pattern,l,c", [(STRIDED, 6, 0), (FIXED, 6, 2)])
def test_sampled_functions_equal_full_results(pattern, l, c):
    B, H, T, D = 2, 2, 40, 4
    q, k, v, dO = (rand((B, H, T, D), s) for s in (24, 25, 26, 27))
    O, L = oracle.forward(q, k, v, pattern, l, c)
    dq, dk, dv = oracle.backward(q, k, v, dO, pattern, l, c)
    rows = [0, 3, 7, 17, 39]
    Os, Ls = oracle.forward_rows(q, k, v, pattern, l, c, rows)
    np.testing.assert_array_equal(Os, O[:, :, rows])
    np.testing.assert_array_equal(Ls, L[:, :, rows])
    np.testing.assert_allclose(oracle.backward_dq_rows(q, k, v, dO, pattern, l, c, rows),
                               dq[:, :, rows], atol=1e-13, rtol=0)
    keys = [0, 4, 5, 11, 33, 39]
    dks, dvs = oracle.backward_dkdv_keys(q, k, v, dO, pattern, l, c, keys)
    np.testing.assert_allclose(dks, dk[:, :, keys], atol=1e-13, rtol=0)
    np.testing.assert_allclose(dvs, dv[:, :, keys], atol=1e-13, rtol=0)


@pytest.mark.parametrize("pattern,T,l,c", [(STRIDED, 23, 4, 0), (FIXED, 24, 4, 2), (FIXED_R1, 21, 5, 2),
                                           (FIXED_UNION, 20, 4, 2)])
def test_backward_given_forward_results(pattern, T, l, c):
    """The backward takes O and lse as its inputs.  Given the exact ones it is the default;
    Delta = dO . O enters linearly, so a change E of O moves dq_t by
    -(dO_t . E_t) sum_j p_tj k_j / sqrt(D), dk_j by -sum_t p_tj (dO_t . E_t) q_t / sqrt(D) and
    leaves dv; a shift d of every lse scales every weight, hence dq, dk, dv, by exp(-d).
    The row- and key-sampled variants agree with the full backward on the same inputs."""
    B, H, D = 1, 2, 5
    q, k, v, dO = (rand((B, H, T, D), s) for s in (30, 31, 32, 33))
    O, L = oracle.forward(q, k, v, pattern, l, c)
    ref = oracle.backward(q, k, v, dO, pattern, l, c)
    for a, b in zip(ref, oracle.backward(q, k, v, dO, pattern, l, c, O=O, lse=L)):
        np.testing.assert_array_equal(a, b)
    E = 1e-3 * rand((B, H, T, D), 34)
    dq2, dk2, dv2 = oracle.backward(q, k, v, dO, pattern, l, c, O=O + E, lse=L)
    scale = 1.0 / np.sqrt(D)
    want_dq = np.zeros_like(q)
    want_dk = np.zeros_like(k)
    for h in range(H):
        kind = oracle.head_kind(h)
        for t in range(T):
            S = oracle.key_set(pattern, kind, t, T, l, c)
            if S.size == 0:
                continue
            p = np.exp((k[0, h, S] @ q[0, h, t]) * scale - L[0, h, t])
            g = float(dO[0, h, t] @ E[0, h, t])
            want_dq[0, h, t] = -g * scale * (p @ k[0, h, S])
            want_dk[0, h, S] += -g * scale * np.outer(p, q[0, h, t])
    np.testing.assert_allclose(dq2 - ref[0], want_dq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk2 - ref[1], want_dk, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv2, ref[2], rtol=0, atol=1e-14)
    d = 0.3
    for a, b in zip(ref, oracle.backward(q, k, v, dO, pattern, l, c, O=O, lse=L + d)):
        np.testing.assert_allclose(b, np.exp(-d) * a, rtol=1e-12, atol=1e-14)
    Og, Lg = O + E, L + 0.01 * rand((B, H, T), 35)
    full = oracle.backward(q, k, v, dO, pattern, l, c, O=Og, lse=Lg)
    rows = np.array([0, 3, T // 2, T - 1])
    np.testing.assert_allclose(oracle.backward_dq_rows(q, k, v, dO, pattern, l, c, rows, O=Og, lse=Lg),
                               full[0][:, :, rows], rtol=1e-12, atol=1e-13)
    rk, rv = oracle.backward_dkdv_keys(q, k, v, dO, pattern, l, c, rows, O=Og, lse=Lg)
    np.testing.assert_allclose(rk, full[1][:, :, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rv, full[2][:, :, rows], rtol=1e-12, atol=1e-13)
