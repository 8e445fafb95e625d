"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every comparison is end to end: the oracle computes its own fp64 forward (O and
lse) from q, k and v, and its own backward from q, k, v and dO alone, and the
library's out, lse, dq, dk and dv are held to it element by element.  The bound
is max |error| <= 2e-2 for bf16 and fp16 inputs and <= 1e-4 for fp32 inputs,
and 1e-4 for lse everywhere.  It is the bound itself wherever a result rounded
correctly to the output type can meet it; only where half an output ulp of the
exact value is larger than the bound (bf16 values of magnitude 8 or more, whose
spacing is 1/16) is that half ulp added.  Each check prints its worst ratio of
error to bound.

Rows with an empty key set must give out == 0 and lse == -inf exactly, single-
key rows out == v exactly, and keys nobody attends dk == dv == 0 exactly.

Small cases run the whole oracle and span several 64-row blocks with ragged
tails, hand-picked and seeded-random (pattern, dtype, D, T, l, summary set; a
second random set is long enough for split key columns); the workloads run at
their full sizes in the launch configuration the benchmark times, and are
compared on seeded samples of rows (out, lse, dq) and keys (dk, dv) that the
oracle computes one by one, as are the largest T and B*H the library accepts.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from factorized_sparse_self_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-4}
SIGNIFICAND_BITS = {"bf16": 8, "f16": 11, "f32": 24}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def allowed_error(ref, dtype):
    """The stated bound, widened by half an output ulp of the exact value only where
    that half ulp exceeds the bound: there even the correctly rounded result can miss
    the bound (a bf16 value in [8, 16) is a multiple of 1/16)."""
    mag = np.abs(np.where(np.isfinite(ref), ref, 0.0))
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    half_ulp = np.where(mag > 0, np.exp2(e - SIGNIFICAND_BITS[dtype]), 0.0)
    base = TOL[dtype]
    return np.where(half_ulp > base, base + half_ulp, base)


@pytest.fixture(autouse=True)
def _parity_record(request):
    """Name the running test for the per-test ratio record."""
    global _CURRENT
    _CURRENT = request.node.name
    yield
    _CURRENT = None


_CURRENT = None


def _record(what, ratio):
    import conftest
    if _CURRENT is None:
        return
    checks = conftest.PARITY_RATIOS.setdefault(_CURRENT, {})
    key = what.split()[0]
    checks[key] = max(checks.get(key, 0.0), ratio)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def assert_close(got, ref, dtype, what):
    """Element-by-element check against the bound; returns the worst error / bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = allowed_error(ref, dtype)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    ninf_g, ninf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf pattern differs ({ninf_g.sum()} vs {ninf_r.sum()})"
    fin = ~ninf_r
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite values"
    if not fin.any():
        return 0.0
    err = np.where(fin, np.abs(got - np.where(fin, ref, 0)), 0)
    ratio = err / tol
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    worst = np.unravel_index(int(np.argmax(ratio)), err.shape)
    mag = float(np.max(np.abs(np.where(fin, ref, 0))))
    print(f"  {what}: max abs err {err[i]:.3e} at {tuple(int(x) for x in i)} (got {got[i]:.6g}, "
          f"ref {ref[i]:.6g}); max |ref| {mag:.3g}; worst err/bound {ratio[worst]:.3f} "
          f"(ref {ref[worst]:.6g}); over bound: {int((ratio > 1).sum())}", flush=True)
    _record(what, float(ratio[worst]))
    assert ratio[worst] <= 1.0, (f"{what}: error {err[worst]:.3e} at {tuple(int(x) for x in worst)} "
                                 f"(ref {ref[worst]:.6g}) exceeds {tol[worst]:.3e}")
    return float(ratio[worst])


def run_fwd(q, k, v, pattern, l, c):
    from factorized_sparse_self_amd import st_sparse_attn_fwd
    out, lse = st_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), pattern, l, c)
    torch.cuda.synchronize()
    return out, lse


def run_bwd(q, k, v, out, lse, do, pattern, l, c):
    from factorized_sparse_self_amd import st_sparse_attn_bwd
    dq, dk, dv = st_sparse_attn_bwd(q.cuda(), k.cuda(), v.cuda(), out, lse, do.cuda(), pattern, l, c)
    torch.cuda.synchronize()
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Small cases: the whole oracle, several blocks, ragged tails
# ---------------------------------------------------------------------------

SMALL = [
    # pattern, B, H, T, D, l, c
    (inputs.STRIDED, 2, 3, 300, 64, 16, 0),
    (inputs.STRIDED, 1, 2, 333, 32, 20, 0),
    (inputs.STRIDED, 1, 2, 200, 64, 7, 0),
    (inputs.STRIDED, 1, 4, 190, 64, 96, 0),
    (inputs.FIXED, 2, 3, 300, 64, 16, 3),
    (inputs.FIXED, 1, 2, 333, 32, 20, 20),
    (inputs.FIXED, 1, 2, 250, 64, 64, 4),
    (inputs.FIXED, 1, 2, 260, 64, 5, 1),
    (inputs.FIXED_R1, 1, 2, 300, 64, 16, 3),
    # l = 128 (the benchmark's fixed configuration) at a size the oracle runs whole
    (inputs.FIXED, 1, 2, 300, 64, 128, 8),
    (inputs.FIXED_R1, 2, 2, 390, 32, 128, 4),
    (inputs.DENSE, 1, 2, 200, 64, 16, 0),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"p{c[0]}_B{c[1]}H{c[2]}T{c[3]}D{c[4]}l{c[5]}c{c[6]}")
def test_small_forward_backward(case, dtype):
    pattern, B, H, T, D, l, c = case
    log(f"small fwd+bwd {case} {dtype}")
    tdt = TORCH_DTYPE[dtype]
    q, k, v, do = inputs.draw(B, H, T, D, dtype=tdt, seed=7 + T + l, n=4)
    out, lse = run_fwd(q, k, v, pattern, l, c)
    qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
    O, L = oracle.forward(qn, kn, vn, pattern, l, c)
    assert_close(f64(out), O, dtype, "out")
    assert_close(f64(lse), L, "f32", "lse")
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, pattern, l, c)
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
    assert_close(f64(dq), rq, dtype, "dq")
    assert_close(f64(dk), rk, dtype, "dk")
    assert_close(f64(dv), rv, dtype, "dv")


# Merged heads (every head attends both sets)
SMALL_UNION = [
    (inputs.STRIDED_UNION, 2, 3, 300, 64, 16, 0),
    (inputs.STRIDED_UNION, 1, 2, 333, 32, 20, 0),
    (inputs.STRIDED_UNION, 1, 2, 200, 64, 7, 0),
    (inputs.STRIDED_UNION, 1, 2, 190, 64, 96, 0),
    (inputs.STRIDED_UNION, 1, 2, 130, 64, 1, 0),
    (inputs.STRIDED_UNION, 1, 3, 10, 64, 16, 0),
    (inputs.STRIDED_UNION, 1, 1, 1, 64, 4, 0),
    (inputs.FIXED_UNION, 2, 3, 300, 64, 16, 3),
    (inputs.FIXED_UNION, 1, 2, 333, 32, 20, 20),
    (inputs.FIXED_UNION, 1, 2, 250, 64, 64, 4),
    (inputs.FIXED_UNION, 1, 2, 260, 64, 5, 1),
    (inputs.FIXED_UNION, 1, 3, 10, 64, 16, 3),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", SMALL_UNION, ids=lambda c: f"p{c[0]}_B{c[1]}H{c[2]}T{c[3]}D{c[4]}l{c[5]}c{c[6]}")
def test_small_merged_heads(case, dtype):
    pattern, B, H, T, D, l, c = case
    log(f"small merged heads fwd+bwd {case} {dtype}")
    q, k, v, do = inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=17 + T + l, n=4)
    out, lse = run_fwd(q, k, v, pattern, l, c)
    qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
    O, L = oracle.forward(qn, kn, vn, pattern, l, c)
    assert_close(f64(out), O, dtype, "out")
    assert_close(f64(lse), L, "f32", "lse")
    # position 0 attends only itself in both sets: out == v exactly
    assert torch.equal(out[:, :, 0].cpu(), v[:, :, 0])
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, pattern, l, c)
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
    assert_close(f64(dq), rq, dtype, "dq")
    assert_close(f64(dk), rk, dtype, "dk")
    assert_close(f64(dv), rv, dtype, "dv")


# General summary sets (offsets within each l-block) for the fixed patterns
SMALL_SIGMA = [
    (inputs.FIXED, 2, 3, 300, 64, 16, (0, 5, 9)),
    (inputs.FIXED, 1, 2, 333, 32, 20, (0, 7, 19)),
    (inputs.FIXED_R1, 1, 2, 300, 64, 16, (2, 15)),
    (inputs.FIXED_R1, 1, 2, 260, 64, 5, (0,)),
    (inputs.FIXED_UNION, 1, 2, 250, 64, 32, (0, 31)),
    (inputs.FIXED_UNION, 1, 3, 200, 64, 16, (3, 4, 8, 12)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", SMALL_SIGMA, ids=lambda c: f"p{c[0]}_H{c[2]}T{c[3]}D{c[4]}l{c[5]}S{'-'.join(map(str, c[6]))}")
def test_small_summary_sets(case, dtype):
    pattern, B, H, T, D, l, S = case
    log(f"small summary set fwd+bwd {case} {dtype}")
    q, k, v, do = inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=23 + T + l, n=4)
    out, lse = run_fwd(q, k, v, pattern, l, S)
    qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
    O, L = oracle.forward(qn, kn, vn, pattern, l, S)
    assert_close(f64(out), O, dtype, "out")
    assert_close(f64(lse), L, "f32", "lse")
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, pattern, l, S)
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, S)
    assert_close(f64(dq), rq, dtype, "dq")
    assert_close(f64(dk), rk, dtype, "dk")
    assert_close(f64(dv), rv, dtype, "dv")
    if pattern == inputs.FIXED:
        # summary heads: positions outside S, and the last block, are never attended
        pos = torch.arange(T)
        never = ~torch.isin(pos % l, torch.tensor(S)) | (pos >= (-(-T // l) - 1) * l)
        dkc, dvc = dk.cpu(), dv.cpu()
        assert (dkc[:, 1::2][:, :, never] == 0).all() and (dvc[:, 1::2][:, :, never] == 0).all()


def test_explicit_default_summary_set_matches_count():
    """The last c offsets given explicitly run the same plan: identical bits."""
    B, H, T, D, l, c = 1, 2, 300, 64, 16, 3
    q, k, v, do = inputs.draw(B, H, T, D, dtype=torch.bfloat16, seed=31, n=4)
    o1, l1 = run_fwd(q, k, v, inputs.FIXED_R1, l, c)
    o2, l2 = run_fwd(q, k, v, inputs.FIXED_R1, l, (13, 14, 15))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = run_bwd(q, k, v, o1, l1, do, inputs.FIXED_R1, l, c)
    g2 = run_bwd(q, k, v, o1, l1, do, inputs.FIXED_R1, l, (13, 14, 15))
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


# Head dimension 128
SMALL_D128 = [
    (inputs.STRIDED, 1, 2, 300, 128, 16, 0),
    (inputs.FIXED, 1, 3, 250, 128, 32, 4),
    (inputs.FIXED_R1, 1, 2, 200, 128, 16, (1, 9)),
    (inputs.DENSE, 1, 2, 130, 128, 16, 0),
    (inputs.STRIDED_UNION, 1, 2, 190, 128, 20, 0),
    (inputs.FIXED_UNION, 1, 2, 200, 128, 16, 3),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", SMALL_D128, ids=lambda c: f"p{c[0]}_H{c[2]}T{c[3]}l{c[5]}")
def test_small_head_dim_128(case, dtype):
    pattern, B, H, T, D, l, c = case
    log(f"small D=128 fwd+bwd {case} {dtype}")
    q, k, v, do = inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=41 + T + l, n=4)
    out, lse = run_fwd(q, k, v, pattern, l, c)
    qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
    O, L = oracle.forward(qn, kn, vn, pattern, l, c)
    assert_close(f64(out), O, dtype, "out")
    assert_close(f64(lse), L, "f32", "lse")
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, pattern, l, c)
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
    assert_close(f64(dq), rq, dtype, "dq")
    assert_close(f64(dk), rk, dtype, "dk")
    assert_close(f64(dv), rv, dtype, "dv")


def test_edge_shapes():
    """T = 1 (every pattern, every head dimension), T < l, l = 1, c = l, a single row
    block and one more row, odd H."""
    cases = [
        (inputs.STRIDED, 1, 2, 1, 64, 4, 0), (inputs.FIXED, 1, 2, 1, 64, 4, 2),
        (inputs.STRIDED, 1, 3, 10, 64, 16, 0), (inputs.FIXED, 1, 3, 10, 64, 16, 3),
        (inputs.STRIDED, 2, 2, 70, 32, 1, 0), (inputs.FIXED, 1, 2, 70, 64, 1, 1),
        (inputs.FIXED, 1, 5, 130, 64, 8, 8), (inputs.DENSE, 1, 1, 65, 64, 1, 0),
        # every pattern at T = 1, and the other head dimensions at T = 1 and at one block plus one row
        (inputs.FIXED_R1, 1, 2, 1, 64, 4, 2), (inputs.DENSE, 1, 2, 1, 64, 4, 0),
        (inputs.STRIDED_UNION, 1, 2, 1, 64, 4, 0), (inputs.FIXED_UNION, 1, 2, 1, 64, 4, 2),
        (inputs.STRIDED, 1, 2, 1, 32, 4, 0), (inputs.FIXED, 1, 2, 1, 128, 4, 2),
        (inputs.FIXED_R1, 1, 3, 65, 32, 16, 16), (inputs.STRIDED, 1, 2, 65, 128, 8, 0),
        # l larger than T for the merged heads (the second pass of the fixed head attends nothing)
        (inputs.FIXED_UNION, 1, 2, 40, 64, 64, 4), (inputs.STRIDED_UNION, 1, 2, 40, 64, 64, 0),
    ]
    for dtype in ("bf16", "f16", "f32"):
        tdt = TORCH_DTYPE[dtype]
        for pattern, B, H, T, D, l, c in cases:
            log(f"edge {pattern} B{B} H{H} T{T} D{D} l{l} c{c} {dtype}")
            q, k, v, do = inputs.draw(B, H, T, D, dtype=tdt, seed=99 + T, n=4)
            out, lse = run_fwd(q, k, v, pattern, l, c)
            qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
            O, L = oracle.forward(qn, kn, vn, pattern, l, c)
            assert_close(f64(out), O, dtype, "out")
            assert_close(f64(lse), L, "f32", "lse")
            dq, dk, dv = run_bwd(q, k, v, out, lse, do, pattern, l, c)
            rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
            assert_close(f64(dq), rq, dtype, "dq")
            assert_close(f64(dk), rk, dtype, "dk")
            assert_close(f64(dv), rv, dtype, "dv")


def _random_cases(n, seed):
    """n seeded random small problems: pattern, B, H, T, D, l, summary (a count or a set), dtype."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        pattern = int(rng.integers(0, 6))
        dtype = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
        D = [32, 64, 128][int(rng.integers(0, 3))]
        T = int(rng.integers(1, 420))
        l = int(rng.integers(1, 150))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        c = 0
        if pattern in (inputs.FIXED, inputs.FIXED_R1, inputs.FIXED_UNION):
            if rng.random() < 0.5:
                c = int(rng.integers(1, l + 1))
            else:
                k = int(rng.integers(1, l + 1))
                c = tuple(int(x) for x in sorted(rng.choice(l, size=k, replace=False)))
        cases.append((pattern, B, H, T, D, l, c, dtype))
    return cases


def test_summary_key_weight_rounding():
    """A bf16 case where a summary key's dv sums 145 rows' weights, most of them large
    (rows that see only four summary keys).  Rounding each weight to bf16 before the dV
    product moved dv[0, 1, 74, 23] by 0.029, past the bound (0.0278); the summary heads
    carry the weights to dV in two parts instead.  Found by the seeded random sweep."""
    _check_random((inputs.FIXED, 2, 3, 249, 32, 104, (13, 23, 74, 96), "bf16"))


def _random_long_cases(n, seed):
    """n seeded random problems long enough (T > 2048) that key columns of more than 32
    row blocks exist, so that dk/dv runs its split partials and reduction."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        pattern = [inputs.FIXED, inputs.FIXED_R1, inputs.DENSE, inputs.FIXED_UNION][int(rng.integers(0, 4))]
        T = int(rng.integers(2100, 3300))
        l = int(rng.integers(8, 130))
        c = int(rng.integers(1, l + 1)) if pattern != inputs.DENSE else 0
        dtype = ["bf16", "f32"][int(rng.integers(0, 2))]
        cases.append((pattern, 1, 2, T, 64, l, c, dtype))
    return cases


@pytest.mark.parametrize("case", _random_long_cases(6, 4711),
                         ids=lambda c: f"p{c[0]}_T{c[3]}l{c[5]}c{c[6]}_{c[7]}")
def test_random_long_shapes(case):
    """As test_random_shapes, at lengths where long key columns are split."""
    _check_random(case)


@pytest.mark.parametrize("case", _random_cases(100, 31337),
                         ids=lambda c: f"p{c[0]}_B{c[1]}H{c[2]}T{c[3]}D{c[4]}l{c[5]}_{c[7]}")
def test_random_shapes(case):
    """Seeded random patterns, dtypes, head dims, lengths, strides and summary sets (counts
    or explicit offsets), each against the whole oracle."""
    _check_random(case)


def _random_medium_cases(n, seed):
    """n seeded random problems between the small sweep and the split-column lengths
    (T from 420 to 2100), every pattern, dtype and head dimension."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        pattern = int(rng.integers(0, 6))
        dtype = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
        D = [32, 64, 128][int(rng.integers(0, 3))]
        T = int(rng.integers(420, 2100))
        l = int(rng.integers(1, 300))
        c = 0
        if pattern in (inputs.FIXED, inputs.FIXED_R1, inputs.FIXED_UNION):
            c = int(rng.integers(1, l + 1))
        cases.append((pattern, 1, int(rng.integers(1, 4)), T, D, l, c, dtype))
    return cases


@pytest.mark.parametrize("case", _random_medium_cases(30, 2718),
                         ids=lambda c: f"p{c[0]}_H{c[2]}T{c[3]}D{c[4]}l{c[5]}c{c[6]}_{c[7]}")
def test_random_medium_shapes(case):
    """As test_random_shapes, at lengths of several to thirty row-block pairs."""
    _check_random(case)


def _check_random(case):
    pattern, B, H, T, D, l, c, dtype = case
    log(f"random shape {case}")
    q, k, v, do = inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=T * 131 + l, n=4)
    out, lse = run_fwd(q, k, v, pattern, l, c)
    qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
    O, L = oracle.forward(qn, kn, vn, pattern, l, c)
    assert_close(f64(out), O, dtype, "out")
    assert_close(f64(lse), L, "f32", "lse")
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, pattern, l, c)
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
    assert_close(f64(dq), rq, dtype, "dq")
    assert_close(f64(dk), rk, dtype, "dk")
    assert_close(f64(dv), rv, dtype, "dv")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_special_rows(dtype):
    """Empty rows: out == 0, lse == -inf, dq == 0.  Single-key rows: out == v (the
    one weight is exactly 1).  Keys nobody attends: dk == dv == 0."""
    B, H, T, D, l, c = 1, 2, 256, 64, 32, 4
    q, k, v, do = inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=5, n=4)
    out, lse = run_fwd(q, k, v, inputs.FIXED, l, c)
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, inputs.FIXED, l, c)
    o, L, dq_, dk_, dv_ = (x.cpu() for x in (out, lse, dq, dk, dv))
    # head 1 (summary head), first block: empty key sets
    assert (o[0, 1, :l] == 0).all() and torch.isneginf(L[0, 1, :l]).all() and (dq_[0, 1, :l] == 0).all()
    # head 0 (own block), block starts: the only key is t itself
    starts = torch.arange(0, T, l)
    assert torch.equal(o[0, 0, starts], v[0, 0, starts])
    # head 1: positions that are not summary keys of an earlier block are never attended
    pos = torch.arange(T)
    never = ((pos % l) < l - c) | (pos >= (T // l - 1) * l)
    assert (dk_[0, 1, never] == 0).all() and (dv_[0, 1, never] == 0).all()
    # strided heads: t < l on the strided head, and t = 0 on the local head, have one key
    out_s, _ = run_fwd(q, k, v, inputs.STRIDED, l, 0)
    os_ = out_s.cpu()
    assert torch.equal(os_[0, 1, :l], v[0, 1, :l])
    assert torch.equal(os_[0, 0, 0], v[0, 0, 0])


@pytest.mark.parametrize("pattern", [inputs.FIXED, inputs.FIXED_UNION, inputs.DENSE],
                         ids=lambda p: inputs.PATTERN_NAMES[p])
def test_results_repeat_bit_for_bit(pattern):
    """The same inputs give the same bits on every call, also from another stream: the
    split key blocks (T = 4096 gives key columns of up to 64 row blocks, split at 24)
    are summed in slot order, and nothing depends on the order workgroups finish."""
    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, T, D, l, c = 1, 4, 4096, 64, 128, 8
    log(f"repeat: pattern {inputs.PATTERN_NAMES[pattern]} B{B} H{H} T{T} D{D} l{l} c{c}")
    g = torch.Generator().manual_seed(4242)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g).to(torch.bfloat16).cuda() for _ in range(4))

    def run():
        out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)
        dq, dk, dv = st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)
        return [t.clone() for t in (out, lse, dq, dk, dv)]

    first = run()
    again = run()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = run()
    torch.cuda.synchronize()
    for name, a, b, o in zip(("out", "lse", "dq", "dk", "dv"), first, again, other):
        bits = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(bits), b.view(bits)), f"{name}: second call differs"
        assert torch.equal(a.view(bits), o.view(bits)), f"{name}: call on another stream differs"


FWD_SHAPE_CASES = [
    # (pattern, dtype, D, B, H, T, l, c): ragged T, residue classes straddling 64-blocks at
    # D = 32, merged heads (carry and merge passes), a general summary set, full attention;
    # D = 128 and fp32 always take the four-wave forward
    (inputs.FIXED, "bf16", 64, 2, 3, 1000, 96, 8),
    (inputs.STRIDED, "bf16", 32, 1, 2, 395, 33, 0),
    (inputs.FIXED_UNION, "bf16", 64, 1, 2, 333, 20, 4),
    (inputs.STRIDED_UNION, "f16", 64, 2, 2, 700, 20, 0),
    (inputs.FIXED_R1, "f16", 32, 1, 3, 900, 64, (1, 30, 63)),
    (inputs.DENSE, "f16", 32, 1, 2, 300, 16, 0),
    (inputs.FIXED, "bf16", 128, 1, 2, 500, 96, 8),
    (inputs.STRIDED, "f32", 64, 1, 2, 300, 17, 0),
]


@pytest.mark.parametrize("case", FWD_SHAPE_CASES,
                         ids=lambda c: f"{inputs.PATTERN_NAMES[c[0]]}_{c[1]}_D{c[2]}_T{c[5]}_l{c[6]}")
def test_forward_kernel_shapes_agree_bit_for_bit(case):
    """The forward's two shapes (16 or 32 rows per wave; the library picks 16 only for
    short launches) compute every row with the same operations in the same order: forced
    either way, out and lse are the same bits, and the 32-row result meets the oracle's
    bound."""
    from factorized_sparse_self_amd import st_set_fwd_rows_per_wave, st_sparse_attn_fwd
    pattern, dtype, D, B, H, T, l, c = case
    log(f"forward shapes {case}")
    q, k, v = (x.cuda() for x in inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=2 * T + l, n=3))
    res = {}
    try:
        for rows in (16, 32):
            st_set_fwd_rows_per_wave(rows)
            res[rows] = [t.clone() for t in st_sparse_attn_fwd(q, k, v, pattern, l, c)]
            torch.cuda.synchronize()
    finally:
        st_set_fwd_rows_per_wave(0)
    bits = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(res[16][0].view(bits), res[32][0].view(bits)), "out: 16 and 32 rows per wave differ"
    assert torch.equal(res[16][1].view(torch.int32), res[32][1].view(torch.int32)), "lse: the shapes differ"
    O, L = oracle.forward(f64(q), f64(k), f64(v), pattern, l, c)
    assert_close(f64(res[32][0]), O, dtype, "out")
    assert_close(f64(res[32][1]), L, "f32", "lse")


DKDV_SHAPE_CASES = [
    # (pattern, dtype, D, B, H, T, l, c): split summary columns (T > 24 row blocks), merged
    # heads (carry and merge passes), residue classes straddling 64-blocks at D = 32, a
    # general summary set, full attention; D = 128 and fp32 always take 16 keys per wave
    (inputs.FIXED, "bf16", 64, 1, 2, 3000, 64, 4),
    (inputs.FIXED_UNION, "bf16", 64, 1, 2, 2500, 100, 5),
    (inputs.FIXED_R1, "f16", 32, 2, 2, 2300, 50, 3),
    (inputs.FIXED, "bf16", 64, 1, 3, 2200, 96, (0, 40, 95)),
    (inputs.STRIDED, "bf16", 32, 1, 2, 395, 33, 0),
    (inputs.STRIDED_UNION, "f16", 64, 2, 2, 700, 20, 0),
    (inputs.DENSE, "bf16", 64, 1, 2, 1000, 16, 0),
    (inputs.FIXED, "bf16", 128, 1, 2, 1000, 96, 8),
    (inputs.FIXED, "f32", 64, 1, 2, 700, 32, 4),
]


@pytest.mark.parametrize("case", DKDV_SHAPE_CASES,
                         ids=lambda c: f"{inputs.PATTERN_NAMES[c[0]]}_{c[1]}_D{c[2]}_T{c[5]}_l{c[6]}")
def test_dkdv_kernel_shapes_agree_bit_for_bit(case):
    """The dK/dV kernel's two shapes (16 or 32 keys per wave; the library picks 32 only
    for long launches) sum the same products in the same order: forced either way, the
    backward returns the same bits, and the 32-key result meets the oracle's bound."""
    from factorized_sparse_self_amd import st_set_dkdv_keys_per_wave, st_sparse_attn_bwd
    pattern, dtype, D, B, H, T, l, c = case
    log(f"dkdv shapes {case}")
    q, k, v, do = (x.cuda() for x in inputs.draw(B, H, T, D, dtype=TORCH_DTYPE[dtype], seed=T + 3 * l, n=4))
    out, lse = run_fwd(q, k, v, pattern, l, c)
    res = {}
    try:
        for keys in (16, 32):
            st_set_dkdv_keys_per_wave(keys)
            res[keys] = [t.clone() for t in st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)]
            torch.cuda.synchronize()
    finally:
        st_set_dkdv_keys_per_wave(0)
    bits = torch.int32 if dtype == "f32" else torch.int16
    for name, a, b in zip(("dq", "dk", "dv"), res[16], res[32]):
        assert torch.equal(a.view(bits), b.view(bits)), f"{name}: 16 and 32 keys per wave differ"
    qn, kn, vn, don = (f64(x) for x in (q, k, v, do))
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
    dq, dk, dv = res[32]
    assert_close(f64(dq), rq, dtype, "dq")
    assert_close(f64(dk), rk, dtype, "dk")
    assert_close(f64(dv), rv, dtype, "dv")


GUARD_CASES = [
    # (pattern, dtype, D, T, l, c): ragged T; a strided T whose classes straddle 64-blocks;
    # a merged head; fp32
    (inputs.STRIDED, "bf16", 64, 395, 33, 0),
    (inputs.STRIDED, "bf16", 32, 395, 33, 0),
    (inputs.FIXED, "bf16", 128, 1000, 96, 8),
    (inputs.FIXED, "bf16", 64, 1000, 96, 8),
    (inputs.FIXED, "f16", 32, 300, 20, 3),
    (inputs.DENSE, "bf16", 128, 200, 16, 0),
    (inputs.FIXED_UNION, "bf16", 64, 333, 20, 4),
    (inputs.STRIDED_UNION, "f16", 64, 250, 16, 0),
    (inputs.STRIDED, "f32", 64, 250, 16, 0),
]


@pytest.mark.parametrize("case", GUARD_CASES,
                         ids=lambda c: f"{inputs.PATTERN_NAMES[c[0]]}_{c[1]}_D{c[2]}_T{c[3]}_l{c[4]}")
def test_outputs_stay_inside_their_tensors(case):
    """Outputs carved out of larger buffers: every byte before and after them keeps its
    sentinel (the whole-line row stores and the zero fill write only rows of the tensor),
    and the results equal, bit for bit, those written into plain tensors."""
    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    pattern, dtype, D, T, l, c = case
    B, H, G = 1, 3, 32768  # G: a whole row block of fp32 rows at D = 128
    log(f"guard: pattern {inputs.PATTERN_NAMES[pattern]} {dtype} B{B} H{H} T{T} D{D} l{l} c{c}")
    td = TORCH_DTYPE[dtype]
    g = torch.Generator().manual_seed(515)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g).to(td).cuda() for _ in range(4))

    def guarded(shape, dt):
        n = math.prod(shape)
        big = torch.full((n + 2 * G,), -3.0, dtype=dt, device="cuda")
        return big, big[G:G + n].view(shape)

    bufs = {name: guarded((B, H, T, D), td) for name in ("out", "dq", "dk", "dv")}
    bufs["lse"] = guarded((B, H, T), torch.float32)
    st_sparse_attn_fwd(q, k, v, pattern, l, c, out=bufs["out"][1], lse=bufs["lse"][1])
    st_sparse_attn_bwd(q, k, v, bufs["out"][1], bufs["lse"][1], do, pattern, l, c,
                       dq=bufs["dq"][1], dk=bufs["dk"][1], dv=bufs["dv"][1])
    out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)
    dq, dk, dv = st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)
    torch.cuda.synchronize()
    for name, ref in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        big, view = bufs[name]
        n = view.numel()
        assert bool((big[:G] == -3.0).all()), f"{name}: written before the tensor"
        assert bool((big[G + n:] == -3.0).all()), f"{name}: written after the tensor"
        bits = torch.int32 if ref.dtype == torch.float32 else torch.int16
        assert torch.equal(view.view(bits), ref.view(bits)), f"{name}: differs from a plain tensor's result"


def test_two_streams_share_the_workspace_safely():
    """Backward calls on two streams with no ordering between them give the same bits
    as the same calls made one after the other: the library orders its workspace
    across streams (each call waits for the last user's kernels on another stream)."""
    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, T, D, l, c = 2, 8, 4096, 64, 128, 8
    log(f"two streams: fixed B{B} H{H} T{T} D{D} l{l} c{c}")
    problems = []
    for seed in (77, 78):
        q, k, v, do = (x.cuda() for x in inputs.draw(B, H, T, D, dtype=torch.bfloat16, seed=seed, n=4))
        out, lse = st_sparse_attn_fwd(q, k, v, inputs.FIXED, l, c)
        problems.append((q, k, v, out, lse, do))
    torch.cuda.synchronize()
    serial = [[g.clone() for g in st_sparse_attn_bwd(*p, inputs.FIXED, l, c)] for p in problems]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    results = []
    for rep in range(3):
        for p, s_ in zip(problems, streams):
            with torch.cuda.stream(s_):
                results.append(st_sparse_attn_bwd(*p, inputs.FIXED, l, c))
    torch.cuda.synchronize()
    for i, got in enumerate(results):
        for name, a, b in zip(("dq", "dk", "dv"), serial[i % 2], got):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} of call {i} differs"


def test_calls_from_two_host_threads():
    """Forward and backward called from two host threads at once, each on its own
    stream and with its own problem, give the bits of the same calls made one after
    the other (the library serialises its host state with a lock and orders its
    shared workspace across the streams)."""
    import threading

    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, T, D, l, c = 1, 8, 3000, 64, 64, 4
    log(f"two threads: fixed B{B} H{H} T{T} D{D} l{l} c{c}")
    problems = [tuple(x.cuda() for x in inputs.draw(B, H, T, D, dtype=torch.bfloat16, seed=s, n=4)) for s in (91, 92)]
    torch.cuda.synchronize()

    def run(p):
        q, k, v, do = p
        out, lse = st_sparse_attn_fwd(q, k, v, inputs.FIXED, l, c)
        return [out, lse] + list(st_sparse_attn_bwd(q, k, v, out, lse, do, inputs.FIXED, l, c))

    serial = [[t.clone() for t in run(p)] for p in problems]
    torch.cuda.synchronize()
    results = [[None] * 4 for _ in problems]
    errors = []

    def worker(i):
        try:
            s_ = torch.cuda.Stream()
            s_.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s_):
                for rep in range(4):
                    results[i][rep] = run(problems[i])
            s_.synchronize()
        except Exception as exc:  # reported in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(problems))]
    for t_ in threads:
        t_.start()
    for t_ in threads:
        t_.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i, reps in enumerate(results):
        for rep, got in enumerate(reps):
            for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), serial[i], got):
                bits = torch.int32 if a.dtype == torch.float32 else torch.int16
                assert torch.equal(a.view(bits), b.view(bits)), f"{name} of thread {i}, call {rep} differs"


def test_evicted_and_released_plans_rebuild_to_the_same_bits():
    """More shapes than the plan cache holds (64), launched back to back without
    waiting, so that plans are dropped while earlier calls' kernels may still be
    queued; then the same calls again (their plans rebuilt), and again after
    st_release() freed every plan and workspace.  Every repeat gives the first
    pass's bits, and sampled problems agree with the oracle."""
    from factorized_sparse_self_amd import st_release, st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, D, l, c = 1, 2, 32, 16, 2
    Ts = list(range(100, 100 + 3 * 80, 3))  # 80 distinct shapes
    log(f"plan cache: fixed B{B} H{H} D{D} l{l} c{c}, {len(Ts)} lengths")
    probs = [tuple(x.cuda() for x in inputs.draw(B, H, T, D, dtype=torch.bfloat16, seed=T, n=4)) for T in Ts]

    def run_all(idx):
        res = []
        for i in idx:
            q, k, v, do = probs[i]
            out, lse = st_sparse_attn_fwd(q, k, v, inputs.FIXED, l, c)
            res.append([out, lse, *st_sparse_attn_bwd(q, k, v, out, lse, do, inputs.FIXED, l, c)])
        torch.cuda.synchronize()
        return res

    first = run_all(range(len(Ts)))
    for i in (0, 37, len(Ts) - 1):
        q, k, v, do = (f64(x) for x in probs[i])
        O, L = oracle.forward(q, k, v, inputs.FIXED, l, c)
        rq, rk, rv = oracle.backward(q, k, v, do, inputs.FIXED, l, c)
        for name, got, ref, dt in zip(("out", "lse", "dq", "dk", "dv"), first[i], (O, L, rq, rk, rv),
                                      ("bf16", "f32", "bf16", "bf16", "bf16")):
            assert_close(f64(got), ref, dt, f"T={Ts[i]} {name}")
    again = run_all(range(len(Ts)))
    st_release()
    after = run_all(range(0, len(Ts), 7))
    for label, res, idx in (("rebuilt", again, range(len(Ts))), ("after release", after, range(0, len(Ts), 7))):
        for r, i in zip(res, idx):
            for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), first[i], r):
                bits = torch.int32 if a.dtype == torch.float32 else torch.int16
                assert torch.equal(a.view(bits), b.view(bits)), f"{label}: T={Ts[i]} {name} differs"


class DeviceRows:
    """A GPU tensor [B, H, T, ...] seen by the oracle as an array: indexing [b, h, t] or
    [b, h, positions] copies only those rows to the host, as float64.  Lets the oracle
    sample outputs of tensors too large to copy whole."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        b, h, r = idx
        if isinstance(r, (int, np.integer)):
            x = self.t[int(b), int(h), int(r)]
        else:
            x = self.t[int(b), int(h)].index_select(0, torch.as_tensor(np.asarray(r), device=self.t.device))
        return x.double().cpu().numpy()


def test_maximum_length():
    """T = 2^24 at D = 64, the largest head the 16-bit kernels address (T*D*2 = 2^31
    bytes): sampled rows and keys at both ends of the sequence against the oracle."""
    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, T, D, l, c = 1, 2, 1 << 24, 64, 4096, 0
    pattern = inputs.STRIDED
    log(f"maximum length: strided B{B} H{H} T{T} D{D} l{l}")
    g = torch.Generator(device="cuda").manual_seed(2024)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
    out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)
    dq, dk, dv = st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)
    torch.cuda.synchronize()
    for name, x in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(x).all(), name
    Q, K, V, G = (DeviceRows(x) for x in (q, k, v, do))
    rows = [0, 1, l - 1, l, T // 2 + 3, T - l - 1, T - 2, T - 1]
    O, L = oracle.forward_rows(Q, K, V, pattern, l, c, rows)
    assert_close(f64(out[:, :, rows]), O, "bf16", "out")
    assert_close(f64(lse[:, :, rows]), L, "f32", "lse")
    rq = oracle.backward_dq_rows(Q, K, V, G, pattern, l, c, rows)
    assert_close(f64(dq[:, :, rows]), rq, "bf16", "dq")
    keys = [5, T - 100, T - 1]
    for h in range(H):
        log(f"  oracle keys head {h}: {keys}")
        rk, rv = oracle.backward_dkdv_keys(Q, K, V, G, pattern, l, c, keys, heads=[h])
        assert_close(f64(dk[:, h, keys]), rk[:, h], "bf16", f"dk head {h}")
        assert_close(f64(dv[:, h, keys]), rv[:, h], "bf16", f"dv head {h}")


def test_maximum_heads():
    """B*H = 2^20 (the largest head count): the first and last heads of each kind against
    the oracle, whole."""
    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, T, D, l, c = 1, 1 << 20, 100, 32, 16, 4
    pattern = inputs.FIXED
    log(f"maximum heads: fixed B{B} H{H} T{T} D{D} l{l} c{c}")
    g = torch.Generator(device="cuda").manual_seed(2025)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
    out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)
    dq, dk, dv = st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)
    torch.cuda.synchronize()
    # heads 0, 1, H-2, H-1 keep their kinds (h mod 2) as heads 0..3 of a 4-head problem
    heads = torch.tensor([0, 1, H - 2, H - 1], device="cuda")
    pick = lambda x: x.index_select(1, heads)
    qn, kn, vn, don = (f64(pick(x)) for x in (q, k, v, do))
    O, L = oracle.forward(qn, kn, vn, pattern, l, c)
    assert_close(f64(pick(out)), O, "bf16", "out")
    assert_close(f64(pick(lse)), L, "f32", "lse")
    rq, rk, rv = oracle.backward(qn, kn, vn, don, pattern, l, c)
    assert_close(f64(pick(dq)), rq, "bf16", "dq")
    assert_close(f64(pick(dk)), rk, "bf16", "dk")
    assert_close(f64(pick(dv)), rv, "bf16", "dv")


def test_split_columns_of_a_longer_launch():
    """Fixed pattern, T = 12288, l = 128, with 80 heads: the launch is long enough that
    the summary heads' key columns (up to 190 row blocks) are split at 64 row blocks
    rather than 32.  Sampled rows and keys of the first and last heads of each kind
    against the oracle; the keys cover split and unsplit columns."""
    from factorized_sparse_self_amd import st_sparse_attn_bwd, st_sparse_attn_fwd
    B, H, T, D, l, c = 1, 80, 12288, 64, 128, 8
    pattern = inputs.FIXED
    log(f"split columns: fixed B{B} H{H} T{T} D{D} l{l} c{c}")
    g = torch.Generator(device="cuda").manual_seed(2026)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
    out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)
    dq, dk, dv = st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)
    torch.cuda.synchronize()
    # heads 0, 1, H-2, H-1 keep their kinds (h mod 2) as heads 0..3 of a 4-head problem
    heads = torch.tensor([0, 1, H - 2, H - 1], device="cuda")
    pick = lambda x: x.index_select(1, heads)
    qn, kn, vn, don = (f64(pick(x)) for x in (q, k, v, do))
    rows = sample_rows(T, l, 64, 7)
    O, L = oracle.forward_rows(qn, kn, vn, pattern, l, c, rows)
    assert_close(f64(pick(out))[:, :, rows], O, "bf16", "out")
    assert_close(f64(pick(lse))[:, :, rows], L, "f32", "lse")
    rq = oracle.backward_dq_rows(qn, kn, vn, don, pattern, l, c, rows)
    assert_close(f64(pick(dq))[:, :, rows], rq, "bf16", "dq")
    S = inputs.summary_offsets(l, c)
    nb = T // l
    # summary keys: block 0 (a column of 190 row blocks, three splits), the middle,
    # and block nb - 3 (a column of 4 row blocks, one piece); own-block keys
    keys = {1: [S[0], (nb // 2) * l + S[3], (nb - 3) * l + S[-1]], 0: [0, 127, T // 2 + 5, T - 1]}
    for h in range(4):
        log(f"  oracle keys head {h}")
        kk = keys[h % 2]
        rk, rv = oracle.backward_dkdv_keys(qn, kn, vn, don, pattern, l, c, kk, heads=[h])
        assert_close(f64(pick(dk))[:, h, kk], rk[:, h], "bf16", f"dk head {h}")
        assert_close(f64(pick(dv))[:, h, kk], rv[:, h], "bf16", f"dv head {h}")


def test_autograd_wrapper_matches_entry_points():
    from factorized_sparse_self_amd import sparse_attention
    B, H, T, D, l, c = 1, 2, 200, 64, 16, 3
    q, k, v, do = (x.cuda() for x in inputs.draw(B, H, T, D, dtype=torch.bfloat16, seed=11, n=4))
    qq, kk, vv = (x.clone().requires_grad_() for x in (q, k, v))
    out = sparse_attention(qq, kk, vv, inputs.FIXED, l, c)
    out.backward(do)
    out2, lse2 = run_fwd(q, k, v, inputs.FIXED, l, c)
    dq2, dk2, dv2 = run_bwd(q, k, v, out2, lse2, do, inputs.FIXED, l, c)
    assert torch.equal(out, out2)
    assert torch.equal(qq.grad, dq2) and torch.equal(kk.grad, dk2) and torch.equal(vv.grad, dv2)


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def sample_rows(T, l, n, seed):
    """About n query rows: the special rows (block and tile edges, the last rows) and
    seeded random ones."""
    rng = np.random.default_rng(seed)
    special = {s for s in (0, 1, l - 1, l, l + 1, T - 1, T - 2, T - l, 63, 64, 65) if 0 <= s < T}
    rest = [int(x) for x in rng.choice(T, size=min(n, T), replace=False) if int(x) not in special]
    rows = special | set(rest[:max(0, n - len(special))])
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("w", inputs.WORKLOADS[:2], ids=lambda w: w.name)
def test_workload_forward_full(w):
    log(f"workload {w.name}: full forward")
    q, k, v = inputs.draw_workload(w, n=3)
    out, lse = run_fwd(q, k, v, w.pattern, w.l, w.c)
    O, L = oracle.forward(f64(q), f64(k), f64(v), w.pattern, w.l, w.c)
    assert_close(f64(out), O, w.dtype, "out")
    assert_close(f64(lse), L, "f32", "lse")


def test_workload_strided_12288_forward_sampled():
    w = inputs.WORKLOADS[2]
    log(f"workload {w.name}: forward, 512 sampled rows per head")
    q, k, v = inputs.draw_workload(w, n=3)
    out, lse = run_fwd(q, k, v, w.pattern, w.l, w.c)
    rows = sample_rows(w.T, w.l, 512, w.seed)
    O, L = oracle.forward_rows(f64(q), f64(k), f64(v), w.pattern, w.l, w.c, rows)
    assert_close(f64(out)[:, :, rows], O, w.dtype, "out")
    assert_close(f64(lse)[:, :, rows], L, "f32", "lse")
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def _keys_for_head(w, kind, n, seed):
    rng = np.random.default_rng(seed + kind)
    if w.pattern in (inputs.FIXED, inputs.FIXED_R1) and kind == 1:
        nb = -(-w.T // w.l)
        S = inputs.summary_offsets(w.l, w.c)
        blocks = sorted({0, 1, nb // 2, nb - 2} | set(int(b) for b in rng.integers(0, nb - 1, size=2)))
        return np.array([b * w.l + S[int(rng.integers(0, len(S)))] for b in blocks], dtype=np.int64)
    if w.pattern == inputs.FIXED_UNION:
        # summary positions (attended by their own block and every later one),
        # other positions, and the last block's summary positions
        nb = -(-w.T // w.l)
        S = inputs.summary_offsets(w.l, w.c)
        keys = {b * w.l + S[int(rng.integers(0, len(S)))] for b in (0, 1, nb // 2, nb - 2, nb - 1)}
        keys |= set(int(x) for x in rng.choice(w.T, size=n // 2, replace=False)) | {0, w.T - 1}
        return np.array(sorted(k for k in keys if k < w.T), dtype=np.int64)
    if w.pattern == inputs.DENSE:
        # every later query attends key j, and the oracle recomputes each of them in
        # full, so the dense keys come from the last 512 positions (up to 512
        # attending queries each)
        tail = max(0, w.T - 512)
        keys = set(int(x) for x in rng.choice(np.arange(tail, w.T), size=min(3, w.T - tail),
                                              replace=False)) | {w.T - 1, w.T - 64, w.T - 65, tail}
        return np.array(sorted(keys), dtype=np.int64)
    keys = set(int(x) for x in rng.choice(w.T, size=n, replace=False)) | {0, w.T - 1, w.l}
    return np.array(sorted(keys), dtype=np.int64)


@pytest.mark.parametrize("w", inputs.WORKLOADS[3:] + inputs.EXTRA_WORKLOADS, ids=lambda w: w.name)
def test_workload_forward_backward_sampled(w):
    log(f"workload {w.name}: forward + backward at full size")
    q, k, v, do = inputs.draw_workload(w, n=4)
    out, lse = run_fwd(q, k, v, w.pattern, w.l, w.c)
    dq, dk, dv = run_bwd(q, k, v, out, lse, do, w.pattern, w.l, w.c)
    for x in (out, dq, dk, dv):
        assert torch.isfinite(x).all()
    # dense rows are long (up to T keys each), so fewer of them
    rows = sample_rows(w.T, w.l, 128 if w.pattern == inputs.DENSE else 512, w.seed)
    # batch 0 only for the oracle (batches are independent)
    qn, kn, vn, don = (f64(x[:1]) for x in (q, k, v, do))
    log(f"  oracle rows: {len(rows)} per head")
    O, L = oracle.forward_rows(qn, kn, vn, w.pattern, w.l, w.c, rows)
    assert_close(f64(out[:1])[:, :, rows], O, w.dtype, "out")
    assert_close(f64(lse[:1])[:, :, rows], L, "f32", "lse")
    rq = oracle.backward_dq_rows(qn, kn, vn, don, w.pattern, w.l, w.c, rows)
    assert_close(f64(dq[:1])[:, :, rows], rq, w.dtype, "dq")
    # dense: every head has the same key sets and a key's queries are many, so two heads
    for h in range(2 if w.pattern == inputs.DENSE else w.H):
        kind = h % 2
        # long rows (l >= 1024): every attending query is recomputed, so fewer keys
        keys = _keys_for_head(w, kind, 8 if w.l >= 1024 else 24, w.seed + h)
        log(f"  oracle keys head {h}: {len(keys)}")
        rk, rv = oracle.backward_dkdv_keys(qn, kn, vn, don, w.pattern, w.l, w.c, keys, heads=[h])
        assert_close(f64(dk[:1])[:, h, keys], rk[:, h], w.dtype, f"dk head {h}")
        assert_close(f64(dv[:1])[:, h, keys], rv[:, h], w.dtype, f"dv head {h}")
    if w.pattern in (inputs.FIXED, inputs.FIXED_R1):
        # summary heads: non-summary positions are never attended; under FIXED the
        # last block's summary positions are not either (no later block)
        pos = torch.arange(w.T)
        never = ~torch.isin(pos % w.l, torch.tensor(inputs.summary_offsets(w.l, w.c)))
        if w.pattern == inputs.FIXED:
            never |= pos >= (-(-w.T // w.l) - 1) * w.l  # the last l-block, partial or not
        dkc, dvc = dk.cpu(), dv.cpu()
        assert (dkc[:, 1::2][:, :, never] == 0).all() and (dvc[:, 1::2][:, :, never] == 0).all()
