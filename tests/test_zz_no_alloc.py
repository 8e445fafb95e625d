"""The backward entry point that allocates nothing (st_sparse_attn_bwd_noalloc),
through the C ABI, against the allocating entry point it varies
(st_sparse_attn_bwd_ex): the same kernels on the same inputs, so the results
must agree bit for bit.  Two calls in a row, the second on a smaller problem
(the static scratch keeps the first call's contents), and the size limit."""
import sys

import pytest
import torch

from factorized_sparse_self_amd import StError, inputs, st_sparse_attn_bwd, st_sparse_attn_bwd_noalloc, st_sparse_attn_fwd

pytestmark = pytest.mark.gpu


def _case(pattern, B, H, T, D, l, c, dtype, seed):
    print(f"no-alloc backward: pattern {pattern} B{B} H{H} T{T} D{D} l{l} c{c} {dtype}", flush=True)
    q, k, v, do = (x.cuda() for x in inputs.draw(B, H, T, D, dtype=dtype, seed=seed, n=4))
    out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)          # builds the plan
    ref = st_sparse_attn_bwd(q, k, v, out, lse, do, pattern, l, c)  # the allocating entry point
    got = st_sparse_attn_bwd_noalloc(q, k, v, out, lse, do, pattern, l, c)
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(bits), b.view(bits)), f"{name} differs from st_sparse_attn_bwd_ex"


def test_noalloc_matches_allocating_backward_twice_then_smaller():
    # the benchmark's fixed configuration (split key columns, the reduction), then a
    # smaller ragged problem with rows whose Delta comes from the pre-pass
    _case(inputs.FIXED, 4, 8, 12288, 64, 128, 8, torch.bfloat16, 5)
    _case(inputs.FIXED, 1, 3, 403, 32, 82, 5, torch.bfloat16, 6)
    # merged heads and the fp32 path at a small size
    _case(inputs.STRIDED_UNION, 1, 2, 300, 64, 20, 0, torch.bfloat16, 7)
    _case(inputs.STRIDED, 1, 2, 256, 32, 16, 0, torch.float32, 8)
    # D = 128 (four-wave dq workgroups) with split key columns
    _case(inputs.FIXED, 1, 4, 4096, 128, 64, 8, torch.float16, 10)


def test_noalloc_refuses_what_it_cannot_hold():
    q, k, v, do = (x.cuda() for x in inputs.draw(1, 2, 97, 64, dtype=torch.bfloat16, seed=9, n=4))
    out = torch.empty_like(q)
    lse = torch.empty(1, 2, 97, device="cuda")
    # no cached plan for these shapes yet (no other test uses them): refused, nothing launched
    with pytest.raises(StError, match="no cached plan"):
        st_sparse_attn_bwd_noalloc(q, k, v, out, lse, do, inputs.FIXED, 13, 3)
    # merged heads carry three fp32 copies of the gradients: 2^20 rows of D = 64
    # need 768 MiB, past the 64 MiB scratch
    B, H, T, D = 1, 8, 1 << 17, 64
    big = torch.zeros(B, H, T, D, dtype=torch.bfloat16, device="cuda")
    lse_big = torch.zeros(B, H, T, device="cuda")
    st_sparse_attn_fwd(big, big, big, inputs.FIXED_UNION, 128, 8, out=big.clone(), lse=lse_big)
    with pytest.raises(StError, match="static scratch holds"):
        st_sparse_attn_bwd_noalloc(big, big, big, big, lse_big, big, inputs.FIXED_UNION, 128, 8)
    torch.cuda.synchronize()


def test_noalloc_backward_replays_in_a_graph():
    """The callers the entry point is for: a HIP graph captures the forward and the
    allocation-free backward once (plan cached and scratch looked up beforehand), and
    every replay -- with new input values copied in, the outputs poisoned, and the
    library's allocating and allocation-free calls run eagerly on other problems
    between replays -- gives the bits of eager calls on the same values."""
    B, H, T, D, l, c = 1, 4, 2048, 64, 128, 8
    pattern = inputs.FIXED
    print(f"graph replay: fixed B{B} H{H} T{T} D{D} l{l} c{c} bf16", flush=True)
    sets = [tuple(x.cuda() for x in inputs.draw(B, H, T, D, dtype=torch.bfloat16, seed=s, n=4)) for s in (21, 22, 23)]
    q, k, v, do = (x.clone() for x in sets[0])  # the graph's static inputs
    out, lse = torch.empty_like(q), torch.empty(B, H, T, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    st_sparse_attn_fwd(q, k, v, pattern, l, c, out=out, lse=lse)
    st_sparse_attn_bwd_noalloc(q, k, v, out, lse, do, pattern, l, c, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st_sparse_attn_fwd(q, k, v, pattern, l, c, out=out, lse=lse)
        st_sparse_attn_bwd_noalloc(q, k, v, out, lse, do, pattern, l, c, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for rep in range(6):
        src = sets[rep % 3]
        for dst, x in zip((q, k, v, do), src):
            dst.copy_(x)
        for t in (out, lse, dq, dk, dv):
            t.fill_(float("nan"))  # a replay that leaves anything unwritten fails
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, lse, dq, dk, dv)]
        # eager work between replays: the allocating entry points on the same values
        # (the reference), then an allocation-free call on other values, which leaves
        # its own contents in the static scratch
        e_out, e_lse = st_sparse_attn_fwd(*src[:3], pattern, l, c)
        ref = [e_out, e_lse, *st_sparse_attn_bwd(*src[:3], e_out, e_lse, src[3], pattern, l, c)]
        other = sets[(rep + 1) % 3]
        o_out, o_lse = st_sparse_attn_fwd(*other[:3], pattern, l, c)
        st_sparse_attn_bwd_noalloc(*other[:3], o_out, o_lse, other[3], pattern, l, c)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), ref, got):
            bits = torch.int32 if a.dtype == torch.float32 else torch.int16
            assert torch.equal(a.view(bits), b.view(bits)), f"replay {rep}: {name} differs from eager calls"
