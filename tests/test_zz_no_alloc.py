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
