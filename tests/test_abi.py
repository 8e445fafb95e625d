"""The C-ABI library loads and exports every entry point include/st.h declares.

Host only: argument errors are raised by the library's own checks before any
HIP call, so they can be exercised without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "st.h")
LIB = os.path.join(ROOT, "factorized_sparse_self_amd", "libst.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libst.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(st_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("st_layout_build", "st_sparse_attn_fwd", "st_sparse_attn_bwd", "st_sparse_attn_fwd_f16",
              "st_sparse_attn_bwd_f16", "st_sparse_attn_fwd_f32",
              "st_sparse_attn_bwd_f32", "st_layout_csr", "st_layout_csc", "st_layout_maps",
              "st_layout_build_ex", "st_sparse_attn_fwd_ex", "st_sparse_attn_bwd_ex"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    from factorized_sparse_self_amd import EXPORTED
    assert sorted(EXPORTED) == declared_functions()


def test_status_strings_and_block_size():
    from factorized_sparse_self_amd import lib
    L = lib()
    assert L.st_block_size() == 64
    assert L.st_status_string(0) == b"ok"
    assert L.st_status_string(-2) == b"unsupported configuration"


def test_kernel_shape_settings_accept_only_their_values():
    from factorized_sparse_self_amd import StError, lib, st_set_dkdv_keys_per_wave, st_set_fwd_rows_per_wave
    L = lib()
    for bad in (-1, 1, 8, 24, 64):
        assert L.st_set_dkdv_keys_per_wave(bad) == -1
        assert b"keys must be 0, 16 or 32" in L.st_last_error()
        assert L.st_set_fwd_rows_per_wave(bad) == -1
        assert b"rows must be 0, 16 or 32" in L.st_last_error()
    with pytest.raises(StError):
        st_set_dkdv_keys_per_wave(48)
    with pytest.raises(StError):
        st_set_fwd_rows_per_wave(48)
    for good in (16, 32, 0):
        st_set_dkdv_keys_per_wave(good)
        st_set_fwd_rows_per_wave(good)


def _call_fwd(name, ptr, B=1, H=2, T=64, D=64, pattern=0, l=8, c=0):
    from factorized_sparse_self_amd import lib
    return getattr(lib(), name)(ptr, ptr, ptr, ptr, ptr, B, H, T, D, pattern, l, c, None)


@pytest.mark.parametrize("name", ["st_sparse_attn_fwd", "st_sparse_attn_fwd_f16", "st_sparse_attn_fwd_f32"])
def test_attention_argument_errors_without_gpu(name):
    from factorized_sparse_self_amd import lib
    fake = 1 << 20  # aligned, never dereferenced: every case fails the checks first
    assert _call_fwd(name, None) == -1
    assert _call_fwd(name, fake + 8) == -1          # misaligned
    assert _call_fwd(name, fake, B=0) == -1
    assert _call_fwd(name, fake, T=0) == -1
    assert _call_fwd(name, fake, pattern=7) == -1
    assert _call_fwd(name, fake, pattern=1, c=0) == -1
    assert _call_fwd(name, fake, pattern=1, l=4, c=5) == -1
    assert _call_fwd(name, fake, D=48) == -2
    assert _call_fwd(name, fake, D=256) == -2
    assert b"D must be 32, 64 or 128" in lib().st_last_error()
    assert _call_fwd(name, fake, pattern=5, c=0) == -1   # merged fixed heads need c too
    # the 16-bit paths address a head with 32-bit offsets: T*D <= 2^30 (the fp32
    # path has no such limit, so its call would pass the checks: not made here)
    if not name.endswith("_f32"):
        assert _call_fwd(name, fake, T=(1 << 23) + 1, D=128, l=1024) == -2
        assert b"2^31 bytes" in lib().st_last_error()


def test_backward_argument_errors_without_gpu():
    from factorized_sparse_self_amd import lib
    L = lib()
    fake = 1 << 20
    args = [fake] * 9
    assert L.st_sparse_attn_bwd(*args, 1, 2, 64, 48, 0, 8, 0, None) == -2
    args[5] = None
    assert L.st_sparse_attn_bwd(*args, 1, 2, 64, 64, 0, 8, 0, None) == -1
    assert b"pointer 5" in L.st_last_error()


def test_extended_entry_points_check_dtype_and_summary_without_gpu():
    from factorized_sparse_self_amd import lib
    L = lib()
    fake = 1 << 20
    good = (ctypes.c_int32 * 2)(1, 5)
    bad = (ctypes.c_int32 * 2)(5, 1)
    assert L.st_sparse_attn_fwd_ex(7, fake, fake, fake, fake, fake, 1, 2, 64, 64, 1, 8, 2, good, None) == -1
    assert b"unknown dtype" in L.st_last_error()
    assert L.st_sparse_attn_fwd_ex(0, fake, fake, fake, fake, fake, 1, 2, 64, 64, 1, 8, 2, bad, None) == -1
    assert b"ascending" in L.st_last_error()
    assert L.st_sparse_attn_bwd_ex(1, *([fake] * 9), 1, 2, 64, 64, 0, 8, 0, good, None) == -1
    assert b"only taken by the fixed patterns" in L.st_last_error()


def test_layout_copy_outs_check_capacity():
    """A buffer one element short is refused with ST_ERR_BUFFER_TOO_SMALL and left
    untouched; a null buffer for a non-empty table is ST_ERR_INVALID."""
    import numpy as np
    from factorized_sparse_self_amd import lib
    L = lib()
    P = ctypes.c_void_p
    handle = P()
    assert L.st_layout_build(1, 300, 16, 3, ctypes.byref(handle)) == 0
    try:
        dims = (ctypes.c_int32 * 6)()
        assert L.st_layout_dims(handle, 1, dims) == 0
        nq, nnz, rows, keys = dims[3], dims[5], dims[1], dims[2]
        ptr = np.full(nq + 1, -7, np.int32)
        idx = np.full(nnz, -7, np.int32)
        flg = np.full(nnz, 9, np.uint8)
        buf = lambda a, n=None: (a.ctypes.data_as(P), a.size if n is None else n)  # noqa: E731
        assert L.st_layout_csr(handle, 1, *buf(ptr, nq), *buf(idx), *buf(flg)) == -5
        assert b"needs" in L.st_last_error()
        assert (ptr == -7).all() and (idx == -7).all() and (flg == 9).all()
        assert L.st_layout_csc(handle, 1, *buf(ptr), *buf(idx, nnz - 1), *buf(flg)) == -5
        assert L.st_layout_csc(handle, 1, *buf(ptr), *buf(idx), *buf(flg, nnz - 1)) == -5
        assert L.st_layout_csr(handle, 1, *buf(ptr), None, nnz, *buf(flg)) == -1
        rp, kp = np.zeros(rows, np.int32), np.zeros(keys, np.int32)
        assert L.st_layout_maps(handle, 1, *buf(rp), *buf(kp, keys - 1)) == -5
        assert L.st_layout_maps(handle, 1, *buf(rp), *buf(kp)) == 0
        assert L.st_layout_csr(handle, 1, *buf(ptr), *buf(idx), *buf(flg)) == 0
        assert ptr[0] == 0 and ptr[-1] == nnz
        assert L.st_status_string(-5) == b"caller buffer too small"
    finally:
        L.st_layout_free(handle)


def test_binding_rejects_an_lse_off_the_gpu():
    """The binding checks lse like the other tensors: a host tensor never reaches
    the library (checked here without a GPU on the lse check itself)."""
    import torch
    from factorized_sparse_self_amd._lib import _lse_check
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lse_check(torch.zeros(1, 2, 8), q)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lse_check(None, q)
