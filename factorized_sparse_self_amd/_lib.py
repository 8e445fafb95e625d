"""ctypes binding of libst.so (argument marshalling only).

Every function here forwards to the C entry point of the same name in
``include/st.h``; all attention arithmetic runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no fallback:
if ``libst.so`` is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libst.so")

ST_STRIDED, ST_FIXED, ST_FIXED_R1, ST_DENSE, ST_STRIDED_UNION, ST_FIXED_UNION = range(6)
ST_DIM_BLOCK, ST_DIM_ROWS, ST_DIM_KEYS, ST_DIM_QBLOCKS, ST_DIM_KBLOCKS, ST_DIM_NNZ = range(6)
ST_BF16, ST_F16, ST_F32 = range(3)


def _summary(c):
    """(count, int32 array or None) for a summary argument: an integer c (the last c
    offsets of each block) or the summary offsets themselves (a sequence)."""
    if isinstance(c, (int, np.integer)):
        return int(c), None
    offs = np.ascontiguousarray(np.asarray(list(c), dtype=np.int32))
    return int(offs.size), offs

# name -> (restype, argtypes) of every exported symbol
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_SIG = {
    "st_layout_build": (_I, [_I, _I, _I, _I, ctypes.POINTER(_P)]),
    "st_layout_build_ex": (_I, [_I, _I, _I, _I, _P, ctypes.POINTER(_P)]),
    "st_layout_dims": (_I, [_P, _I, ctypes.POINTER(ctypes.c_int32)]),
    "st_layout_pairs": (_I, [_P, _I, ctypes.POINTER(ctypes.c_int64)]),
    "st_layout_maps": (_I, [_P, _I, _P, _Z, _P, _Z]),
    "st_layout_csr": (_I, [_P, _I, _P, _Z, _P, _Z, _P, _Z]),
    "st_layout_csc": (_I, [_P, _I, _P, _Z, _P, _Z, _P, _Z]),
    "st_layout_free": (None, [_P]),
    "st_sparse_attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "st_sparse_attn_fwd_f16": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "st_sparse_attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "st_sparse_attn_bwd": (_I, [_P] * 9 + [_I] * 7 + [_P]),
    "st_sparse_attn_bwd_f16": (_I, [_P] * 9 + [_I] * 7 + [_P]),
    "st_sparse_attn_bwd_f32": (_I, [_P] * 9 + [_I] * 7 + [_P]),
    "st_sparse_attn_fwd_ex": (_I, [_I] + [_P] * 5 + [_I] * 7 + [_P, _P]),
    "st_sparse_attn_bwd_ex": (_I, [_I] + [_P] * 9 + [_I] * 7 + [_P, _P]),
    "st_sparse_attn_bwd_noalloc": (_I, [_I] + [_P] * 9 + [_I] * 7 + [_P, _P]),
    "st_set_fwd_rows_per_wave": (_I, [_I]),
    "st_set_dkdv_keys_per_wave": (_I, [_I]),
    "st_timing_enable": (_I, [_I]),
    "st_timing_read": (_I, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]),
    "st_timing_reset": (None, []),
    "st_block_size": (_I, []),
    "st_status_string": (ctypes.c_char_p, [_I]),
    "st_last_error": (ctypes.c_char_p, []),
    "st_release": (None, []),
}
EXPORTED = tuple(_SIG)

_lib = None


class StError(RuntimeError):
    """A libst entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libst.so (once).  Raises when the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: the HIP library is not built "
                               "(python -m factorized_sparse_self_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = lib()
        raise StError(fn, status, f"{L.st_status_string(status).decode()}: {L.st_last_error().decode()}")


# ---------------------------------------------------------------------------
# Layout (host only)
# ---------------------------------------------------------------------------

def st_layout_build(pattern: int, T: int, l: int, c=0) -> list[dict]:
    """Block LUTs of both head kinds as numpy arrays: [kind0, kind1].  ``c``: the
    summary count (last c offsets) or the summary offsets (a sequence)."""
    L = lib()
    handle = _P()
    n, offs = _summary(c)
    if offs is None:
        _check("st_layout_build", L.st_layout_build(pattern, T, l, n, ctypes.byref(handle)))
    else:
        _check("st_layout_build_ex", L.st_layout_build_ex(pattern, T, l, n, offs.ctypes.data_as(_P),
                                                          ctypes.byref(handle)))
    try:
        out = []
        for kind in (0, 1):
            dims = (ctypes.c_int32 * 6)()
            _check("st_layout_dims", L.st_layout_dims(handle, kind, dims))
            dims = list(dims)
            pairs = ctypes.c_int64()
            _check("st_layout_pairs", L.st_layout_pairs(handle, kind, ctypes.byref(pairs)))
            nnz = dims[ST_DIM_NNZ]
            row_pos = np.zeros(dims[ST_DIM_ROWS], np.int32)
            key_pos = np.zeros(max(dims[ST_DIM_KEYS], 1), np.int32)
            row_ptr = np.zeros(dims[ST_DIM_QBLOCKS] + 1, np.int32)
            col_idx = np.zeros(max(nnz, 1), np.int32)
            flags = np.zeros(max(nnz, 1), np.uint8)
            col_ptr = np.zeros(dims[ST_DIM_KBLOCKS] + 1, np.int32)
            row_idx = np.zeros(max(nnz, 1), np.int32)
            csc_flags = np.zeros(max(nnz, 1), np.uint8)
            buf = lambda a: (a.ctypes.data_as(_P), a.size)  # noqa: E731  (pointer, capacity)
            _check("st_layout_maps", L.st_layout_maps(handle, kind, *buf(row_pos), *buf(key_pos)))
            _check("st_layout_csr", L.st_layout_csr(handle, kind, *buf(row_ptr), *buf(col_idx), *buf(flags)))
            _check("st_layout_csc", L.st_layout_csc(handle, kind, *buf(col_ptr), *buf(row_idx), *buf(csc_flags)))
            out.append({
                "block": dims[ST_DIM_BLOCK], "n_rows": dims[ST_DIM_ROWS], "n_keys": dims[ST_DIM_KEYS],
                "n_qb": dims[ST_DIM_QBLOCKS], "n_kb": dims[ST_DIM_KBLOCKS], "nnz": nnz,
                "pairs": pairs.value, "row_pos": row_pos, "key_pos": key_pos[:dims[ST_DIM_KEYS]],
                "row_ptr": row_ptr, "col_idx": col_idx[:nnz], "flags": flags[:nnz],
                "col_ptr": col_ptr, "row_idx": row_idx[:nnz], "csc_flags": csc_flags[:nnz],
            })
        return out
    finally:
        L.st_layout_free(handle)


def st_block_size() -> int:
    return lib().st_block_size()


def st_release() -> None:
    lib().st_release()


KERNEL_NAMES = ("fwd", "bwd_pre", "bwd_dq", "bwd_dkdv", "bwd_reduce", "bwd_delta")


def st_set_fwd_rows_per_wave(rows: int) -> None:
    """Shape of the 16-bit forward: 0 = chosen per launch, 16 or 32 = forced (results are identical)."""
    _check("st_set_fwd_rows_per_wave", lib().st_set_fwd_rows_per_wave(int(rows)))


def st_set_dkdv_keys_per_wave(keys: int) -> None:
    """Shape of the 16-bit dK/dV kernel: 0 = chosen per launch, 16 or 32 = forced (results are identical)."""
    _check("st_set_dkdv_keys_per_wave", lib().st_set_dkdv_keys_per_wave(int(keys)))


def st_timing_enable(on: bool) -> None:
    _check("st_timing_enable", lib().st_timing_enable(1 if on else 0))


def st_timing_reset() -> None:
    lib().st_timing_reset()


def st_timing_read(kernel: str) -> tuple[int, float]:
    """(launches, summed milliseconds) of one kernel since the last reset."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check("st_timing_read", lib().st_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


# ---------------------------------------------------------------------------
# Attention (device tensors)
# ---------------------------------------------------------------------------

def _shape_check(name, x, like):
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if x.dtype != like.dtype or tuple(x.shape) != tuple(like.shape):
        raise ValueError(f"{name} must match q in dtype and shape [B, H, T, D]")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.device != like.device:
        raise ValueError(f"{name} must be on q's device")


def _lse_check(lse, q):
    import torch
    B, H, T, _ = q.shape
    if not isinstance(lse, torch.Tensor) or not lse.is_cuda:
        raise ValueError("lse must be a GPU tensor")
    if lse.device != q.device:
        raise ValueError("lse must be on q's device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")


def _dtype_code(dtype):
    import torch
    codes = {torch.bfloat16: ST_BF16, torch.float16: ST_F16, torch.float32: ST_F32}
    if dtype not in codes:
        raise TypeError("q, k, v must be bfloat16, float16 or float32")
    return codes[dtype]


def _entry(dtype, base):
    return base + ("", "_f16", "_f32")[_dtype_code(dtype)]


def st_sparse_attn_fwd(q, k, v, pattern: int, l: int, c=0, out=None, lse=None):
    """out [B,H,T,D] and lse [B,H,T] fp32 of sparse causal attention.  ``c``: the
    summary count (last c offsets of each block) or the summary offsets."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, D]")
    B, H, T, D = q.shape
    _shape_check("q", q, q)
    _shape_check("k", k, q)
    _shape_check("v", v, q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    _shape_check("out", out, q)
    _lse_check(lse, q)
    n, offs = _summary(c)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
        if offs is None:
            name = _entry(q.dtype, "st_sparse_attn_fwd")
            _check(name, getattr(lib(), name)(*ptrs, B, H, T, D, pattern, l, n, stream))
        else:
            _check("st_sparse_attn_fwd_ex", lib().st_sparse_attn_fwd_ex(
                _dtype_code(q.dtype), *ptrs, B, H, T, D, pattern, l, n, offs.ctypes.data_as(_P), stream))
    return out, lse


def st_sparse_attn_bwd(q, k, v, out, lse, dout, pattern: int, l: int, c=0,
                       dq=None, dk=None, dv=None):
    """dq, dk, dv of L = <dout, out>, recomputing the attention weights from lse."""
    import torch
    B, H, T, D = q.shape
    for name, x in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _shape_check(name, x, q)
    _lse_check(lse, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _shape_check(name, x, q)
    n, offs = _summary(c)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
        if offs is None:
            name = _entry(q.dtype, "st_sparse_attn_bwd")
            _check(name, getattr(lib(), name)(*ptrs, B, H, T, D, pattern, l, n, stream))
        else:
            _check("st_sparse_attn_bwd_ex", lib().st_sparse_attn_bwd_ex(
                _dtype_code(q.dtype), *ptrs, B, H, T, D, pattern, l, n, offs.ctypes.data_as(_P), stream))
    return dq, dk, dv


def st_sparse_attn_bwd_noalloc(q, k, v, out, lse, dout, pattern: int, l: int, c=0, dq=None, dk=None, dv=None):
    """st_sparse_attn_bwd through the entry point that allocates nothing in the library
    (its workspace is a static device array; the plan must already be cached)."""
    import torch
    B, H, T, D = q.shape
    for name, x in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _shape_check(name, x, q)
    _lse_check(lse, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _shape_check(name, x, q)
    n, offs = _summary(c)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
        _check("st_sparse_attn_bwd_noalloc", lib().st_sparse_attn_bwd_noalloc(
            _dtype_code(q.dtype), *ptrs, B, H, T, D, pattern, l, n,
            None if offs is None else offs.ctypes.data_as(_P), stream))
    return dq, dk, dv


def _autograd_function():
    import torch

    class SparseAttention(torch.autograd.Function):
        """Forward keeps only (q, k, v, out, lse); the backward recomputes the weights."""

        @staticmethod
        def forward(ctx, q, k, v, pattern, l, c):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            out, lse = st_sparse_attn_fwd(q, k, v, pattern, l, c)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.cfg = (pattern, l, c)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            dq, dk, dv = st_sparse_attn_bwd(q, k, v, out, lse, dout.contiguous(), *ctx.cfg)
            return dq, dk, dv, None, None, None

    return SparseAttention


_SparseAttention = None


def sparse_attention(q, k, v, pattern: int, l: int, c=0):
    """Differentiable sparse attention (torch.autograd) over st_sparse_attn_fwd / _bwd."""
    global _SparseAttention
    if _SparseAttention is None:
        _SparseAttention = _autograd_function()
    return _SparseAttention.apply(q, k, v, pattern, l, c)
