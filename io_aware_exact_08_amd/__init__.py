"""Exact scaled-dot-product attention for MI355X (gfx950).

The computation runs entirely in the HIP library ``libflash_attn.so``; this
module only marshals torch tensors (device memory and streams) into its C ABI:

    flash_attn_fwd(q, k, v, causal=False, scale=None, out_f32=False) -> (o, lse)
    flash_attn_fwd_bias(q, k, v, bias, causal=False, scale=None) -> (o, lse)
    flash_attn_fwd_splitkv(q, k, v, causal=False, scale=None, num_splits=0) -> (o, lse)
    flash_attn_bwd(q, k, v, o, lse, dout, causal=False, scale=None) -> (dq, dk, dv)
    flash_attn_bwd_bias(q, k, v, bias, o, lse, dout, causal=False, scale=None) -> (dq, dk, dv)

Layout [B, H, N, d], d in {64, 128, 256}, fp16 or bf16 inputs.
"""
from __future__ import annotations

import math

from . import _lib
from ._lib import FlashAttnError, status_string  # noqa: F401

__all__ = ["flash_attn_fwd", "flash_attn_fwd_bias", "flash_attn_fwd_splitkv", "flash_attn_bwd",
           "flash_attn_bwd_bias", "flash_attn_bwd_noalloc", "flash_attn_bwd_preprocess",
           "flash_attn_bwd_dkdv", "flash_attn_bwd_dq", "FlashAttnError", "status_string",
           "dtype_code", "workspace_bytes"]


def _torch():
    import torch
    return torch


def dtype_code(in_dtype, out_f32: bool) -> int:
    torch = _torch()
    if in_dtype == torch.float16:
        return _lib.FA_F16_OUT_F32 if out_f32 else _lib.FA_F16
    if in_dtype == torch.bfloat16:
        return _lib.FA_BF16_OUT_F32 if out_f32 else _lib.FA_BF16
    raise TypeError(f"unsupported input dtype {in_dtype}; expected float16 or bfloat16")


def _check(t, name, shape, dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t):
    torch = _torch()
    return ctypes_stream(torch.cuda.current_stream(t.device))


def ctypes_stream(s):
    return s.cuda_stream


def workspace_bytes(B, H, N, d) -> int:
    return _lib.flash_attn_bwd_workspace_bytes(B, H, N, d)


def flash_attn_fwd(q, k, v, causal: bool = False, scale=None, out_f32: bool = False,
                   o=None, lse=None):
    """Forward: returns (o [B,H,N,d], lse [B,H,N] float32).

    ``o``/``lse`` may be passed to write into existing buffers.  ``scale``
    defaults to 1/sqrt(d), rounded to float32.
    """
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (B, H, N, d), q.dtype)
    code = dtype_code(q.dtype, out_f32)
    odt = torch.float32 if out_f32 else q.dtype
    if o is None:
        o = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    _check(o, "o", (B, H, N, d), odt)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lse, "lse", (B, H, N), torch.float32)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, H, N, d, sc, int(bool(causal)), code, _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd")
    return o, lse


def flash_attn_fwd_bias(q, k, v, bias, causal: bool = False, scale=None, out_f32: bool = False,
                        o=None, lse=None):
    """Forward with an additive attention bias: softmax(scale Q K^T + bias) V.

    ``bias`` has the input dtype and shape [N, N], [H, N, N], [B, H, N, N] or
    any shape that broadcasts to [B, H, N, N] with contiguous [N, N] rows
    (e.g. an expanded view); -inf entries hide keys."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (B, H, N, d), q.dtype)
    if not bias.is_cuda or bias.dtype != q.dtype:
        raise TypeError("bias must be a device tensor of the input dtype")
    bb = bias.expand(B, H, N, N)
    if bb.stride(3) != 1 or bb.stride(2) != N:
        raise ValueError("bias rows must be contiguous [N, N] blocks")
    code = dtype_code(q.dtype, out_f32)
    odt = torch.float32 if out_f32 else q.dtype
    if o is None:
        o = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    _check(o, "o", (B, H, N, d), odt)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lse, "lse", (B, H, N), torch.float32)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_fwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), bb.data_ptr(),
                                  bb.stride(0), bb.stride(1), o.data_ptr(), lse.data_ptr(),
                                  B, H, N, d, sc, int(bool(causal)), code, _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_bias")
    return o, lse


def flash_attn_fwd_splitkv(q, k, v, causal: bool = False, scale=None, out_f32: bool = False,
                           num_splits: int = 0, o=None, lse=None, workspace=None):
    """Forward with the key range split over ``num_splits`` workgroups per query
    tile and merged (0: the library's automatic plan for this shape, which may
    split only the items of the last partial round, or none).  Same result as
    flash_attn_fwd within rounding.  The float32 workspace is allocated here
    unless given."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (B, H, N, d), q.dtype)
    code = dtype_code(q.dtype, out_f32)
    odt = torch.float32 if out_f32 else q.dtype
    if o is None:
        o = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    _check(o, "o", (B, H, N, d), odt)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lse, "lse", (B, H, N), torch.float32)
    nbytes = _lib.flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=q.device)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), B, H, N, d,
                                     sc, int(bool(causal)), code, num_splits, _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_splitkv")
    return o, lse


def flash_attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale=None,
                   dq=None, dk=None, dv=None, workspace=None):
    """Backward: returns (dq, dk, dv) in the input dtype.

    ``o`` is the forward output (input dtype or float32); ``dout`` has the
    input dtype.  The workspace (8*B*H*N bytes) is allocated here unless given.
    """
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, (B, H, N, d), q.dtype)
    out_f32 = o.dtype == torch.float32
    _check(o, "o", (B, H, N, d), o.dtype)
    if not out_f32 and o.dtype != q.dtype:
        raise TypeError("o must have the input dtype or float32")
    _check(lse, "lse", (B, H, N), torch.float32)
    code = dtype_code(q.dtype, out_f32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, (B, H, N, d), q.dtype)
    nbytes = workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=q.device)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(),
                             B, H, N, d, sc, int(bool(causal)), code, _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd")
    return dq, dk, dv


def flash_attn_bwd_noalloc(q, k, v, o, lse, dout, causal: bool = False, scale=None,
                           dq=None, dk=None, dv=None):
    """flash_attn_bwd without a workspace argument: the library keeps the
    per-row terms in its static device scratch (8*B*H*N bytes must fit it).
    The C call allocates nothing; dq/dk/dv are allocated here unless given."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, (B, H, N, d), q.dtype)
    out_f32 = o.dtype == torch.float32
    _check(o, "o", (B, H, N, d), o.dtype)
    if not out_f32 and o.dtype != q.dtype:
        raise TypeError("o must have the input dtype or float32")
    _check(lse, "lse", (B, H, N), torch.float32)
    code = dtype_code(q.dtype, out_f32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, (B, H, N, d), q.dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                     dv.data_ptr(), B, H, N, d, sc, int(bool(causal)), code,
                                     _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_noalloc")
    return dq, dk, dv


def flash_attn_bwd_bias(q, k, v, bias, o, lse, dout, causal: bool = False, scale=None,
                        dq=None, dk=None, dv=None, workspace=None):
    """Backward of flash_attn_fwd_bias (same bias): returns (dq, dk, dv)."""
    torch = _torch()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, (B, H, N, d), q.dtype)
    if not bias.is_cuda or bias.dtype != q.dtype:
        raise TypeError("bias must be a device tensor of the input dtype")
    bb = bias.expand(B, H, N, N)
    if bb.stride(3) != 1 or bb.stride(2) != N:
        raise ValueError("bias rows must be contiguous [N, N] blocks")
    out_f32 = o.dtype == torch.float32
    _check(o, "o", (B, H, N, d), o.dtype)
    _check(lse, "lse", (B, H, N), torch.float32)
    code = dtype_code(q.dtype, out_f32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    nbytes = workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=q.device)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_bwd_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), bb.data_ptr(),
                                  bb.stride(0), bb.stride(1), o.data_ptr(), lse.data_ptr(),
                                  dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  B, H, N, d, sc, int(bool(causal)), code, _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_bias")
    return dq, dk, dv


def _bwd_common(q, k, v, dout):
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, (B, H, N, d), q.dtype)
    return B, H, N, d


def _check_ws(workspace, B, H, N, d):
    torch = _torch()
    if not workspace.is_cuda or workspace.dtype != torch.float32 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 device tensor")
    if workspace.numel() * 4 < workspace_bytes(B, H, N, d):
        raise ValueError("workspace too small")


def flash_attn_bwd_preprocess(o, lse, dout, workspace, in_dtype=None):
    """Stage 1 of the backward: -D and -LSE*log2(e) into `workspace`."""
    torch = _torch()
    B, H, N, d = dout.shape
    in_dtype = dout.dtype if in_dtype is None else in_dtype
    _check(dout, "dout", (B, H, N, d), in_dtype)
    _check(o, "o", (B, H, N, d), o.dtype)
    _check(lse, "lse", (B, H, N), torch.float32)
    _check_ws(workspace, B, H, N, d)
    code = dtype_code(in_dtype, o.dtype == torch.float32)
    st = _lib.flash_attn_bwd_preprocess(o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                        workspace.data_ptr(), workspace.numel() * 4,
                                        B, H, N, d, code, _stream(dout))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_preprocess")


def flash_attn_bwd_dkdv(q, k, v, dout, workspace, causal=False, scale=None, dk=None, dv=None):
    """Stage 2 of the backward: dK, dV (needs the preprocessed workspace)."""
    B, H, N, d = _bwd_common(q, k, v, dout)
    _check_ws(workspace, B, H, N, d)
    dk = _torch().empty_like(k) if dk is None else dk
    dv = _torch().empty_like(v) if dv is None else dv
    for name, t in (("dk", dk), ("dv", dv)):
        _check(t, name, (B, H, N, d), q.dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * 4, dk.data_ptr(),
                                  dv.data_ptr(), B, H, N, d, sc, int(bool(causal)),
                                  dtype_code(q.dtype, False), _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_dkdv")
    return dk, dv


def flash_attn_bwd_dq(q, k, v, dout, workspace, causal=False, scale=None, dq=None):
    """Stage 3 of the backward: dQ (needs the preprocessed workspace)."""
    B, H, N, d = _bwd_common(q, k, v, dout)
    _check_ws(workspace, B, H, N, d)
    dq = _torch().empty_like(q) if dq is None else dq
    _check(dq, "dq", (B, H, N, d), q.dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    st = _lib.flash_attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                workspace.data_ptr(), workspace.numel() * 4, dq.data_ptr(),
                                B, H, N, d, sc, int(bool(causal)), dtype_code(q.dtype, False),
                                _stream(q))
    if st != _lib.FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_dq")
    return dq
