"""ctypes view of libflash_attn.so: the C entry points with the same names.

Argument marshalling only.  Loading fails loudly if the library has not been
built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflash_attn.so")

FA_OK = 0
FA_F16, FA_BF16, FA_F16_OUT_F32, FA_BF16_OUT_F32 = 0, 1, 2, 3
FA_ERR_SCRATCH = 10
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # FA_NOALLOC_SCRATCH_BYTES in the header

# every extern "C" symbol declared in include/flash_attn.h
EXPORTED = (
    "flash_attn_fwd",
    "flash_attn_fwd_bias",
    "flash_attn_fwd_splitkv",
    "flash_attn_fwd_splitkv_workspace_bytes",
    "flash_attn_fwd_splitkv_default_splits",
    "flash_attn_bwd",
    "flash_attn_bwd_bias",
    "flash_attn_bwd_preprocess",
    "flash_attn_bwd_dkdv",
    "flash_attn_bwd_dq",
    "flash_attn_bwd_workspace_bytes",
    "flash_attn_bwd_noalloc",
    "flash_attn_status_string",
    "flash_attn_version",
)

_lib = None


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """Load the built HIP library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python io_aware_exact_08_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_fwd.restype = i
    ll = ctypes.c_longlong
    lib.flash_attn_fwd_bias.argtypes = [vp, vp, vp, vp, ll, ll, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_fwd_bias.restype = i
    lib.flash_attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_fwd_splitkv.restype = i
    lib.flash_attn_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.flash_attn_fwd_splitkv_workspace_bytes.restype = sz
    lib.flash_attn_fwd_splitkv_default_splits.argtypes = [i, i, i, i, i]
    lib.flash_attn_fwd_splitkv_default_splits.restype = i
    lib.flash_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                   i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd.restype = i
    lib.flash_attn_bwd_bias.argtypes = [vp, vp, vp, vp, ll, ll, vp, vp, vp, vp, vp, vp, vp, sz,
                                        i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd_bias.restype = i
    lib.flash_attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, i, vp]
    lib.flash_attn_bwd_preprocess.restype = i
    lib.flash_attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd_dkdv.restype = i
    lib.flash_attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, sz, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd_dq.restype = i
    lib.flash_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd_noalloc.restype = i
    lib.flash_attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.flash_attn_bwd_workspace_bytes.restype = sz
    lib.flash_attn_status_string.argtypes = [i]
    lib.flash_attn_status_string.restype = ctypes.c_char_p
    lib.flash_attn_version.argtypes = []
    lib.flash_attn_version.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().flash_attn_status_string(int(status)).decode()


def flash_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw C call with integer device pointers; returns the fa_status."""
    return load().flash_attn_fwd(q, k, v, o, lse, B, H, N, d, float(scale), int(causal),
                                 int(dtype), stream)


def flash_attn_fwd_bias(q, k, v, bias, bias_stride_b, bias_stride_h, o, lse, B, H, N, d, scale,
                        causal, dtype, stream) -> int:
    """Raw C call with integer device pointers; returns the fa_status."""
    return load().flash_attn_fwd_bias(q, k, v, bias, int(bias_stride_b), int(bias_stride_h), o, lse,
                                      B, H, N, d, float(scale), int(causal), int(dtype), stream)


def flash_attn_fwd_splitkv(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                           causal, dtype, num_splits, stream) -> int:
    """Raw C call with integer device pointers; returns the fa_status."""
    return load().flash_attn_fwd_splitkv(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d,
                                         float(scale), int(causal), int(dtype), int(num_splits),
                                         stream)


def flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits) -> int:
    return int(load().flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits))


def flash_attn_fwd_splitkv_default_splits(B, H, N, d, causal) -> int:
    return int(load().flash_attn_fwd_splitkv_default_splits(B, H, N, d, int(causal)))


def flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                   B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw C call with integer device pointers; returns the fa_status."""
    return load().flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                 workspace_bytes, B, H, N, d, float(scale), int(causal),
                                 int(dtype), stream)


def flash_attn_bwd_bias(q, k, v, bias, bias_stride_b, bias_stride_h, o, lse, dout, dq, dk, dv,
                        workspace, workspace_bytes, B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw C call with integer device pointers; returns the fa_status."""
    return load().flash_attn_bwd_bias(q, k, v, bias, int(bias_stride_b), int(bias_stride_h), o, lse,
                                      dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                                      float(scale), int(causal), int(dtype), stream)


def flash_attn_bwd_preprocess(o, lse, dout, workspace, workspace_bytes, B, H, N, d, dtype,
                              stream) -> int:
    return load().flash_attn_bwd_preprocess(o, lse, dout, workspace, workspace_bytes, B, H, N, d,
                                            int(dtype), stream)


def flash_attn_bwd_dkdv(q, k, v, dout, workspace, workspace_bytes, dk, dv, B, H, N, d, scale,
                        causal, dtype, stream) -> int:
    return load().flash_attn_bwd_dkdv(q, k, v, dout, workspace, workspace_bytes, dk, dv, B, H, N,
                                      d, float(scale), int(causal), int(dtype), stream)


def flash_attn_bwd_dq(q, k, v, dout, workspace, workspace_bytes, dq, B, H, N, d, scale, causal,
                      dtype, stream) -> int:
    return load().flash_attn_bwd_dq(q, k, v, dout, workspace, workspace_bytes, dq, B, H, N, d,
                                    float(scale), int(causal), int(dtype), stream)


def flash_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, dtype,
                           stream) -> int:
    """Raw C call with integer device pointers; returns the fa_status."""
    return load().flash_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d,
                                         float(scale), int(causal), int(dtype), stream)


def flash_attn_bwd_workspace_bytes(B, H, N, d) -> int:
    return int(load().flash_attn_bwd_workspace_bytes(B, H, N, d))


def flash_attn_version() -> int:
    return int(load().flash_attn_version())
