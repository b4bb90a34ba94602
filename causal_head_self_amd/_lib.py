"""ctypes loader for libcausal_attn.so (the C ABI in include/causal_attn.h).

The library is built in-tree by ``python -m causal_head_self_amd.build``.  If
it is missing, loading raises: there is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcausal_attn.so")

ATTN_F32 = 0
ATTN_BF16 = 1

STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED_D",
    4: "ATTN_ERR_DTYPE",
    5: "ATTN_ERR_ALIGN",
    6: "ATTN_ERR_OVERFLOW",
    7: "ATTN_ERR_SCALE",
    8: "ATTN_ERR_ALIAS",
    9: "ATTN_ERR_HIP",
    10: "ATTN_ERR_LAYOUT",
    11: "ATTN_ERR_WORKSPACE",
    12: "ATTN_ERR_PARAM",
    13: "ATTN_ERR_SCRATCH",
}

ATTN_ROPE = 1
ATTN_QK_NORM = 2

# every symbol include/causal_attn.h declares
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_fwd_strided",
           "attn_bwd_strided", "attn_dropout_keep_bytes", "attn_fwd_strided_keep",
           "attn_bwd_strided_keep", "attn_decode", "attn_decode_workspace_bytes",
           "attn_decode_noalloc", "attn_rope_qknorm_fwd", "attn_rope_qknorm_bwd",
           "attn_fwd_strided_rope", "attn_bwd_strided_rope", "attn_layernorm_workspace_bytes",
           "attn_layernorm_fwd", "attn_layernorm_bwd", "attn_colsum_workspace_bytes",
           "attn_colsum", "attn_status_str", "attn_abi_version")
ABI_VERSION = (1 << 16) | 8
# the fixed device scratch of attn_decode_noalloc (CAUSAL_ATTN_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 16 << 20


class AttnView(ctypes.Structure):
    """attn_view_t: a [B][H][T][D] tensor with element strides."""
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_longlong),
                ("stride_h", ctypes.c_longlong), ("stride_t", ctypes.c_longlong)]


class AttnError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_vp = ctypes.c_void_p
_int = ctypes.c_int
_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is not built: run `python -m causal_head_self_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, ctypes.c_float,
                             _int, _vp]
    lib.attn_fwd.restype = _int
    lib.attn_bwd.argtypes = [_vp] * 10 + [_int, _int, _int, _int, ctypes.c_float, _int, _vp]
    lib.attn_bwd.restype = _int
    lib.attn_bwd_dq.argtypes = [_vp] * 8 + [_int] * 4 + [ctypes.c_float, _int, _vp]
    lib.attn_bwd_dq.restype = _int
    lib.attn_bwd_dkdv.argtypes = [_vp] * 8 + [_int] * 4 + [ctypes.c_float, _int, _vp]
    lib.attn_bwd_dkdv.restype = _int
    lib.attn_fwd_strided.argtypes = [AttnView] * 4 + [_vp, _int, _int, _int, _int, _int,
                                                      ctypes.c_float, ctypes.c_ulonglong,
                                                      ctypes.c_float, _int, _vp]
    lib.attn_fwd_strided.restype = _int
    lib.attn_bwd_strided.argtypes = ([AttnView] * 4 + [_vp] + [AttnView] * 4 +
                                     [_vp, _int, _int, _int, _int, _int, ctypes.c_float,
                                      ctypes.c_ulonglong, ctypes.c_float, _int, _vp])
    lib.attn_bwd_strided.restype = _int
    lib.attn_dropout_keep_bytes.argtypes = [_int] * 3
    lib.attn_dropout_keep_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_strided_keep.argtypes = ([AttnView] * 4 + [_vp, _int, _int, _int, _int, _int,
                                           ctypes.c_float, ctypes.c_ulonglong, ctypes.c_float,
                                           _int, _vp, ctypes.c_size_t, _vp])
    lib.attn_fwd_strided_keep.restype = _int
    lib.attn_bwd_strided_keep.argtypes = ([AttnView] * 4 + [_vp] + [AttnView] * 4 +
                                          [_vp, _int, _int, _int, _int, _int, ctypes.c_float,
                                           ctypes.c_float, _int, _vp, ctypes.c_size_t, _vp])
    lib.attn_bwd_strided_keep.restype = _int
    lib.attn_decode_workspace_bytes.argtypes = [_int] * 4
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode.argtypes = ([_vp] * 7 + [ctypes.c_size_t] + [_int] * 5 +
                                [ctypes.c_float, _int, _vp])
    lib.attn_decode.restype = _int
    lib.attn_decode_noalloc.argtypes = [_vp] * 6 + [_int] * 5 + [ctypes.c_float, _int, _vp]
    lib.attn_decode_noalloc.restype = _int
    _rope_tail = [_int] * 5 + [ctypes.c_float] * 4 + [_int, _int, _vp]
    lib.attn_rope_qknorm_fwd.argtypes = [AttnView] * 4 + _rope_tail
    lib.attn_rope_qknorm_fwd.restype = _int
    lib.attn_rope_qknorm_bwd.argtypes = [AttnView] * 6 + _rope_tail
    lib.attn_rope_qknorm_bwd.restype = _int
    lib.attn_fwd_strided_rope.argtypes = ([AttnView] * 4 + [_vp] + [AttnView] * 2 +
                                          [_int] * 5 + [ctypes.c_float] + [_int] +
                                          [ctypes.c_float] * 4 + [_int, _int, _vp])
    lib.attn_fwd_strided_rope.restype = _int
    lib.attn_bwd_strided_rope.argtypes = ([AttnView] * 6 + [_vp] + [AttnView] * 4 + [_vp] +
                                          [_int] * 5 + [ctypes.c_float] + [_int] +
                                          [ctypes.c_float] * 4 + [_int, _int, _vp])
    lib.attn_bwd_strided_rope.restype = _int
    _ll, _sz = ctypes.c_longlong, ctypes.c_size_t
    lib.attn_layernorm_workspace_bytes.argtypes = [_int, _int]
    lib.attn_layernorm_workspace_bytes.restype = _sz
    lib.attn_layernorm_fwd.argtypes = [_vp] * 4 + [_int, _int, _ll, ctypes.c_float, _int, _vp]
    lib.attn_layernorm_fwd.restype = _int
    lib.attn_layernorm_bwd.argtypes = ([_vp] * 8 + [_sz, _int, _int, _ll, ctypes.c_float, _int,
                                                    _vp])
    lib.attn_layernorm_bwd.restype = _int
    lib.attn_colsum_workspace_bytes.argtypes = [_int, _int]
    lib.attn_colsum_workspace_bytes.restype = _sz
    lib.attn_colsum.argtypes = [_vp] * 3 + [_sz, _int, _int, _ll, _int, _vp]
    lib.attn_colsum.restype = _int
    lib.attn_status_str.argtypes = [_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = _int
    if lib.attn_abi_version() != ABI_VERSION:
        raise ImportError(f"{p}: ABI version {lib.attn_abi_version():#x}, expected {ABI_VERSION:#x}")
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def check(status: int) -> None:
    if status != 0:
        raise AttnError(status, status_str(status))
