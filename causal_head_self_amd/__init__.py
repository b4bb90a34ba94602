"""causal_head_self_amd -- causal multi-head self-attention (forward and
backward) for MI355X (gfx950), behind the C ABI of include/causal_attn.h.

This module is argument marshalling only: it hands tensor pointers, sizes and
the current HIP stream to libcausal_attn.so, whose kernels do every step of
the computation.  PyTorch supplies device memory and streams.

    attn_fwd(q, k, v, o, lse, scale)                        -- C ABI attn_fwd
    attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, scale) -- C ABI attn_bwd
    attn_bwd_dq / attn_bwd_dkdv                             -- its two stages
    causal_attention(q, k, v, scale=None)                   -- autograd op

Tensors are contiguous [B, H, T, D] (D in {32, 64}) of float32 or bfloat16 on
the current GPU; lse and delta are float32 [B, H, T].
"""
from __future__ import annotations

import math

import torch

from ._lib import (ABI_VERSION, ATTN_BF16, ATTN_F32, EXPORTS, LIB_PATH, AttnError, check,
                   load_library, status_str)

__all__ = [
    "attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_status_str",
    "causal_attention", "AttnError",
    "ATTN_F32", "ATTN_BF16", "load_library", "LIB_PATH", "EXPORTS", "ABI_VERSION",
]

_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def attn_status_str(status: int) -> str:
    return status_str(status)


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _ptr(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError(f"expected [B, H, T, D], got shape {tuple(q.shape)}")
    return tuple(int(s) for s in q.shape)


def attn_fwd(q, k, v, o, lse, scale: float | None = None, stream=None) -> None:
    """C ABI attn_fwd: writes o and lse in place."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_fwd(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(o, "o"), _ptr(lse, "lse"),
        B, H, T, D, scale, _dtype_code(q), _stream(stream))
    check(rc)


def attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, scale: float | None = None,
             stream=None) -> None:
    """C ABI attn_bwd: writes dq, dk, dv and delta in place."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_bwd(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(o, "o"), _ptr(lse, "lse"),
        _ptr(dO, "dO"), _ptr(dq, "dq"), _ptr(dk, "dk"), _ptr(dv, "dv"), _ptr(delta, "delta"),
        B, H, T, D, scale, _dtype_code(q), _stream(stream))
    check(rc)


def attn_bwd_dq(q, k, v, o, dO, lse, delta, dq, scale: float | None = None,
                stream=None) -> None:
    """C ABI attn_bwd_dq: writes delta and dq."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_bwd_dq(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(o, "o"), _ptr(dO, "dO"),
        _ptr(lse, "lse"), _ptr(delta, "delta"), _ptr(dq, "dq"), B, H, T, D, scale,
        _dtype_code(q), _stream(stream))
    check(rc)


def attn_bwd_dkdv(q, k, v, dO, lse, delta, dk, dv, scale: float | None = None,
                  stream=None) -> None:
    """C ABI attn_bwd_dkdv."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_bwd_dkdv(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(dO, "dO"), _ptr(lse, "lse"),
        _ptr(delta, "delta"), _ptr(dk, "dk"), _ptr(dv, "dv"), B, H, T, D, scale,
        _dtype_code(q), _stream(stream))
    check(rc)


def _same_layout(name, t, ref):
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{name} must match q in shape, dtype and device")


class _CausalAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale):
        _same_layout("k", k, q)
        _same_layout("v", v, q)
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        B, H, T, D = _shape(q)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        attn_fwd(q, k, v, o, lse, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse = ctx.saved_tensors
        dO = dO.contiguous()
        if dO.dtype != q.dtype:
            dO = dO.to(q.dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)
        attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, ctx.scale)
        return dq, dk, dv, None


def causal_attention(q, k, v, scale: float | None = None):
    """Causal scaled dot-product attention per (batch, head) with autograd.

    q, k, v: [B, H, T, D] float32 or bfloat16 GPU tensors.  scale defaults to
    1/sqrt(D), the pages' choice."""
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return _CausalAttention.apply(q, k, v, scale)
