"""causal_head_self_amd -- causal multi-head self-attention (forward and
backward) for MI355X (gfx950), behind the C ABI of include/causal_attn.h.

This module is argument marshalling only: it hands tensor pointers, sizes and
the current HIP stream to libcausal_attn.so, whose kernels do every step of
the computation.  PyTorch supplies device memory and streams.

    attn_fwd(q, k, v, o, lse, scale)                        -- C ABI attn_fwd
    attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, scale) -- C ABI attn_bwd
    attn_bwd_dq / attn_bwd_dkdv                             -- its two stages
    attn_fwd_strided / attn_bwd_strided                     -- on strided views
    causal_attention(q, k, v, scale=None)                   -- autograd op
    causal_attention_qkv(qkv, n_head)                       -- autograd op on the
        fused [B, T, 3C] c_attn output, returning [B, T, C] with no layout copies
    attn_decode / decode_attention                          -- one new token per
        sequence against a [B, T_max, H, D] KV cache
    attn_decode_noalloc                                     -- the same without a
        workspace (the library's fixed device scratch), for callers that cannot allocate
    rope_qknorm_fwd / rope_qknorm_bwd                       -- RoPE and QK norm on
        query and key rows (also as causal_attention_qkv(..., prologue=Prologue()))
    attn_fwd_strided_rope / attn_bwd_strided_rope           -- attention with that
        prologue fused into its kernels (what causal_attention_qkv uses without dropout)
    layernorm_fwd / layernorm_bwd / colsum                  -- the row passes of the
        pre-norm sublayer (LayerNorm, its gradient with the residual term, bias gradients)

Tensors are contiguous [B, H, T, D] (D in {32, 64}; 128 in bf16) of float32 or bfloat16 on
the current GPU; lse and delta are float32 [B, H, T].
"""
from __future__ import annotations

import dataclasses
import math

import torch

from ._lib import (ABI_VERSION, ATTN_BF16, ATTN_F32, DECODE_SCRATCH_BYTES, EXPORTS, LIB_PATH,
                   AttnError, AttnView, check, load_library, status_str)

__all__ = [
    "attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_fwd_strided",
    "attn_bwd_strided", "attn_decode", "attn_decode_noalloc", "decode_workspace_bytes",
    "decode_attention", "DECODE_SCRATCH_BYTES",
    "rope_qknorm_fwd", "rope_qknorm_bwd", "Prologue", "attn_fwd_strided_rope",
    "attn_bwd_strided_rope", "layernorm_fwd", "layernorm_bwd", "layernorm_workspace_bytes",
    "colsum", "colsum_workspace_bytes",
    "attn_status_str", "causal_attention", "causal_attention_qkv", "qkv_heads", "AttnError",
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


def _view(t: torch.Tensor, name: str) -> AttnView:
    """A [B, H, T, D] tensor (any strides, D contiguous) as an attn_view_t."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be a [B, H, T, D] view with contiguous D")
    sb, sh, st, _ = t.stride()
    return AttnView(t.data_ptr(), sb, sh, st)


def attn_fwd_strided(q, k, v, o, lse, scale: float | None = None, stream=None,
                     window: int = 0, dropout_p: float = 0.0, seed: int = 0) -> None:
    """C ABI attn_fwd_strided: q, k, v, o are [B, H, T, D] views (D contiguous);
    window W > 0 keeps keys i-W < j <= i (0 = plain causal); dropout_p > 0
    drops attention weights with the Philox draws of `seed`."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_fwd_strided(
        _view(q, "q"), _view(k, "k"), _view(v, "v"), _view(o, "o"), _ptr(lse, "lse"),
        B, H, T, D, int(window), float(dropout_p), int(seed) & (2 ** 64 - 1), scale,
        _dtype_code(q), _stream(stream))
    check(rc)


def attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, scale: float | None = None,
                     stream=None, window: int = 0, dropout_p: float = 0.0, seed: int = 0) -> None:
    """C ABI attn_bwd_strided: every [B, H, T, D] argument is a view; window,
    dropout_p and seed as in the forward call."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_bwd_strided(
        _view(q, "q"), _view(k, "k"), _view(v, "v"), _view(o, "o"), _ptr(lse, "lse"),
        _view(dO, "dO"), _view(dq, "dq"), _view(dk, "dk"), _view(dv, "dv"),
        _ptr(delta, "delta"), B, H, T, D, int(window), float(dropout_p),
        int(seed) & (2 ** 64 - 1), scale, _dtype_code(q), _stream(stream))
    check(rc)


def attn_fwd_strided_rope(q, k, v, o, lse, q_rot, k_rot, prologue: "Prologue" = None,
                          scale: float | None = None, stream=None, window: int = 0) -> None:
    """C ABI attn_fwd_strided_rope: the prologue (RoPE / QK norm) fused into the
    attention forward.  q, k are the rows before the prologue; q_rot, k_rot
    receive them after it (the backward needs both)."""
    p = prologue or Prologue()
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_fwd_strided_rope(
        _view(q, "q"), _view(k, "k"), _view(v, "v"), _view(o, "o"), _ptr(lse, "lse"),
        _view(q_rot, "q_rot"), _view(k_rot, "k_rot"), B, H, T, D, int(window), scale,
        *p.args(), _dtype_code(q), _stream(stream))
    check(rc)


def attn_bwd_strided_rope(q, k, q_rot, k_rot, v, o, lse, dO, dq, dk, dv, delta,
                          prologue: "Prologue" = None, scale: float | None = None, stream=None,
                          window: int = 0) -> None:
    """C ABI attn_bwd_strided_rope: dq and dk with respect to the rows before the
    prologue (q, k), from the forward's q_rot, k_rot, o and lse."""
    p = prologue or Prologue()
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_bwd_strided_rope(
        _view(q, "q"), _view(k, "k"), _view(q_rot, "q_rot"), _view(k_rot, "k_rot"),
        _view(v, "v"), _view(o, "o"), _ptr(lse, "lse"), _view(dO, "dO"), _view(dq, "dq"),
        _view(dk, "dk"), _view(dv, "dv"), _ptr(delta, "delta"), B, H, T, D, int(window), scale,
        *p.args(), _dtype_code(q), _stream(stream))
    check(rc)


def dropout_keep_bytes(B: int, H: int, T: int) -> int:
    """C ABI attn_dropout_keep_bytes: size of the stored keep bits of one call."""
    return int(load_library().attn_dropout_keep_bytes(int(B), int(H), int(T)))


def _keep_buf(keep: torch.Tensor, name: str = "keep") -> tuple[int, int]:
    if not keep.is_cuda or not keep.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return keep.data_ptr(), keep.numel() * keep.element_size()


def attn_fwd_strided_keep(q, k, v, o, lse, keep, scale: float | None = None, stream=None,
                          window: int = 0, dropout_p: float = 0.0, seed: int = 0) -> None:
    """C ABI attn_fwd_strided_keep: attn_fwd_strided that also stores its keep
    bits in `keep` (a GPU tensor of at least dropout_keep_bytes(B, H, T) bytes)."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    kp, kb = _keep_buf(keep)
    rc = load_library().attn_fwd_strided_keep(
        _view(q, "q"), _view(k, "k"), _view(v, "v"), _view(o, "o"), _ptr(lse, "lse"),
        B, H, T, D, int(window), float(dropout_p), int(seed) & (2 ** 64 - 1), scale,
        _dtype_code(q), kp, kb, _stream(stream))
    check(rc)


def attn_bwd_strided_keep(q, k, v, o, lse, dO, dq, dk, dv, delta, keep,
                          scale: float | None = None, stream=None, window: int = 0,
                          dropout_p: float = 0.0) -> None:
    """C ABI attn_bwd_strided_keep: attn_bwd_strided with the keep bits loaded
    from `keep` (written by attn_fwd_strided_keep) instead of drawn."""
    B, H, T, D = _shape(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    kp, kb = _keep_buf(keep)
    rc = load_library().attn_bwd_strided_keep(
        _view(q, "q"), _view(k, "k"), _view(v, "v"), _view(o, "o"), _ptr(lse, "lse"),
        _view(dO, "dO"), _view(dq, "dq"), _view(dk, "dk"), _view(dv, "dv"),
        _ptr(delta, "delta"), B, H, T, D, int(window), float(dropout_p), scale,
        _dtype_code(q), kp, kb, _stream(stream))
    check(rc)


def qkv_heads(qkv: torch.Tensor, n_head: int):
    """q, k, v as [B, H, T, D] views of a [B, T, 3C] tensor (no copies)."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    D = C // n_head
    x = qkv.view(B, T, 3, n_head, D)
    return tuple(x[:, :, i].permute(0, 2, 1, 3) for i in range(3))


class _CausalAttentionQKV(torch.autograd.Function):
    @staticmethod
    def forward(ctx, qkv, n_head, window, prologue, dropout_p, seed, keep_bits):
        if qkv.dim() != 3 or qkv.shape[-1] % (3 * n_head) != 0 or qkv.stride(-1) != 1:
            raise ValueError("qkv must be [B, T, 3C] with contiguous last dim and C % n_head == 0")
        qkv = qkv if qkv.is_contiguous() else qkv.contiguous()
        B, T, C3 = qkv.shape
        C = C3 // 3
        q, k, v = qkv_heads(qkv, n_head)
        y = torch.empty((B, T, C), dtype=qkv.dtype, device=qkv.device)
        o = y.view(B, T, n_head, C // n_head).permute(0, 2, 1, 3)  # [B, H, T, D] view of y
        lse = torch.empty((B, n_head, T), dtype=torch.float32, device=qkv.device)
        fused = prologue is not None and dropout_p == 0.0
        if prologue is not None:  # rotated / normalised q and k, contiguous [B, H, T, D]
            qa = torch.empty(q.shape, dtype=q.dtype, device=q.device)
            ka = torch.empty_like(qa)
            if not fused:
                rope_qknorm_fwd(q, k, qa, ka, prologue)
        else:
            qa, ka = q, k
        keep = None
        if fused:  # the prologue inside the attention kernels
            attn_fwd_strided_rope(q, k, v, o, lse, qa, ka, prologue, window=window)
        elif dropout_p > 0.0 and keep_bits:  # the forward's keep decisions, for the backward
            keep = torch.empty((dropout_keep_bytes(B, n_head, T) // 4,), dtype=torch.int32,
                               device=qkv.device)
            attn_fwd_strided_keep(qa, ka, v, o, lse, keep, window=window, dropout_p=dropout_p,
                                  seed=seed)
        else:
            attn_fwd_strided(qa, ka, v, o, lse, window=window, dropout_p=dropout_p, seed=seed)
        saved = [qkv, y, lse] + ([qa, ka] if prologue is not None else [])
        ctx.has_keep = keep is not None
        ctx.save_for_backward(*saved, *([keep] if keep is not None else []))
        ctx.n_head = n_head
        ctx.window = window
        ctx.prologue = prologue
        ctx.dropout = (dropout_p, seed)
        return y

    @staticmethod
    def backward(ctx, dy):
        qkv, y, lse = ctx.saved_tensors[:3]
        n_head = ctx.n_head
        B, T, C3 = qkv.shape
        C = C3 // 3
        D = C // n_head
        dy = dy if dy.stride(-1) == 1 else dy.contiguous()
        q, k, v = qkv_heads(qkv, n_head)
        o = y.view(B, T, n_head, D).permute(0, 2, 1, 3)
        dO = dy.view(B, T, n_head, D).permute(0, 2, 1, 3) if dy.is_contiguous() else \
            dy.contiguous().view(B, T, n_head, D).permute(0, 2, 1, 3)
        dqkv = torch.empty_like(qkv)
        dq, dk, dv = qkv_heads(dqkv, n_head)
        delta = torch.empty_like(lse)
        keep = ctx.saved_tensors[-1] if ctx.has_keep else None

        def bwd(qx, kx, dqx, dkx):
            if keep is not None:
                attn_bwd_strided_keep(qx, kx, v, o, lse, dO, dqx, dkx, dv, delta, keep,
                                      window=ctx.window, dropout_p=ctx.dropout[0])
            else:
                attn_bwd_strided(qx, kx, v, o, lse, dO, dqx, dkx, dv, delta, window=ctx.window,
                                 dropout_p=ctx.dropout[0], seed=ctx.dropout[1])

        if ctx.prologue is None:
            bwd(q, k, dq, dk)
        elif ctx.dropout[0] == 0.0:  # the prologue's gradient inside the attention kernels
            qa, ka = ctx.saved_tensors[3:5]
            attn_bwd_strided_rope(q, k, qa, ka, v, o, lse, dO, dq, dk, dv, delta, ctx.prologue,
                                  window=ctx.window)
        else:
            qa, ka = ctx.saved_tensors[3:5]
            dqa, dka = torch.empty_like(qa), torch.empty_like(ka)
            bwd(qa, ka, dqa, dka)
            rope_qknorm_bwd(q, k, dqa, dka, dq, dk, ctx.prologue)
        return dqkv, None, None, None, None, None, None


def causal_attention_qkv(qkv: torch.Tensor, n_head: int, window: int = 0,
                         prologue: Prologue | None = None, dropout_p: float = 0.0,
                         seed: int | None = None, keep_bits: bool = True) -> torch.Tensor:
    """Causal attention on the fused c_attn output: qkv [B, T, 3C] (q, k, v
    chunks of C, each [B, T, H, D]) -> y [B, T, C] (heads merged), read and
    written in place through strided views (bf16, head dim 64 or 128).  window W > 0
    restricts query i to keys i-W < j <= i (sliding window).  prologue applies
    RoPE and/or QK norm to q and k first: without dropout inside the attention
    kernels (attn_fwd_strided_rope / attn_bwd_strided_rope), with dropout as
    separate passes (one extra read and write of q and k each way).  dropout_p > 0 drops attention weights (training mode); the
    Philox seed is drawn from torch's default generator unless given, and the
    backward reuses it.  With keep_bits (the default) the forward stores its
    keep decisions (dropout_keep_bytes(B, H, T) bytes, held for the backward)
    and the backward loads them instead of drawing them again; the results are
    the same bits either way."""
    if dropout_p > 0.0 and seed is None:
        seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    return _CausalAttentionQKV.apply(qkv, n_head, int(window), prologue, float(dropout_p),
                                     int(seed or 0), bool(keep_bits))


@dataclasses.dataclass(frozen=True)
class Prologue:
    """RoPE and/or QK norm applied to q and k before the attention (nanochat,
    section 9): RoPE turns column pair (i, i + D/2) at position pos0 + t by
    (pos0 + t) * base^(-2i/D); QK norm divides by sqrt(mean(x^2) + eps) and
    multiplies by q_gain (queries) or k_gain (keys)."""
    rope: bool = True
    qk_norm: bool = True
    pos0: int = 0
    base: float = 10000.0
    q_gain: float = 1.2
    k_gain: float = 1.0
    eps: float = 1e-6

    @property
    def flags(self) -> int:
        return (1 if self.rope else 0) | (2 if self.qk_norm else 0)

    def args(self):
        return (int(self.pos0), float(self.base), float(self.q_gain), float(self.k_gain),
                float(self.eps), self.flags)


def rope_qknorm_fwd(q, k, q_out, k_out, prologue: "Prologue" = None, stream=None) -> None:
    """C ABI attn_rope_qknorm_fwd on [B, H, T, D] views (bf16, D 64 or 128)."""
    p = prologue or Prologue()
    B, H, T, D = _shape(q)
    rc = load_library().attn_rope_qknorm_fwd(
        _view(q, "q"), _view(k, "k"), _view(q_out, "q_out"), _view(k_out, "k_out"), B, H, T, D,
        *p.args(), _dtype_code(q), _stream(stream))
    check(rc)


def rope_qknorm_bwd(q, k, dq_out, dk_out, dq, dk, prologue: "Prologue" = None,
                    stream=None) -> None:
    """C ABI attn_rope_qknorm_bwd: dq, dk from the gradients dq_out, dk_out of
    the forward's results."""
    p = prologue or Prologue()
    B, H, T, D = _shape(q)
    rc = load_library().attn_rope_qknorm_bwd(
        _view(q, "q"), _view(k, "k"), _view(dq_out, "dq_out"), _view(dk_out, "dk_out"),
        _view(dq, "dq"), _view(dk, "dk"), B, H, T, D, *p.args(), _dtype_code(q), _stream(stream))
    check(rc)


def decode_workspace_bytes(B: int, H: int, T_max: int, D: int) -> int:
    """C ABI attn_decode_workspace_bytes."""
    return int(load_library().attn_decode_workspace_bytes(int(B), int(H), int(T_max), int(D)))


def attn_decode(q, k_cache, v_cache, cache_lens, o, lse, workspace, scale: float | None = None,
                window: int = 0, stream=None) -> None:
    """C ABI attn_decode: q, o [B, H, D]; k_cache, v_cache [B, T_max, H, D] (bf16);
    cache_lens int32 [B]; lse fp32 [B, H]; workspace a byte (uint8) tensor of at
    least decode_workspace_bytes(B, H, T_max, D)."""
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache must be [B, T_max, H, D], got {tuple(k_cache.shape)}")
    B, T_max, H, D = (int(s) for s in k_cache.shape)
    if tuple(q.shape) != (B, H, D) or tuple(o.shape) != (B, H, D):
        raise ValueError("q and o must be [B, H, D] for a [B, T_max, H, D] cache")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(lse.shape) != (B, H):
        raise ValueError("v_cache must match k_cache and lse must be [B, H]")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_decode(
        _ptr(q, "q"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(cache_lens, "cache_lens"), _ptr(o, "o"), _ptr(lse, "lse"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), B, H, T_max,
        D, int(window), scale, _dtype_code(q), _stream(stream))
    check(rc)


def attn_decode_noalloc(q, k_cache, v_cache, cache_lens, o, lse, scale: float | None = None,
                        window: int = 0, stream=None) -> None:
    """C ABI attn_decode_noalloc: attn_decode without a workspace (the library's
    fixed device scratch of DECODE_SCRATCH_BYTES holds the split path's
    partials; calls that overlap in time on one device race on it)."""
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache must be [B, T_max, H, D], got {tuple(k_cache.shape)}")
    B, T_max, H, D = (int(s) for s in k_cache.shape)
    if tuple(q.shape) != (B, H, D) or tuple(o.shape) != (B, H, D):
        raise ValueError("q and o must be [B, H, D] for a [B, T_max, H, D] cache")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(lse.shape) != (B, H):
        raise ValueError("v_cache must match k_cache and lse must be [B, H]")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rc = load_library().attn_decode_noalloc(
        _ptr(q, "q"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(cache_lens, "cache_lens"), _ptr(o, "o"), _ptr(lse, "lse"), B, H, T_max, D,
        int(window), scale, _dtype_code(q), _stream(stream))
    check(rc)


def decode_attention(q, k_cache, v_cache, cache_lens, scale: float | None = None,
                     window: int = 0):
    """attn_decode with freshly allocated o, lse and workspace: returns (o, lse)."""
    B, T_max, H, D = (int(s) for s in k_cache.shape)
    o = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    ws = torch.empty(decode_workspace_bytes(B, H, T_max, D), dtype=torch.uint8, device=q.device)
    attn_decode(q, k_cache, v_cache, cache_lens, o, lse, ws, scale, window)
    return o, lse


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


def _rows(t: torch.Tensor, name: str, C: int | None = None, stride: int | None = None):
    """(N, C, row stride) of a 2-D bf16 GPU tensor whose rows are contiguous."""
    if not t.is_cuda or t.dim() != 2 or t.dtype != torch.bfloat16 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D bfloat16 GPU tensor with contiguous rows")
    if C is not None and t.shape[1] != C:
        raise ValueError(f"{name} must have {C} columns")
    if stride is not None and t.stride(0) != stride:
        raise ValueError(f"{name} must have the row stride of x ({stride})")
    return int(t.shape[0]), int(t.shape[1]), int(t.stride(0))


def _vec(t: torch.Tensor, name: str, C: int):
    if not t.is_cuda or t.dtype != torch.bfloat16 or tuple(t.shape) != (C,) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 [{C}] GPU tensor")
    return t.data_ptr()


def layernorm_workspace_bytes(N: int, C: int) -> int:
    """C ABI attn_layernorm_workspace_bytes."""
    return int(load_library().attn_layernorm_workspace_bytes(int(N), int(C)))


def colsum_workspace_bytes(N: int, M: int) -> int:
    """C ABI attn_colsum_workspace_bytes."""
    return int(load_library().attn_colsum_workspace_bytes(int(N), int(M)))


def layernorm_fwd(x, g, b, y, eps: float = 1e-5, stream=None) -> None:
    """C ABI attn_layernorm_fwd: y = LayerNorm(x) * g + b over the rows of x
    [N, C] (bf16; y has x's shape and row stride)."""
    N, C, st = _rows(x, "x")
    _rows(y, "y", C, st)
    if y.shape[0] != N:
        raise ValueError("y must have the rows of x")
    rc = load_library().attn_layernorm_fwd(x.data_ptr(), _vec(g, "g", C), _vec(b, "b", C),
                                           y.data_ptr(), N, C, st, float(eps), ATTN_BF16,
                                           _stream(stream))
    check(rc)


def layernorm_bwd(x, g, dy, dx, dg, db, workspace, dres=None, eps: float = 1e-5,
                  stream=None) -> None:
    """C ABI attn_layernorm_bwd: dx (+ dres, the residual branch's gradient),
    dg, db of LayerNorm from x and dy = d(loss)/d(output); workspace a byte
    tensor of at least layernorm_workspace_bytes(N, C)."""
    N, C, st = _rows(x, "x")
    for t, n in ((dy, "dy"), (dx, "dx")) + (((dres, "dres"),) if dres is not None else ()):
        _rows(t, n, C, st)
        if t.shape[0] != N:
            raise ValueError(f"{n} must have the rows of x")
    rc = load_library().attn_layernorm_bwd(
        x.data_ptr(), _vec(g, "g", C), dy.data_ptr(), None if dres is None else dres.data_ptr(),
        dx.data_ptr(), _vec(dg, "dg", C), _vec(db, "db", C), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), N, C, st, float(eps), ATTN_BF16,
        _stream(stream))
    check(rc)


def colsum(x, out, workspace=None, stream=None) -> None:
    """C ABI attn_colsum: out[j] = sum over the rows of x [N, M] of x[:, j], out
    bf16 [M].  x bf16 (workspace: a byte tensor of at least
    colsum_workspace_bytes(N, M)) or float32 (a few rows; no workspace)."""
    f32 = x.dtype == torch.float32
    if f32:
        if not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
            raise ValueError("x must be a 2-D GPU tensor with contiguous rows")
        N, M, st = int(x.shape[0]), int(x.shape[1]), int(x.stride(0))
    else:
        N, M, st = _rows(x, "x")
    ws, ws_bytes = (None, 0) if workspace is None else (
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size())
    rc = load_library().attn_colsum(x.data_ptr(), _vec(out, "out", M), ws, ws_bytes, N, M, st,
                                    ATTN_F32 if f32 else ATTN_BF16, _stream(stream))
    check(rc)
