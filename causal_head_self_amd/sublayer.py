"""Pre-norm causal self-attention sublayer around the HIP attention op.

    y = x + c_proj(merge_heads(attention(split_heads(c_attn(LN(x))))))

This follows the CS336 from-scratch tutorial (lmnt.cn), section 5.1 model.py:
Block.forward adds attn(ln_1(x)) to x (pre-norm, section 3.4), and
CausalSelfAttention runs c_attn (C -> 3C), chunks the result into q, k, v,
views each as [B, T, H, D] -> [B, H, T, D], attends, merges the heads back and
applies c_proj (C -> C).  LayerNorm uses the biased variance and eps 1e-5
(class LayerNorm on the same page).

In bf16 at head dim 64 or 128 (C a multiple of 8, at most 4096) the whole
sublayer is one autograd function whose steps are the library's kernels and
hipBLASLt GEMMs:
  * LayerNorm forward and its gradient are the HIP row passes
    (attn_layernorm_fwd / attn_layernorm_bwd); the gradient adds the residual
    branch's dy to dx in the same pass, and recomputes the row statistics;
  * the attention reads q, k, v straight out of the c_attn output and writes
    its result in the merged [B, T, C] layout (strided views, no split or
    merge copies);
  * the two linear layers are GEMMs (torch.addmm / mm); their weight
    gradients u^T dqkv and a^T dy, reductions over all B*T rows, are taken
    as a batch of GEMMs over row blocks with fp32 results (split K) that the
    library's column sum adds in fp32 and rounds once, because a single GEMM
    with a short output and a long reduction fills few compute units;
  * the bias gradients are the library's column sums (attn_colsum).
Other shapes use torch's LayerNorm and autograd around the attention op
(contiguous [B, H, T, D] copies when the head dim has no strided kernel).
Weights are stored [in, out] (qkv = u @ W_attn + b_attn).
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

from . import (attn_bwd_strided, attn_fwd_strided, causal_attention, causal_attention_qkv,
               colsum, colsum_workspace_bytes, layernorm_bwd, layernorm_fwd,
               layernorm_workspace_bytes, qkv_heads)


def _weight_grad(a: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """a^T g for a [N, K], g [N, M]: split K over row blocks (a batch of GEMMs
    with fp32 results), the blocks added in order in fp32 (attn_colsum on the
    fp32 partials) and rounded once to bf16.
    Block counts measured at the sublayer's shapes: 2 for the c_attn weight
    (K x M = 768 x 2304), 16 for c_proj (768 x 768)."""
    N, K = a.shape
    M = g.shape[1]
    parts = 2 if (K // 64) * (M // 64) >= 256 else 16
    while parts > 1 and (N % parts or N // parts < 256):
        parts //= 2
    if parts == 1:
        return torch.mm(a.t(), g)
    ap = a.view(parts, N // parts, K).transpose(1, 2)
    gp = g.view(parts, N // parts, M)
    part = torch.bmm(ap, gp, out_dtype=torch.float32)  # [parts, K, M]
    out = torch.empty((K, M), dtype=a.dtype, device=a.device)
    colsum(part.view(parts, K * M), out.view(K * M))  # the blocks in order, one rounding
    return out


def _bias_grad(g: torch.Tensor) -> torch.Tensor:
    N, M = g.shape
    out = torch.empty(M, dtype=g.dtype, device=g.device)
    ws = torch.empty(colsum_workspace_bytes(N, M), dtype=torch.uint8, device=g.device)
    colsum(g, out, ws)
    return out


class _Sublayer(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, ln_w, ln_b, w_attn, b_attn, w_proj, b_proj, n_head, eps):
        B, T, C = x.shape
        N = B * T
        D = C // n_head
        x2 = x.reshape(N, C).contiguous()
        u = torch.empty_like(x2)
        layernorm_fwd(x2, ln_w, ln_b, u, eps)
        qkv = torch.addmm(b_attn, u, w_attn)  # [N, 3C]
        q, k, v = qkv_heads(qkv.view(B, T, 3 * C), n_head)
        a = torch.empty((N, C), dtype=x.dtype, device=x.device)
        o = a.view(B, T, n_head, D).permute(0, 2, 1, 3)
        lse = torch.empty((B, n_head, T), dtype=torch.float32, device=x.device)
        attn_fwd_strided(q, k, v, o, lse)
        y = torch.addmm(b_proj, a, w_proj)
        y += x2
        ctx.save_for_backward(x2, ln_w, w_attn, w_proj, u, qkv, a, lse)
        ctx.n_head, ctx.eps = n_head, eps
        return y.view(B, T, C)

    @staticmethod
    def backward(ctx, dy):
        x2, ln_w, w_attn, w_proj, u, qkv, a, lse = ctx.saved_tensors
        n_head = ctx.n_head
        N, C = x2.shape
        B, T = lse.shape[0], lse.shape[2]
        D = C // n_head
        dy2 = dy.reshape(N, C).contiguous()
        # c_proj: y = x + a W_proj + b_proj
        dw_proj = _weight_grad(a, dy2)
        db_proj = _bias_grad(dy2)
        da = torch.mm(dy2, w_proj.t())
        # attention, on strided views of qkv, a and da
        q, k, v = qkv_heads(qkv.view(B, T, 3 * C), n_head)
        o = a.view(B, T, n_head, D).permute(0, 2, 1, 3)
        dO = da.view(B, T, n_head, D).permute(0, 2, 1, 3)
        dqkv = torch.empty_like(qkv)
        dq, dk, dv = qkv_heads(dqkv.view(B, T, 3 * C), n_head)
        delta = torch.empty_like(lse)
        attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta)
        # c_attn: qkv = u W_attn + b_attn
        dw_attn = _weight_grad(u, dqkv)
        db_attn = _bias_grad(dqkv)
        du = torch.mm(dqkv, w_attn.t())
        # LayerNorm, with the residual branch's dy added to dx
        dx = torch.empty_like(x2)
        dg = torch.empty_like(ln_w)
        db = torch.empty_like(ln_w)
        ws = torch.empty(layernorm_workspace_bytes(N, C), dtype=torch.uint8, device=x2.device)
        layernorm_bwd(x2, ln_w, du, dx, dg, db, ws, dres=dy2, eps=ctx.eps)
        return (dx.view(B, T, C), dg, db, dw_attn, db_attn, dw_proj, db_proj, None, None)


def _fused_ok(x, params, n_head: int) -> bool:
    C = x.shape[-1]
    return (x.dtype == torch.bfloat16 and all(p.dtype == torch.bfloat16 for p in params) and
            x.is_cuda and C % n_head == 0 and C // n_head in (64, 128) and C % 8 == 0 and
            C <= 4096 and all(p.is_contiguous() for p in params))


def attention_sublayer(x, ln_w, ln_b, w_attn, b_attn, w_proj, b_proj, n_head: int,
                       eps: float = 1e-5):
    """x: [B, T, C]; w_attn: [C, 3C]; w_proj: [C, C].  Returns y: [B, T, C]."""
    B, T, C = x.shape
    if C % n_head != 0:
        raise ValueError("n_embd must be divisible by n_head")
    if _fused_ok(x, (ln_w, ln_b, w_attn, b_attn, w_proj, b_proj), n_head):
        return _Sublayer.apply(x, ln_w, ln_b, w_attn, b_attn, w_proj, b_proj, n_head, float(eps))
    D = C // n_head
    u = F.layer_norm(x, (C,), ln_w, ln_b, eps).reshape(B * T, C)
    qkv = torch.addmm(b_attn, u, w_attn)  # [B*T, 3C]
    if D in (64, 128) and qkv.dtype == torch.bfloat16:
        a = causal_attention_qkv(qkv.view(B, T, 3 * C), n_head).view(B * T, C)
        return x + torch.addmm(b_proj, a, w_proj).reshape(B, T, C)
    q, k, v = qkv.split(C, dim=-1)

    def heads(z):
        return z.reshape(B, T, n_head, D).transpose(1, 2).contiguous()

    a = causal_attention(heads(q), heads(k), heads(v))
    a = a.transpose(1, 2).reshape(B * T, C)
    return x + torch.addmm(b_proj, a, w_proj).reshape(B, T, C)
