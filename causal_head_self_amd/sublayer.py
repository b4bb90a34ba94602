"""Pre-norm causal self-attention sublayer around the HIP attention op.

    y = x + c_proj(merge_heads(attention(split_heads(c_attn(LN(x))))))

This follows the CS336 from-scratch tutorial (lmnt.cn), section 5.1 model.py:
Block.forward adds attn(ln_1(x)) to x (pre-norm, section 3.4), and
CausalSelfAttention runs c_attn (C -> 3C), chunks the result into q, k, v,
views each as [B, T, H, D] -> [B, H, T, D], attends, merges the heads back and
applies c_proj (C -> C).  LayerNorm uses the biased variance and eps 1e-5
(class LayerNorm on the same page).

Only the attention core is a hand-written kernel here; LayerNorm and the two
linear layers are PyTorch-ROCm library calls (hipBLASLt GEMMs).  At head dim
64 in bf16 the attention reads q, k, v straight out of the c_attn output and
writes its result in the merged [B, T, C] layout (strided views, no split or
merge copies); other shapes go through contiguous [B, H, T, D] copies.
Weights are stored [in, out] (qkv = u @ W_attn + b_attn).
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

from . import causal_attention, causal_attention_qkv


def attention_sublayer(x, ln_w, ln_b, w_attn, b_attn, w_proj, b_proj, n_head: int,
                       eps: float = 1e-5):
    """x: [B, T, C]; w_attn: [C, 3C]; w_proj: [C, C].  Returns y: [B, T, C]."""
    B, T, C = x.shape
    if C % n_head != 0:
        raise ValueError("n_embd must be divisible by n_head")
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
