"""GPU parity of the RoPE / QK-norm prologue (and its gradient) with the fp64
oracle, alone and in front of the attention (nanochat, section 9 lists RoPE and
QK norm among its attention's parts; standard forms as the reading).

Bar for the prologue's own outputs: |got - ref| <= 2^-8 |ref| + 2e-3, i.e. the
bf16 rounding of the result (at most 2^-9 relative) with room for the fp32
angle (position times a frequency rounded to fp32: under 2.5e-4 rad at
position 4096, which moves a unit-size pair by as much).  End to end, the
attention outputs keep the 2e-2 bar (applied to max(1, |ref|) for the
gradients, which the prologue scales by the gain over the row's RMS).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def close(got, ref, label, rel=2.0 ** -8, abs_=2e-3):
    err = np.abs(got - ref) - (rel * np.abs(ref) + abs_)
    worst = float(np.abs(got - ref).max())
    _note(f"    {label}: max abs err {worst:.2e}")
    assert np.all(np.isfinite(got)), f"{label}: non-finite"
    assert np.all(err <= 0), f"{label}: beyond bound at {np.argwhere(err > 0)[:4].tolist()}"


def _qkv(B, H, T, D, seed):
    q, k, v, dO = workloads.attention_inputs(B, H, T, D, "bf16", seed)
    qkv = torch.cat([t.permute(0, 2, 1, 3).reshape(B, T, H * D) for t in (q, k, v)], dim=-1)
    return q, k, v, dO, qkv


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rope,norm,pos0", [(True, False, 0), (False, True, 0), (True, True, 0),
                                            (True, True, 3000)])
def test_prologue_forward_and_gradient_match_oracle(D, rope, norm, pos0):
    import causal_head_self_amd as cat
    B, H, T = 2, 3, 150
    _note(f"[rope] D={D} rope={rope} norm={norm} pos0={pos0} B={B} H={H} T={T}")
    q, k, _, _, qkv = _qkv(B, H, T, D, 1000 + D + pos0)
    dev = torch.device("cuda")
    qkv = qkv.to(dev)
    qv, kv, _ = cat.qkv_heads(qkv, H)  # strided views of the c_attn layout
    p = cat.Prologue(rope=rope, qk_norm=norm, pos0=pos0, q_gain=1.2, k_gain=0.9, eps=1e-6)
    qo = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    ko = torch.empty_like(qo)
    cat.rope_qknorm_fwd(qv, kv, qo, ko, p)
    gq = workloads.attention_inputs(B, H, T, D, "bf16", 77)[3]
    gk = workloads.attention_inputs(B, H, T, D, "bf16", 78)[3]
    dqkv = torch.zeros_like(qkv)
    dq, dk, _ = cat.qkv_heads(dqkv, H)
    cat.rope_qknorm_bwd(qv, kv, gq.to(dev), gk.to(dev), dq, dk, p)
    torch.cuda.synchronize()
    kw = dict(pos0=pos0, rope=rope, norm=norm, eps=1e-6)
    close(_np(qo), oracle.rope_qknorm_fwd(q, gain=1.2, **kw), "q_out")
    close(_np(ko), oracle.rope_qknorm_fwd(k, gain=0.9, **kw), "k_out")
    close(_np(dq), oracle.rope_qknorm_bwd(q, gq, gain=1.2, **kw), "dq")
    close(_np(dk), oracle.rope_qknorm_bwd(k, gk, gain=0.9, **kw), "dk")
    assert torch.all(dqkv[..., 2 * H * D:] == 0)  # the v third is not touched


@pytest.mark.parametrize("D,window", [(64, 0), (128, 0), (64, 48)])
def test_attention_with_prologue_matches_oracle(D, window):
    """causal_attention_qkv(..., prologue) forward and backward against the
    oracle chain: prologue -> causal attention -> its gradient -> prologue
    gradient."""
    import causal_head_self_amd as cat
    B, H, T = 2, 2, 200
    _note(f"[rope] attention with prologue D={D} window={window} B={B} H={H} T={T}")
    q, k, v, dO, qkv = _qkv(B, H, T, D, 1100 + D + window)
    dev = torch.device("cuda")
    x = qkv.to(dev).requires_grad_(True)
    p = cat.Prologue(pos0=0, q_gain=1.2, k_gain=1.0)
    y = cat.causal_attention_qkv(x, H, window=window, prologue=p)
    y.backward(dO.permute(0, 2, 1, 3).reshape(B, T, H * D).to(dev))
    torch.cuda.synchronize()
    s = oracle.widen_scale(1.0 / math.sqrt(D))
    qa = oracle.rope_qknorm_fwd(q, gain=1.2)
    ka = oracle.rope_qknorm_fwd(k, gain=1.0)
    o, _ = oracle.attn_fwd(qa, ka, v, s, window=window)
    dqa, dka, dv, _ = oracle.attn_bwd(qa, ka, v, dO, s, window=window)
    dq = oracle.rope_qknorm_bwd(q, dqa, gain=1.2)
    dk = oracle.rope_qknorm_bwd(k, dka, gain=1.0)
    got_o = _np(y.view(B, T, H, D).permute(0, 2, 1, 3))
    g = x.grad.view(B, T, 3, H, D).permute(2, 0, 3, 1, 4)
    for name, a, r in (("o", got_o, o), ("dq", _np(g[0]), dq), ("dk", _np(g[1]), dk),
                       ("dv", _np(g[2]), dv)):
        err = np.abs(a - r) / (1.0 if name == "o" else np.maximum(1.0, np.abs(r)))
        _note(f"    {name}: max err {float(err.max()):.2e} (max|ref| {float(np.abs(r).max()):.2f})")
        assert np.all(np.isfinite(a)) and float(err.max()) <= 2e-2, name
