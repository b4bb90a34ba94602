"""GPU parity of the RoPE / QK-norm prologue (and its gradient) with the fp64
oracle, alone and in front of the attention (nanochat, section 9 lists RoPE and
QK norm among its attention's parts; standard forms as the reading).

Bar for the prologue's own outputs: |got - ref| <= 2^-8 |ref| + 2e-3, i.e. the
bf16 rounding of the result (at most 2^-9 relative) with room for the fp32
angle (position times a frequency rounded to fp32: under 2.5e-4 rad at
position 4096, which moves a unit-size pair by as much).  End to end, the
attention outputs keep the stated 2e-2; the q and k gradients get it times
max(1, q_gain * k_gain / rms(row)), the scale the prologue's Jacobian and the
normalised operands put on the attention's gradient errors, plus one bf16 step
of the value for the extra bf16 store between the two launches.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import rounding_model, tolerance

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
    # The prologue's gradient maps the attention's dq (dk) through the norm's
    # Jacobian, whose scale is gain / rms(row) (the rotation keeps lengths), and
    # the attention's own dq (dk) errors carry the other side's gain (dq sums
    # normalised keys, dk normalised queries): the stated 2e-2 times
    # max(1, q_gain * k_gain / rms(row)), plus one bf16 step of the value for the
    # extra bf16 store of the attention's gradient between the two launches.
    gain = 1.2 * 1.0
    rms = lambda x: np.sqrt(np.mean(x.double().numpy() ** 2, axis=-1, keepdims=True))
    for name, a, r, f in (("o", got_o, o, 1.0), ("dq", _np(g[0]), dq, gain / rms(q)),
                          ("dk", _np(g[1]), dk, gain / rms(k)), ("dv", _np(g[2]), dv, 1.0)):
        b = tolerance.BF16 * np.maximum(1.0, f) + (tolerance.ulp_bf16(r) if name in ("dq", "dk")
                                                   else 0.0)
        _note(f"    {name}: max err {float(np.abs(a - r).max()):.2e}, worst err / bar "
              f"{float((np.abs(a - r) / b).max()):.3f} (max|ref| {float(np.abs(r).max()):.2f})")
        assert np.all(np.isfinite(a)) and np.all(np.abs(a - r) <= b), name


def _oracle_given_operands(q, k, q_rot, k_rot, v, dO, p, window, D):
    """The oracle on exactly the values the kernels used: attention (and its
    gradient) on the GPU's bf16 q_rot and k_rot, then the prologue's gradient
    at the raw q and k; and the prologue itself, for q_rot and k_rot."""
    kw = dict(pos0=p.pos0, base=p.base, rope=p.rope, norm=p.qk_norm, eps=p.eps)
    s = oracle.widen_scale(1.0 / math.sqrt(D))
    o, lse = oracle.attn_fwd(q_rot, k_rot, v, s, window=window)
    dqa, dka, dv, _ = oracle.attn_bwd(q_rot, k_rot, v, dO, s, window=window)
    return dict(qa=oracle.rope_qknorm_fwd(q, gain=p.q_gain, **kw),
                ka=oracle.rope_qknorm_fwd(k, gain=p.k_gain, **kw), o=o, lse=lse, dv=dv,
                dq=oracle.rope_qknorm_bwd(q, dqa, gain=p.q_gain, **kw),
                dk=oracle.rope_qknorm_bwd(k, dka, gain=p.k_gain, **kw))


def _check_fused(got, q, k, q_rot, k_rot, v, dO, p, window, D):
    """q_rot, k_rot at the prologue's bar; o, lse, dv at the attention's
    (tests/tolerance.py, with the rounding model on the same operands); dq, dk
    at the attention's bar times max(1, q_gain * k_gain / rms(row)), the scale
    of the prologue's Jacobian and of the other side's normalised operand, plus
    one bf16 step of the value."""
    ref = _oracle_given_operands(q, k, q_rot, k_rot, v, dO, p, window, D)
    close(got["q_rot"], ref["qa"], "q_rot")
    close(got["k_rot"], ref["ka"], "k_rot")
    model = rounding_model.lazy(q_rot, k_rot, v, dO, oracle.widen_scale(1.0 / math.sqrt(D)),
                                window)
    for n in ("o", "lse", "dv"):
        tolerance.check(got[n], ref[n], f"fused {n}", "bf16", lambda n=n: model()[n])
    gain = (p.q_gain * p.k_gain) if p.qk_norm else 1.0
    rms = lambda x: np.sqrt(np.mean(x.double().numpy() ** 2, axis=-1, keepdims=True))
    for n, x in (("dq", q), ("dk", k)):
        f = gain / rms(x) if p.qk_norm else 1.0
        bar = tolerance.BF16 * np.maximum(1.0, f) + tolerance.ulp_bf16(ref[n])
        err = np.abs(got[n] - ref[n])
        _note(f"    {n}: max err {float(err.max()):.2e}, worst err / bar "
              f"{float((err / bar).max()):.3f}")
        assert np.all(np.isfinite(got[n])) and np.all(err <= bar), n


def _run_fused(q, k, v, dO, p, window, H, layout_qkv=True):
    import causal_head_self_amd as cat
    B, _, T, D = q.shape
    dev = torch.device("cuda")
    qkv = torch.cat([t.permute(0, 2, 1, 3).reshape(B, T, H * D) for t in (q, k, v)], -1).to(dev)
    qv, kv, vv = cat.qkv_heads(qkv, H)
    shape = (B, H, T, D)
    q_rot, k_rot = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(2))
    y = torch.empty((B, T, H * D), dtype=torch.bfloat16, device=dev)
    o = y.view(B, T, H, D).permute(0, 2, 1, 3)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    cat.attn_fwd_strided_rope(qv, kv, vv, o, lse, q_rot, k_rot, p, window=window)
    dqkv = torch.zeros_like(qkv)
    dq, dk, dv = cat.qkv_heads(dqkv, H)
    delta = torch.empty_like(lse)
    cat.attn_bwd_strided_rope(qv, kv, q_rot, k_rot, vv, o, lse, dO.to(dev), dq, dk, dv, delta, p,
                              window=window)
    torch.cuda.synchronize()
    return dict(q_rot=_np(q_rot), k_rot=_np(k_rot), o=_np(o), lse=_np(lse), dq=_np(dq),
                dk=_np(dk), dv=_np(dv))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rope,norm,pos0,window", [(True, True, 0, 0), (True, False, 0, 0),
                                                   (False, True, 0, 0), (True, True, 3000, 0),
                                                   (True, True, 17, 48)])
def test_fused_prologue_matches_oracle(D, rope, norm, pos0, window):
    """attn_fwd_strided_rope / attn_bwd_strided_rope on views of a [B, T, 3C]
    c_attn output against the oracle."""
    import causal_head_self_amd as cat
    B, H, T = 2, 3, 150
    _note(f"[rope] fused D={D} rope={rope} norm={norm} pos0={pos0} window={window}")
    q, k, v, dO, _ = _qkv(B, H, T, D, 2000 + D + pos0 + window)
    p = cat.Prologue(rope=rope, qk_norm=norm, pos0=pos0, q_gain=1.2, k_gain=0.9, eps=1e-6)
    got = _run_fused(q, k, v, dO, p, window, H)
    qr, kr = (torch.from_numpy(got[n]).to(torch.bfloat16) for n in ("q_rot", "k_rot"))
    _check_fused(got, q, k, qr, kr, v, dO, p, window, D)


@pytest.mark.parametrize("D", [64, 128])
def test_fused_prologue_agrees_with_the_two_pass_path(D):
    """The fused entry points against the prologue pass + strided attention +
    prologue-gradient pass on the same inputs: the same key pass bit for bit,
    q_rot within one bf16 step of the separate pass's output (its row sum of
    squares is taken in another order), the rest within twice the attention's
    bar of each other."""
    import causal_head_self_amd as cat
    B, H, T = 2, 2, 200
    _note(f"[rope] fused against two-pass D={D}")
    q, k, v, dO, qkv = _qkv(B, H, T, D, 2100 + D)
    dev = torch.device("cuda")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, dO))
    p = cat.Prologue(pos0=5, q_gain=1.2, k_gain=1.0)
    e = lambda: torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    lse1, lse2 = (torch.empty((B, H, T), dtype=torch.float32, device=dev) for _ in range(2))
    qr, kr, o1 = e(), e(), e()
    cat.attn_fwd_strided_rope(qd, kd, vd, o1, lse1, qr, kr, p)
    dq1, dk1, dv1 = e(), e(), e()
    cat.attn_bwd_strided_rope(qd, kd, qr, kr, vd, o1, lse1, gd, dq1, dk1, dv1,
                              torch.empty_like(lse1), p)
    qa, ka, o2 = e(), e(), e()
    cat.rope_qknorm_fwd(qd, kd, qa, ka, p)
    cat.attn_fwd_strided(qa, ka, vd, o2, lse2)
    dqa, dka, dv2 = e(), e(), e()
    cat.attn_bwd_strided(qa, ka, vd, o2, lse2, gd, dqa, dka, dv2, torch.empty_like(lse2))
    dq2, dk2 = e(), e()
    cat.rope_qknorm_bwd(qd, kd, dqa, dka, dq2, dk2, p)
    torch.cuda.synchronize()
    assert torch.equal(kr, ka)
    assert np.all(np.abs(_np(qr) - _np(qa)) <= tolerance.ulp_bf16(_np(qa)))
    for n, a_, b_ in (("o", o1, o2), ("lse", lse1, lse2), ("dv", dv1, dv2), ("dq", dq1, dq2),
                      ("dk", dk1, dk2)):
        d = float(np.abs(_np(a_) - _np(b_)).max())
        _note(f"    {n}: fused - two-pass max {d:.2e}")
        assert d <= 2 * tolerance.BF16, n


def test_fused_prologue_full_size_every_head():
    """The gpt2s shape (B8 H12 T1024 D64) on the c_attn layout with RoPE and QK
    norm (gain 1.2): every head against the oracle."""
    import causal_head_self_amd as cat
    c = workloads.ATTN_CONFIGS["gpt2s"]
    B, H, T, D = c.B, c.H, c.T, c.D
    _note(f"[rope] fused full size B={B} H={H} T={T} D={D}")
    q, k, v, dO, _ = _qkv(B, H, T, D, 42)
    p = cat.Prologue(pos0=0, q_gain=1.2, k_gain=1.0)
    got = _run_fused(q, k, v, dO, p, 0, H)
    qr, kr = (torch.from_numpy(got[n]).to(torch.bfloat16) for n in ("q_rot", "k_rot"))
    _check_fused(got, q, k, qr, kr, v, dO, p, 0, D)
