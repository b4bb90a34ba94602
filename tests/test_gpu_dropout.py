"""GPU parity of attention dropout with the fp64 oracle (CS336 tutorial,
section 5.1: the softmax weights pass through nn.Dropout before the product
with v; inverted dropout in training mode, keep decisions from Philox4x32-10).

The keep decisions are integer results and are compared exactly: with q = 0
every visible weight of row i is 1/(i+1), and with v = the identity (D >= T)
o[i][j] is nonzero exactly when weight (i, j) is kept.  Values: dropout scales
kept weights by 1/(1-p), and with them the rounding errors of every product
they enter: the stated 2e-2 holds except where the stated roundings alone (the
CPU rounding model, with the same keep decisions) miss it, and then only by
what they cost there (tests/tolerance.py).
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


def gpu_drop(q, k, v, dO, p, seed, window=0):
    import causal_head_self_amd as cat
    dev = torch.device("cuda")
    q, k, v, dO = (t.to(dev).contiguous() for t in (q, k, v, dO))
    B, H, T, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    cat.attn_fwd_strided(q, k, v, o, lse, window=window, dropout_p=p, seed=seed)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)
    cat.attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, window=window, dropout_p=p,
                         seed=seed)
    torch.cuda.synchronize()
    out = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()}


def check(got, ref, label, dO=None, model=None):
    for name in ref:
        a, r = got[name], ref[name]
        if name == "delta":  # defined on the stored bf16 o (as without dropout)
            bound = np.sum(np.abs(dO) * (2.0 ** -8 * np.abs(got["o"]) + 4e-3), axis=-1) + 1e-4
            assert np.all(np.abs(a - r) <= bound), f"{label} delta"
            continue
        _note(f"    {name}: max err {float(np.abs(a - r).max()):.2e} "
              f"(max|ref| {float(np.abs(r).max()):.2f})")
        mf = None if model is None else (lambda n=name: model()[n])
        tolerance.check(a, r, f"{label} {name}", "bf16", mf)


@pytest.mark.parametrize("T,D,window", [(64, 64, 0), (40, 128, 0), (64, 64, 20)])
def test_keep_mask_is_bit_exact(T, D, window):
    """q = 0, v = I: o[i][j] = keep(i, j) / ((1 - p) * n_i) for the n_i visible
    keys of row i, so the kept set is read straight off o."""
    B, H, p, seed = 2, 2, 0.3, 0x5EED5EED1234
    _note(f"[dropout] mask B={B} H={H} T={T} D={D} window={window} p={p}")
    q = torch.zeros(B, H, T, D, dtype=torch.bfloat16)
    k = workloads.attention_inputs(B, H, T, D, "bf16", 5)[1]
    v = torch.zeros(B, H, T, D, dtype=torch.bfloat16)
    v[:, :, torch.arange(T), torch.arange(T)] = 1.0
    got = gpu_drop(q, k, v, torch.zeros_like(q), p, seed, window)
    p16 = oracle.dropout_threshold(p)
    mism = 0
    for bh in range(B * H):
        b, h = divmod(bh, H)
        for i in range(T):
            lo = max(0, i - window + 1) if window else 0
            for j in range(T):
                kept = lo <= j <= i and oracle.dropout_keep(seed, p16, bh, i, j)
                mism += (got["o"][b, h, i, j] != 0.0) != kept
    assert mism == 0


@pytest.mark.parametrize("shape,p,window", [
    ((1, 2, 200, 64), 0.1, 0), ((2, 1, 130, 64), 0.5, 0), ((1, 2, 257, 64), 0.2, 48),
    ((1, 2, 150, 128), 0.25, 0)])
def test_dropout_matches_oracle(shape, p, window):
    B, H, T, D = shape
    seed = 1234567 + T
    _note(f"[dropout] B={B} H={H} T={T} D={D} p={p} window={window}")
    q, k, v, dO = workloads.attention_inputs(B, H, T, D, "bf16", 1300 + T + D)
    got = gpu_drop(q, k, v, dO, p, seed, window)
    s = oracle.widen_scale(1.0 / math.sqrt(D))
    o, lse = oracle.attn_fwd_dropout(q, k, v, s, p, seed, window=window)
    dq, dk, dv, delta = oracle.attn_bwd_dropout(q, k, v, dO, s, p, seed, window=window)
    check(got, dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta), f"p{p} T{T} D{D}",
          dO.double().numpy(), rounding_model.lazy(q, k, v, dO, s, window, p, seed))


def test_dropout_seed_determinism():
    B, H, T, D = 1, 2, 128, 64
    _note("[dropout] seeds")
    q, k, v, dO = workloads.attention_inputs(B, H, T, D, "bf16", 17)
    a = gpu_drop(q, k, v, dO, 0.3, 99)
    b = gpu_drop(q, k, v, dO, 0.3, 99)
    c = gpu_drop(q, k, v, dO, 0.3, 100)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    assert not np.array_equal(a["o"], c["o"])


def test_qkv_autograd_with_dropout():
    import causal_head_self_amd as cat
    B, H, T, D, p, seed = 1, 2, 100, 64, 0.2, 4242
    _note(f"[dropout] causal_attention_qkv p={p}")
    q, k, v, dO = workloads.attention_inputs(B, H, T, D, "bf16", 1401)
    dev = torch.device("cuda")
    qkv = torch.cat([t.permute(0, 2, 1, 3).reshape(B, T, H * D) for t in (q, k, v)], dim=-1)
    x = qkv.to(dev).requires_grad_(True)
    y = cat.causal_attention_qkv(x, H, dropout_p=p, seed=seed)
    y.backward(dO.permute(0, 2, 1, 3).reshape(B, T, H * D).to(dev))
    torch.cuda.synchronize()
    s = oracle.widen_scale(1.0 / math.sqrt(D))
    o, _ = oracle.attn_fwd_dropout(q, k, v, s, p, seed)
    dq, dk, dv, _ = oracle.attn_bwd_dropout(q, k, v, dO, s, p, seed)
    as_np = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    g = x.grad.view(B, T, 3, H, D).permute(2, 0, 3, 1, 4)
    got = dict(o=as_np(y.view(B, T, H, D).permute(0, 2, 1, 3)), dq=as_np(g[0]), dk=as_np(g[1]),
               dv=as_np(g[2]))
    check(got, dict(o=o, dq=dq, dk=dk, dv=dv), "qkv dropout", None,
          rounding_model.lazy(q, k, v, dO, s, 0, p, seed))


@pytest.mark.parametrize("shape,p,window", [
    ((2, 3, 200, 64), 0.2, 0), ((1, 2, 130, 128), 0.3, 50), ((2, 2, 257, 64), 0.1, 0),
    ((1, 1, 33, 64), 0.5, 0), ((1, 2, 300, 64), 0.25, 64)])
def test_stored_keep_bits(shape, p, window):
    """attn_fwd_strided_keep / attn_bwd_strided_keep give the same bits as the
    entry points that draw, and every stored word of a visible (query, key)
    pair holds the oracle's keep decision (bit t of word (bh, w, i) is key
    32w + t)."""
    import causal_head_self_amd as cat
    B, H, T, D = shape
    seed = 0xC0FFEE + T
    _note(f"[dropout] stored keep bits B={B} H={H} T={T} D={D} p={p} window={window}")
    dev = torch.device("cuda")
    q, k, v, dO = (t.to(dev).contiguous()
                   for t in workloads.attention_inputs(B, H, T, D, "bf16", 1500 + T))

    def run(keep):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta = torch.empty_like(lse)
        if keep is None:
            cat.attn_fwd_strided(q, k, v, o, lse, window=window, dropout_p=p, seed=seed)
            cat.attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, window=window,
                                 dropout_p=p, seed=seed)
        else:
            cat.attn_fwd_strided_keep(q, k, v, o, lse, keep, window=window, dropout_p=p,
                                      seed=seed)
            cat.attn_bwd_strided_keep(q, k, v, o, lse, dO, dq, dk, dv, delta, keep,
                                      window=window, dropout_p=p)
        torch.cuda.synchronize()
        return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)

    ref = run(None)
    keep = torch.full((cat.dropout_keep_bytes(B, H, T) // 4,), -1, dtype=torch.int32, device=dev)
    got = run(keep)
    for n in ref:
        assert torch.equal(got[n], ref[n]), n
    words = keep.cpu().numpy().astype(np.uint32).reshape(B * H, (T + 31) // 32, T)
    p16 = oracle.dropout_threshold(p)
    checked = 0
    for bh in range(B * H):
        for i in range(T):
            lo = max(0, i - window + 1) if window else 0
            for j in range(lo, i + 1):
                bit = (int(words[bh, j // 32, i]) >> (j % 32)) & 1
                assert bit == int(oracle.dropout_keep(seed, p16, bh, i, j)), (bh, i, j)
                checked += 1
    _note(f"    {checked} keep decisions checked")


def test_stored_keep_bits_past_2_32_bytes():
    """Dropout p = 0.1 with stored keep bits at B=2 H=17000 T=1000 D=64: every
    tensor holds 2.18e9 elements and the keep buffer takes 4.35 GB, so the keep
    words of the last heads sit past 2^32 bytes.  The sampled heads (the first,
    those that straddle 2^30 and 2^31 tensor elements, and the last) match the
    oracle, given each head's global index, element by element, and 4000 sampled
    stored words of each hold the oracle's keep decisions."""
    import causal_head_self_amd as cat
    B, H, T, D = 2, 17000, 1000, 64
    p, seed = 0.1, 0xBEEF
    per_head, n_words = T * D, (T + 31) // 32
    _note(f"[dropout] stored keep bits B={B} H={H} T={T} D={D} p={p}: "
          f"keep buffer {cat.dropout_keep_bytes(B, H, T)} bytes")
    dev = torch.device("cuda")
    q, k, v, dO = workloads.device_attention_inputs(B, H, T, D, dev, seed=77)
    scale = 1.0 / math.sqrt(D)
    keep = torch.full((cat.dropout_keep_bytes(B, H, T) // 4,), -1, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)
    cat.attn_fwd_strided_keep(q, k, v, o, lse, keep, scale=scale, dropout_p=p, seed=seed)
    cat.attn_bwd_strided_keep(q, k, v, o, lse, dO, dq, dk, dv, delta, keep, scale=scale,
                              dropout_p=p)
    torch.cuda.synchronize()
    p16 = oracle.dropout_threshold(p)
    rng = np.random.default_rng(5)
    for bh in [0, 2 ** 30 // per_head, 2 ** 31 // per_head, B * H - 1]:
        b, h = divmod(bh, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        cpu = lambda t: t[sl].cpu()
        got = {n: t[sl].float().cpu().numpy().astype(np.float64)
               for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                            ("delta", delta))}
        ro, rl = oracle.attn_fwd_dropout(cpu(q), cpu(k), cpu(v), scale, p, seed, bh0=bh)
        rq, rk, rv, rd = oracle.attn_bwd_dropout(cpu(q), cpu(k), cpu(v), cpu(dO), scale, p,
                                                 seed, bh0=bh)
        _note(f"  head {bh}: keep words from byte {bh * n_words * T * 4}")
        check(got, dict(o=ro, lse=rl, dq=rq, dk=rk, dv=rv, delta=rd), f"head {bh}",
              cpu(dO).double().numpy(),
              rounding_model.lazy(cpu(q), cpu(k), cpu(v), cpu(dO), oracle.widen_scale(scale), 0, p,
                                  seed, bh0=bh))
        words = keep[bh * n_words * T:(bh + 1) * n_words * T].cpu().numpy().astype(np.uint32)
        words = words.reshape(n_words, T)
        for _ in range(4000):
            i = int(rng.integers(0, T))
            j = int(rng.integers(0, i + 1))
            bit = (int(words[j // 32, i]) >> (j % 32)) & 1
            assert bit == int(oracle.dropout_keep(seed, p16, bh, i, j)), (bh, i, j)
    del q, k, v, dO, o, dq, dk, dv, keep
    torch.cuda.empty_cache()
