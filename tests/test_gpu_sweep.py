"""A seeded sweep of random combinations of the training-attention options
(batch, heads, ragged length, head dim, window, dropout, strided or contiguous
layout) against the fp64 oracle, element by element; with dropout, the entry
points with stored keep bits must give the same bits.  The cases are drawn
from a fixed seed, so every run checks the same list."""
import math
import random
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import rounding_model, tolerance

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=20261203):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        D = rng.choice([64, 64, 128])
        T = rng.randint(1, 400)
        window = rng.choice([0, 0, rng.randint(1, max(1, T + 10))])
        p = rng.choice([0.0, 0.0, 0.0, round(rng.uniform(0.05, 0.6), 3)])
        out.append((rng.randint(1, 3), rng.randint(1, 4), T, D, window, p, rng.random() < 0.5,
                    rng.randint(0, 2 ** 40)))
    return out


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,H,T,D,window,p,fused,seed", _cases())
def test_random_combination_matches_oracle(B, H, T, D, window, p, fused, seed):
    import causal_head_self_amd as cat
    _note(f"[sweep] B={B} H={H} T={T} D={D} window={window} p={p} fused_layout={fused}")
    q, k, v, dO = workloads.attention_inputs(B, H, T, D, "bf16", seed % 100000)
    dev = torch.device("cuda")
    scale = 1.0 / math.sqrt(D)
    if fused:  # q, k, v as views of one [B, T, 3C] buffer; o and grads in [B, T, C] / [B, T, 3C]
        qkv = torch.cat([t.permute(0, 2, 1, 3).reshape(B, T, H * D) for t in (q, k, v)], -1).to(dev)
        qd, kd, vd = cat.qkv_heads(qkv, H)
        y = torch.empty((B, T, H * D), dtype=torch.bfloat16, device=dev)
        od = y.view(B, T, H, D).permute(0, 2, 1, 3)
        dqkv = torch.empty_like(qkv)
        dqd, dkd, dvd = cat.qkv_heads(dqkv, H)
    else:
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        od = torch.empty_like(qd)
        dqd, dkd, dvd = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    gd = dO.to(dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    cat.attn_fwd_strided(qd, kd, vd, od, lse, scale, window=window, dropout_p=p, seed=seed)
    cat.attn_bwd_strided(qd, kd, vd, od, lse, gd, dqd, dkd, dvd, delta, scale, window=window,
                         dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    s = oracle.widen_scale(scale)
    if p > 0:
        ro, rl = oracle.attn_fwd_dropout(q, k, v, s, p, seed, window=window)
        rdq, rdk, rdv, _ = oracle.attn_bwd_dropout(q, k, v, dO, s, p, seed, window=window)
    else:
        ro, rl = oracle.attn_fwd(q, k, v, s, window=window)
        rdq, rdk, rdv, _ = oracle.attn_bwd(q, k, v, dO, s, window=window)
    as_np = lambda t: t.float().cpu().numpy().astype(np.float64)
    # the stated 2e-2, except where the stated roundings alone (the CPU rounding
    # model) miss it (tests/tolerance.py)
    model = rounding_model.lazy(q, k, v, dO, s, window, p, seed)
    got = dict(o=as_np(od), lse=as_np(lse), dq=as_np(dqd), dk=as_np(dkd), dv=as_np(dvd))
    tolerance.check_all(got, dict(o=ro, lse=rl, dq=rdq, dk=rdk, dv=rdv), "sweep", "bf16", model)
    if p > 0:  # the stored-keep-bit entry points give the same bits as the drawing ones
        keep = torch.full((cat.dropout_keep_bytes(B, H, T) // 4,), -1, dtype=torch.int32,
                          device=dev)
        o2, dq2, dk2, dv2 = (torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
                             for _ in range(4))
        lse2, delta2 = torch.empty_like(lse), torch.empty_like(delta)
        cat.attn_fwd_strided_keep(qd, kd, vd, o2, lse2, keep, scale, window=window, dropout_p=p,
                                  seed=seed)
        cat.attn_bwd_strided_keep(qd, kd, vd, o2, lse2, gd, dq2, dk2, dv2, delta2, keep, scale,
                                  window=window, dropout_p=p)
        torch.cuda.synchronize()
        for name, a, b in (("o", od, o2), ("lse", lse, lse2), ("dq", dqd, dq2), ("dk", dkd, dk2),
                           ("dv", dvd, dv2), ("delta", delta, delta2)):
            assert torch.equal(a.contiguous(), b), f"stored keep bits: {name}"
