"""GPU parity of attn_decode (one new token per sequence against its KV cache)
with the fp64 oracle.

Decode follows nanochat, section 8: a (B, T, H, D) cache, prefilled, then one
token at a time; the token at position len-1 attends to positions 0..len-1
(the W most recent with a window).  All arithmetic after the bf16 loads is
fp32, so the 2e-2 bar of the bf16 configurations is met with a wide margin;
the largest error is printed for each case.  The cases cover both paths of the
library: one launch (T_max <= 1024 at D = 64, 512 at D = 128, or B*H at least
half the compute units) and the two-launch split (few heads, longer caches).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_decode(q, kc, vc, lens, window=0, scale=None):
    import causal_head_self_amd as cat
    dev = torch.device("cuda")
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    o, lse = cat.decode_attention(q.to(dev), kc.to(dev), vc.to(dev), ln, scale, window)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_decode(q, kc, vc, lens, window=0):
    D = q.shape[-1]
    return oracle.attn_decode(q, kc, vc, [min(max(n, 0), kc.shape[1]) for n in lens],
                              oracle.widen_scale(1.0 / math.sqrt(D)), window=window)


def check(q, kc, vc, lens, window, label):
    o, lse = gpu_decode(q, kc, vc, lens, window)
    ro, rlse = oracle_decode(q, kc, vc, lens, window)
    empty = np.isneginf(rlse)  # sequences with nothing cached: o = 0, lse = -inf
    assert np.array_equal(np.isneginf(lse), empty), f"{label}: empty sequences"
    assert np.all(o[empty] == 0.0), f"{label}: o of an empty sequence"
    eo = float(np.abs(o - ro).max())
    el = float(np.abs(lse[~empty] - rlse[~empty]).max()) if (~empty).any() else 0.0
    _note(f"    max |o - ref| {eo:.2e}, max |lse - ref| {el:.2e}")
    assert np.all(np.isfinite(o)), f"{label}: non-finite o"
    assert eo <= TOL, f"{label}: o error {eo:.3e}"
    assert el <= TOL, f"{label}: lse error {el:.3e}"
    return o, lse


@pytest.mark.parametrize("B,H,T_max,D,lens,window", [
    (3, 4, 200, 64, [200, 1, 77], 0),
    (3, 4, 200, 64, [200, 1, 77], 5),
    (3, 4, 200, 64, [200, 64, 65], 64),
    (2, 2, 300, 64, [300, 129], 100),
    (2, 2, 300, 128, [300, 129], 0),
    (2, 3, 257, 128, [257, 63], 31),
    (1, 1, 1, 64, [1], 0),
    (4, 2, 130, 64, [0, 130, 500, -3], 0),   # nothing cached, full, clamped above and below
    (1, 12, 1024, 64, [1024], 0),
    # two launches (few heads, more slices than waves in a one-launch workgroup)
    (2, 2, 1500, 64, [1500, 1100], 300),
    (2, 3, 700, 128, [700, 65], 0),
    # one launch with two slices for some waves (many heads, long caches)
    (1, 130, 1100, 64, [1100], 0),
    (1, 130, 600, 128, [600], 200),
])
def test_decode_matches_oracle(B, H, T_max, D, lens, window):
    _note(f"[decode] B={B} H={H} T_max={T_max} D={D} lens={lens} window={window}")
    q, kc, vc = workloads.decode_inputs(B, H, T_max, D, seed=700 + T_max + D + window)
    check(q, kc, vc, lens, window, f"B{B} H{H} T{T_max} D{D} W{window}")


@pytest.mark.parametrize("name", sorted(workloads.DECODE_CONFIGS))
def test_decode_full_configs(name):
    c = workloads.DECODE_CONFIGS[name]
    _note(f"[decode] config {name} B={c.B} H={c.H} T_max={c.T_max} D={c.D} (every head)")
    q, kc, vc = workloads.decode_inputs(c.B, c.H, c.T_max, c.D)
    check(q, kc, vc, c.lens(), 0, name)


def test_decode_ignores_rows_outside_the_visible_range():
    """Rows at or past len (and before a window) hold NaN and +-inf here; the
    results must equal those on a clean cache bit for bit."""
    B, H, T_max, D, W = 2, 3, 256, 64, 50
    lens = [180, 70]
    _note(f"[decode] poisoned rows B={B} H={H} T_max={T_max} lens={lens} W={W}")
    q, kc, vc = workloads.decode_inputs(B, H, T_max, D, seed=811)
    o1, l1 = gpu_decode(q, kc, vc, lens, W)
    kp, vp = kc.clone(), vc.clone()
    for b, n in enumerate(lens):
        kp[b, n:] = float("nan")
        vp[b, n:] = float("inf")
        kp[b, :n - W] = float("-inf")
        vp[b, :n - W] = float("nan")
    o2, l2 = gpu_decode(q, kp, vp, lens, W)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_deterministic_and_workspace_reuse():
    """Two calls give the same bits; one workspace serves a large call and then
    a smaller one (its content on entry does not matter)."""
    import causal_head_self_amd as cat
    dev = torch.device("cuda")
    _note("[decode] workspace reuse")
    big = workloads.decode_inputs(4, 6, 700, 64, seed=901)
    small = workloads.decode_inputs(2, 3, 90, 128, seed=902)
    ws = torch.full((cat.decode_workspace_bytes(4, 6, 700, 128),), 255, dtype=torch.uint8,
                    device=dev)
    outs = []
    for (q, kc, vc), lens in ((big, [700, 1, 350, 699]), (small, [90, 45]),
                              (big, [700, 1, 350, 699])):
        B, T_max, H, D = kc.shape
        o = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        ln = torch.tensor(lens, dtype=torch.int32, device=dev)
        cat.attn_decode(q.to(dev), kc.to(dev), vc.to(dev), ln, o, lse, ws)
        torch.cuda.synchronize()
        ro, rl = oracle_decode(q, kc, vc, lens)
        assert np.abs(o.float().cpu().numpy() - ro).max() <= TOL
        assert np.abs(lse.cpu().numpy() - rl).max() <= TOL
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])


def test_decode_equals_last_row_of_prefill_forward():
    """Prefill then decode: the decoded token's output matches row len-1 of the
    causal forward over the same sequence (both within the bar of the oracle,
    and of each other)."""
    import causal_head_self_amd as cat
    B, H, T, D = 2, 4, 160, 64
    _note(f"[decode] prefill/decode consistency B={B} H={H} T={T}")
    q, k, v, _ = workloads.attention_inputs(B, H, T, D, "bf16", 933)
    dev = torch.device("cuda")
    o_full = cat.causal_attention(q.to(dev), k.to(dev), v.to(dev))
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    for n in (1, 64, 100, T):
        o, _ = gpu_decode(q[:, :, n - 1].contiguous(), kc, vc, [n] * B)
        full = o_full[:, :, n - 1].float().cpu().numpy()
        assert np.abs(o - full).max() <= 2 * TOL


@pytest.mark.parametrize("B,H,T_max,D,one_launch", [
    (66, 16, 32768, 64, True),       # 1056 heads: one launch
    (1, 100, 336544, 64, False),     # 100 heads, 5259 slices each: two launches
])
def test_decode_caches_past_2_31_elements(B, H, T_max, D, one_launch):
    """K/V caches of more than 2^31 elements (4.3-4.4 GB each in bf16), so the
    positions of the last sequences and heads lie past 2^31 elements.  Each
    case takes the path named (the library's rule: one launch when every wave
    of a workgroup has at most one 64-position slice or when B*H reaches half
    the compute units).  Sampled (sequence, head) pairs, the last one included,
    are compared with the oracle on that head alone."""
    import causal_head_self_amd as cat
    assert B * T_max * H * D > 2 ** 31
    dev = torch.device("cuda")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    assert (-(-T_max // 64) <= 16 or 2 * B * H >= n_cu) == one_launch
    _note(f"[decode] B={B} H={H} T_max={T_max} D={D}: caches of {B * T_max * H * D} elements, "
          f"{'one launch' if one_launch else 'two launches'}")
    q, kc, vc = workloads.device_decode_inputs(B, H, T_max, D, dev, seed=91)
    lens = [T_max - 37 * b for b in range(B)]
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    o, lse = cat.decode_attention(q, kc, vc, ln, scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    for b, h in [(0, 0), (B // 2, H // 3), (B - 1, H - 1)]:
        n = lens[b]
        ro, rlse = oracle.attn_decode(q[b:b + 1, h:h + 1].cpu(), kc[b:b + 1, :n, h:h + 1].cpu(),
                                      vc[b:b + 1, :n, h:h + 1].cpu(), [n],
                                      oracle.widen_scale(scale))
        eo = float(np.abs(o[b, h].float().cpu().numpy() - ro[0, 0]).max())
        el = abs(float(lse[b, h]) - float(rlse[0, 0]))
        _note(f"    (b={b}, h={h}) len {n}: max |o - ref| {eo:.2e}, |lse - ref| {el:.2e}")
        assert eo <= TOL and el <= TOL, (b, h, eo, el)
    del q, kc, vc
    torch.cuda.empty_cache()
