"""attn_decode_noalloc (the decode entry point for callers that cannot allocate:
its split path keeps the per-slice partials in the library's fixed device
scratch) against attn_decode with a caller workspace, through the C ABI.

Both run the same kernels, so their outputs must agree bit for bit; both must
also match the fp64 oracle at the stated 2e-2 bar.  Two calls in a row, the
second on a smaller problem, show that the shared scratch needs no clearing.
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


def _run_pair(B, H, T_max, D, lens, window=0):
    import causal_head_self_amd as cat
    dev = torch.device("cuda")
    q, kc, vc = workloads.decode_inputs(B, H, T_max, D, seed=900 + T_max)
    qd, kd, vd = (t.to(dev) for t in (q, kc, vc))
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    o1 = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    lse1 = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(cat.decode_workspace_bytes(B, H, T_max, D), dtype=torch.uint8, device=dev)
    cat.attn_decode(qd, kd, vd, ln, o1, lse1, ws, scale, window)
    o2 = torch.full_like(o1, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    cat.attn_decode_noalloc(qd, kd, vd, ln, o2, lse2, scale, window)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "o differs from attn_decode"
    assert torch.equal(lse1, lse2), "lse differs from attn_decode"
    ro, rl = oracle.attn_decode(q, kc, vc, lens, oracle.widen_scale(scale), window=window)
    got_o = o2.float().cpu().numpy().astype(np.float64)
    got_l = lse2.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_o - ro)) <= 2e-2
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.max(np.abs(got_l[fin] - rl[fin]), initial=0.0) <= 2e-2


@pytest.mark.parametrize("D", [64, 128])
def test_noalloc_matches_attn_decode_on_two_calls(D):
    """Both calls take the two-launch path (few heads, caches longer than one
    workgroup's waves cover), so both use the scratch; the second is smaller and
    reads only what it wrote."""
    big = (1, 4, 3000) if D == 64 else (1, 3, 1400)
    small = (1, 2, 1500) if D == 64 else (1, 2, 700)
    for (B, H, T_max), lens in ((big, [big[2] - 7]), (small, [small[2] // 2 + 3])):
        _note(f"[noalloc] D={D} B={B} H={H} T_max={T_max} lens={lens}")
        _run_pair(B, H, T_max, D, lens)


def test_noalloc_one_launch_path_needs_no_scratch():
    """128 heads take the one-launch path, which uses no scratch: a shape whose
    split-path partials would exceed the scratch is accepted (caches of 0.5 GB
    each, drawn on the device; two sequences against the oracle)."""
    import causal_head_self_amd as cat
    B, H, T_max, D = 8, 16, 31000, 64
    assert cat.decode_workspace_bytes(B, H, T_max, D) > cat.DECODE_SCRATCH_BYTES
    _note(f"[noalloc] one launch B={B} H={H} T_max={T_max} D={D}")
    dev = torch.device("cuda")
    q, kc, vc = workloads.device_decode_inputs(B, H, T_max, D, dev, seed=31)
    lens = [T_max - 977 * b for b in range(B)]
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    o1 = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    lse1 = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(cat.decode_workspace_bytes(B, H, T_max, D), dtype=torch.uint8, device=dev)
    cat.attn_decode(q, kc, vc, ln, o1, lse1, ws)
    o2, lse2 = torch.full_like(o1, float("nan")), torch.full_like(lse1, float("nan"))
    cat.attn_decode_noalloc(q, kc, vc, ln, o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    s = oracle.widen_scale(1.0 / math.sqrt(D))
    for b in (0, B - 1):
        ro, rl = oracle.attn_decode(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                    [lens[b]], s)
        assert np.max(np.abs(o2[b:b + 1].float().cpu().numpy() - ro)) <= 2e-2
        assert np.max(np.abs(lse2[b:b + 1].cpu().numpy() - rl)) <= 2e-2
    del q, kc, vc, ws
    torch.cuda.empty_cache()


def test_noalloc_rejects_split_path_beyond_the_scratch():
    import causal_head_self_amd as cat
    B, H, T_max, D = 1, 100, 40000, 64
    need = cat.decode_workspace_bytes(B, H, T_max, D)
    assert need > cat.DECODE_SCRATCH_BYTES
    _note(f"[noalloc] rejection B={B} H={H} T_max={T_max} D={D}: {need} bytes of partials")
    dev = torch.device("cuda")
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((B, T_max, H, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    ln = torch.full((B,), T_max, dtype=torch.int32, device=dev)
    o = torch.full((B, H, D), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(cat.AttnError) as e:
        cat.attn_decode_noalloc(q, kc, vc, ln, o, lse)
    assert e.value.status == 13  # ATTN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())  # nothing was enqueued
