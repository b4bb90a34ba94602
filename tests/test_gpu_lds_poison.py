"""Reads of LDS before it is written, caught with the LDS-poisoning build.

libcausal_attn_lds_poison.so is the same kernel sources compiled with
-DCATTN_LDS_POISON: every kernel fills its LDS arrays with all-ones words (NaN
as fp32 and as bf16) before it touches them.  A kernel that reads LDS it never
wrote -- a tile row past the end of a ragged input, an unwritten merge slot, a
buffer read before its copy landed -- then gives a different result (usually a
NaN) than the release library, whose LDS holds whatever an earlier workgroup
left.  Every entry point whose kernels use LDS runs here on both libraries,
and the outputs must agree bit for bit: ragged lengths, windows, dropout (drawn
and stored bits), the fused prologue, head dims 32, 64 and 128, fp32, both
backward forms, both decode paths, and the LayerNorm gradient (whose column
partials meet in LDS).
"""
import math
import os
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import causal_head_self_amd as cat
    from causal_head_self_amd import _lib
    from causal_head_self_amd import build as hip_build
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert os.path.exists(hip_build.LIB_POISON), (
        f"{hip_build.LIB_POISON} is not built: run `python -m causal_head_self_amd.build`")
    release = cat.load_library()
    poison = _lib.load_library(hip_build.LIB_POISON)
    return release, poison


def _both(libs, run):
    """run() with each library current; returns the two lists of outputs (CPU)."""
    from causal_head_self_amd import _lib
    saved = _lib._lib
    outs = []
    try:
        for lib in libs:
            _lib._lib = lib
            got = run()
            torch.cuda.synchronize()
            outs.append([t.detach().cpu().clone() for t in got])
    finally:
        _lib._lib = saved
    return outs


def _same(case, outs):
    a, b = outs
    assert len(a) == len(b)
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), (
            f"{case}: output {i} differs with LDS poisoned "
            f"(max |diff| {float((x.float() - y.float()).abs().nan_to_num(1e30).max()):.3g}, "
            f"NaN count {int(torch.isnan(y.float()).sum())})")


def _note(msg):
    print(msg)
    sys.stdout.flush()


def _inputs(B, H, T, D, dtype, seed):
    dev = torch.device("cuda")
    return [t.to(dev) for t in workloads.attention_inputs(B, H, T, D, dtype, seed)]


# (B, H, T, D, dtype): ragged lengths across the tile sizes of each kernel family
CONTIGUOUS = [
    (1, 2, 333, 64, "bf16"),
    (2, 1, 1000, 64, "bf16"),
    (1, 2, 200, 128, "bf16"),
    (1, 1, 77, 32, "bf16"),
    (2, 2, 130, 32, "bf16"),
    (1, 3, 200, 64, "f32"),
    (1, 2, 65, 32, "f32"),
]


@pytest.mark.parametrize("B,H,T,D,dtype", CONTIGUOUS)
def test_contiguous_forward_and_backward(libs, B, H, T, D, dtype):
    import causal_head_self_amd as cat
    _note(f"[lds poison] contiguous B={B} H={H} T={T} D={D} {dtype}")
    q, k, v, dO = _inputs(B, H, T, D, dtype, 11)

    def run():
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta = torch.empty_like(lse)
        cat.attn_fwd(q, k, v, o, lse)
        cat.attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta)
        # the two-stage backward (dQ and Delta, then dK/dV)
        dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta2 = torch.empty_like(lse)
        cat.attn_bwd_dq(q, k, v, o, dO, lse, delta2, dq2)
        cat.attn_bwd_dkdv(q, k, v, dO, lse, delta2, dk2, dv2)
        return [o, lse, dq, dk, dv, delta, dq2, dk2, dv2, delta2]

    _same(f"B={B} H={H} T={T} D={D} {dtype}", _both(libs, run))


@pytest.mark.parametrize("T,D,window,p", [(333, 64, 100, 0.0), (300, 64, 0, 0.1),
                                          (260, 64, 70, 0.2), (200, 128, 50, 0.1)])
def test_strided_window_dropout(libs, T, D, window, p):
    import causal_head_self_amd as cat
    B, H = 1, 2
    _note(f"[lds poison] strided T={T} D={D} window={window} p={p}")
    q, k, v, dO = _inputs(B, H, T, D, "bf16", 12)
    scale = 1.0 / math.sqrt(D)

    def run():
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta = torch.empty_like(lse)
        cat.attn_fwd_strided(q, k, v, o, lse, scale, window=window, dropout_p=p, seed=5)
        cat.attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, scale, window=window,
                             dropout_p=p, seed=5)
        out = [o, lse, dq, dk, dv, delta]
        if p > 0:
            keep = torch.zeros((cat.dropout_keep_bytes(B, H, T) // 4,), dtype=torch.int32,
                               device=q.device)
            o2, dq2, dk2, dv2 = (torch.empty_like(q) for _ in range(4))
            lse2, delta2 = torch.empty_like(lse), torch.empty_like(lse)
            cat.attn_fwd_strided_keep(q, k, v, o2, lse2, keep, scale, window=window,
                                      dropout_p=p, seed=5)
            cat.attn_bwd_strided_keep(q, k, v, o2, lse2, dO, dq2, dk2, dv2, delta2, keep, scale,
                                      window=window, dropout_p=p)
            out += [o2, lse2, dq2, dk2, dv2, delta2]
        return out

    _same(f"T={T} D={D} window={window} p={p}", _both(libs, run))


@pytest.mark.parametrize("T,D", [(333, 64), (200, 128)])
def test_fused_prologue(libs, T, D):
    import causal_head_self_amd as cat
    B, H = 1, 2
    _note(f"[lds poison] fused prologue T={T} D={D}")
    q, k, v, dO = _inputs(B, H, T, D, "bf16", 13)
    pro = cat.Prologue()

    def run():
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        q_rot, k_rot = torch.empty_like(q), torch.empty_like(q)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta = torch.empty_like(lse)
        cat.attn_fwd_strided_rope(q, k, v, o, lse, q_rot, k_rot, pro)
        cat.attn_bwd_strided_rope(q, k, q_rot, k_rot, v, o, lse, dO, dq, dk, dv, delta, pro)
        return [o, lse, q_rot, k_rot, dq, dk, dv, delta]

    _same(f"prologue T={T} D={D}", _both(libs, run))


@pytest.mark.parametrize("B,H,T_max,D", [(2, 3, 700, 64), (1, 2, 3000, 64), (2, 2, 300, 128),
                                         (1, 2, 1500, 128)])
def test_decode_both_paths(libs, B, H, T_max, D):
    import causal_head_self_amd as cat
    _note(f"[lds poison] decode B={B} H={H} T_max={T_max} D={D}")
    dev = torch.device("cuda")
    q, kc, vc = (t.to(dev) for t in workloads.decode_inputs(B, H, T_max, D, seed=14))
    lens = torch.tensor([T_max - 37 * b for b in range(B)], dtype=torch.int32, device=dev)

    def run():
        o, lse = cat.decode_attention(q, kc, vc, lens)
        o2 = torch.empty_like(o)
        lse2 = torch.empty_like(lse)
        cat.attn_decode_noalloc(q, kc, vc, lens, o2, lse2, window=200)
        return [o, lse, o2, lse2]

    _same(f"decode B={B} H={H} T_max={T_max} D={D}", _both(libs, run))


@pytest.mark.parametrize("N,C", [(333, 768), (70, 1000), (9, 4096)])
def test_layernorm_gradient(libs, N, C):
    import causal_head_self_amd as cat
    _note(f"[lds poison] layernorm bwd N={N} C={C}")
    dev = torch.device("cuda")
    g0 = torch.Generator().manual_seed(15)
    x, dy, dres = (torch.randn((N, C), generator=g0).to(torch.bfloat16).to(dev) for _ in range(3))
    gain = torch.randn(C, generator=g0).to(torch.bfloat16).to(dev)

    def run():
        dx = torch.empty_like(x)
        dg = torch.empty(C, dtype=torch.bfloat16, device=dev)
        db = torch.empty_like(dg)
        ws = torch.empty(cat.layernorm_workspace_bytes(N, C), dtype=torch.uint8, device=dev)
        cat.layernorm_bwd(x, gain, dy, dx, dg, db, ws, dres=dres)
        return [dx, dg, db]

    _same(f"layernorm bwd N={N} C={C}", _both(libs, run))
