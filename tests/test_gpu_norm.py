"""GPU parity of the sublayer's row passes (attn_layernorm_fwd,
attn_layernorm_bwd, attn_colsum) against the fp64 oracle, element by element.

The inputs use random gains and biases, so no output here is unit variance
(in the sublayer, with gain 1 and bias 0, y and dx are, and keep the plain bf16
bar 2e-2 there).  Every tensor is held, as the sublayer test holds its
non-unit-variance ones, to 2e-2 * max(1, rms(ref)) + 2^-8 * |ref|: the stated
bar after normalising the tensor to unit rms, plus the rounding of the bf16
result itself (a |y| near 10 has a bf16 spacing of 1/16).
Shapes span one chunk per lane and several (C up to 4096), a partial last
chunk round (C = 1000), a row stride beyond C, single rows, and the full
sublayer size (N = 8192, C = 768); the gradient runs with and without the
residual term.
"""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _note(msg):
    print(msg)
    sys.stdout.flush()


def _bf16(shape, seed, scale=1.0, shift=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale + shift).to(torch.bfloat16)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(name, got, ref):
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    tol = TOL * max(1.0, rms) + 2.0 ** -8 * np.abs(ref)
    worst = int(np.argmax(err - tol))
    _note(f"  {name}: max abs err {float(err.max()):.3e} (at the worst margin err "
          f"{float(err.flat[worst]):.3e}, tol {float(tol.flat[worst]):.3e})")
    assert np.all(err <= tol), f"{name}: error beyond its bound at flat index {worst}"


def _rows(N, C, stride, seed, scale=1.0, shift=0.0):
    """[N, C] bf16 on the GPU with row stride `stride` (a view of a wider buffer)."""
    full = _bf16((N, stride), seed, scale, shift).cuda()
    return full[:, :C]


CASES = [  # N, C, row stride
    (1, 8, 8),
    (7, 64, 64),
    (333, 768, 768),
    (130, 1000, 1008),
    (65, 1536, 1536),
    (9, 4096, 4104),
    (8192, 768, 768),
]


@pytest.mark.parametrize("N,C,stride", CASES)
def test_layernorm_forward_matches_oracle(N, C, stride):
    import causal_head_self_amd as cat
    _note(f"[layernorm fwd] N={N} C={C} stride={stride}")
    x = _rows(N, C, stride, 11, scale=2.0, shift=0.7)
    g, b = _bf16(C, 12).cuda(), _bf16(C, 13).cuda()
    y = torch.full((N, stride), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :C]
    cat.layernorm_fwd(x, g, b, y, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.layernorm_fwd(_np(x), _np(g), _np(b), eps=1e-5)
    _check("y", _np(y), ref)
    if stride > C:  # the gap between rows is not written
        assert torch.isnan(torch.as_strided(y, (N, stride - C), (stride, 1), C).float()).all()


@pytest.mark.parametrize("N,C,stride", CASES)
@pytest.mark.parametrize("residual", [True, False])
def test_layernorm_backward_matches_oracle(N, C, stride, residual):
    import causal_head_self_amd as cat
    _note(f"[layernorm bwd] N={N} C={C} stride={stride} residual={residual}")
    x = _rows(N, C, stride, 21, scale=1.5, shift=-0.3)
    g, b = _bf16(C, 22).cuda(), _bf16(C, 23).cuda()
    dy = _rows(N, C, stride, 24)
    dres = _rows(N, C, stride, 25) if residual else None
    dx = torch.empty((N, stride), dtype=torch.bfloat16, device="cuda")[:, :C]
    dg, db = torch.empty(C, dtype=torch.bfloat16, device="cuda"), torch.empty(
        C, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(cat.layernorm_workspace_bytes(N, C), dtype=torch.uint8, device="cuda")
    cat.layernorm_bwd(x, g, dy, dx, dg, db, ws, dres=dres, eps=1e-5)
    torch.cuda.synchronize()
    rdx, rdg, rdb = oracle.layernorm_bwd(_np(x), _np(g), _np(b), _np(dy),
                                         None if dres is None else _np(dres), eps=1e-5)
    _check("dx", _np(dx), rdx)
    _check("dg", _np(dg), rdg)
    _check("db", _np(db), rdb)


@pytest.mark.parametrize("N,M,stride", [(1, 8, 8), (31, 72, 80), (33, 2304, 2304),
                                        (8192, 2304, 2304), (8192, 768, 768), (100, 4104, 4104)])
def test_colsum_matches_oracle(N, M, stride):
    import causal_head_self_amd as cat
    _note(f"[colsum] N={N} M={M} stride={stride}")
    x = _rows(N, M, stride, 31)
    out = torch.empty(M, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(cat.colsum_workspace_bytes(N, M), dtype=torch.uint8, device="cuda")
    cat.colsum(x, out, ws)
    torch.cuda.synchronize()
    _check("colsum", _np(out), oracle.colsum(_np(x)))


@pytest.mark.parametrize("P,M", [(1, 8), (2, 768 * 2304), (16, 768 * 768), (5, 1032)])
def test_colsum_of_fp32_rows_matches_oracle(P, M):
    """The split-K epilogue of the weight gradients: a few fp32 rows added in
    order and rounded once to bf16."""
    import causal_head_self_amd as cat
    _note(f"[colsum fp32] P={P} M={M}")
    g = torch.Generator().manual_seed(51)
    x = (torch.randn((P, M), generator=g) * 30.0).cuda()
    out = torch.empty(M, dtype=torch.bfloat16, device="cuda")
    cat.colsum(x, out)
    torch.cuda.synchronize()
    _check("colsum fp32", _np(out), oracle.colsum(x.double().cpu().numpy()))


def test_row_passes_are_deterministic():
    import causal_head_self_amd as cat
    N, C = 1000, 768
    x, dy = _rows(N, C, C, 41), _rows(N, C, C, 42)
    g, b = _bf16(C, 43).cuda(), _bf16(C, 44).cuda()
    ws = torch.empty(cat.layernorm_workspace_bytes(N, C), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        y, dx = torch.empty_like(x), torch.empty_like(x)
        dg, db, cs = (torch.empty(C, dtype=torch.bfloat16, device="cuda") for _ in range(3))
        cat.layernorm_fwd(x, g, b, y)
        cat.layernorm_bwd(x, g, dy, dx, dg, db, ws, dres=dy)
        cat.colsum(dy, cs, torch.empty(cat.colsum_workspace_bytes(N, C), dtype=torch.uint8,
                                       device="cuda"))
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (y, dx, dg, db, cs)])
    for a, c in zip(*outs):
        assert torch.equal(a, c)
