"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with a retyped copy of itself.  They check
hand-derived worked examples (tests/golden), closed forms, invariants the pages
state (causal mask: a row cannot see later keys; softmax weights sum to 1), an
independent library routine (PyTorch's fp64 CPU scaled_dot_product_attention
with is_causal=True, the SDPA fallback the nanochat page names), and central
finite differences for the backward pass.  The planted-mistake test in
test_oracle_mutants.py shows that each plausible slip fails at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY_SHAPES = [(1, 1, 1, 1), (1, 1, 3, 2), (2, 2, 5, 3), (1, 2, 8, 4)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(shape, seed=0):
    return _rand(shape, seed), _rand(shape, seed + 1), _rand(shape, seed + 2)


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    shp = (g["B"], g["H"], g["T"], g["D"])
    return g, shp


# --------------------------------------------------------------------------
# worked examples (hand-derived, exact)
# --------------------------------------------------------------------------

def test_golden_forward_worked_example():
    g, shp = _load_golden("causal_fwd_T3_D1.json")
    arr = lambda key: np.array(g[key], dtype=np.float64).reshape(shp)
    o, lse = oracle.attn_fwd(arr("q"), arr("k"), arr("v"), g["scale"])
    np.testing.assert_allclose(o.ravel(), g["o"], rtol=0, atol=g["tol"] * 20)
    np.testing.assert_allclose(lse.ravel(), g["lse"], rtol=0, atol=g["tol"] * 20)


def test_golden_backward_worked_example():
    g, shp = _load_golden("causal_bwd_T2_D1.json")
    arr = lambda key: np.array(g[key], dtype=np.float64).reshape(shp)
    o, lse = oracle.attn_fwd(arr("q"), arr("k"), arr("v"), g["scale"])
    np.testing.assert_allclose(o.ravel(), g["o"], atol=g["tol"] * 20, rtol=0)
    np.testing.assert_allclose(lse.ravel(), g["lse"], atol=g["tol"] * 20, rtol=0)
    dq, dk, dv, delta = oracle.attn_bwd(arr("q"), arr("k"), arr("v"), arr("dO"), g["scale"])
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("delta", delta)):
        np.testing.assert_allclose(got.ravel(), g[name], atol=g["tol"] * 20, rtol=0, err_msg=name)


# --------------------------------------------------------------------------
# closed forms and special cases
# --------------------------------------------------------------------------

def test_single_token_is_identity():
    """T = 1: the only visible key is the query's own, weight 1: o = v and
    lse = scale * q.k."""
    q, k, v = _qkv((3, 2, 1, 5), seed=3)
    s = 0.37
    o, lse = oracle.attn_fwd(q, k, v, s)
    assert np.array_equal(o, v)
    np.testing.assert_allclose(lse, s * np.sum(q * k, axis=-1), rtol=1e-15, atol=1e-15)


def test_row0_equals_v_row0_exactly():
    """Row 0 sees only key 0 (diagonal kept), so its weight is exactly 1."""
    q, k, v = _qkv((2, 3, 17, 8), seed=5)
    o, _ = oracle.attn_fwd(q, k, v, 1 / math.sqrt(8))
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])


def test_zero_queries_give_running_prefix_mean():
    """q = 0: all visible scores are equal, the weights are uniform over
    j <= i, so o_i is the mean of v_0..v_i and lse_i = ln(i + 1)."""
    B, H, T, D = 2, 2, 33, 4
    _, k, v = _qkv((B, H, T, D), seed=7)
    q = np.zeros((B, H, T, D))
    o, lse = oracle.attn_fwd(q, k, v, 0.125)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(o, prefix_mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, T + 1)), (B, H, T)),
                               rtol=0, atol=1e-13)


def test_constant_values_pass_through():
    """Softmax weights of every row sum to 1, so v = c gives o = c."""
    q, k, _ = _qkv((2, 2, 19, 3), seed=11)
    v = np.full(q.shape, -2.75)
    o, _ = oracle.attn_fwd(q, k, v, 0.6)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


def test_identity_values_expose_the_weight_matrix():
    """With D = T and v_j = e_j, o_i is row i of the weight matrix: every row
    is non-negative, sums to 1, and is exactly 0 above the diagonal (the
    -inf upper triangle becomes weight 0)."""
    T = 12
    q, k, _ = _qkv((1, 1, T, T), seed=13)
    v = np.eye(T)[None, None]
    P, _ = oracle.attn_fwd(q, k, v, 0.3)
    P = P[0, 0]
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(axis=1), np.ones(T), rtol=0, atol=1e-15)
    assert np.all(P[np.triu_indices(T, k=1)] == 0.0)
    assert np.all(np.diag(P) > 0)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_causality_later_rows_do_not_leak():
    """Changing q, k, v in rows > i leaves output rows <= i bit-identical."""
    B, H, T, D = 2, 2, 24, 6
    q, k, v = _qkv((B, H, T, D), seed=17)
    o, lse = oracle.attn_fwd(q, k, v, 0.4)
    for cut in (0, 5, 23):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        r = _rand((B, H, T - cut - 1, D), 99 + cut)
        q2[:, :, cut + 1:] += r
        k2[:, :, cut + 1:] -= 2 * r
        v2[:, :, cut + 1:] += 3 * r
        o2, lse2 = oracle.attn_fwd(q2, k2, v2, 0.4)
        assert np.array_equal(o2[:, :, :cut + 1], o[:, :, :cut + 1])
        assert np.array_equal(lse2[:, :, :cut + 1], lse[:, :, :cut + 1])
        if cut + 1 < T:
            assert not np.array_equal(o2[:, :, cut + 1:], o[:, :, cut + 1:])


def test_key_shift_invariance():
    """k_j -> k_j + c for every j adds scale*q_i.c to every score of row i:
    o is unchanged and lse_i shifts by scale*q_i.c."""
    B, H, T, D = 1, 3, 20, 5
    q, k, v = _qkv((B, H, T, D), seed=19)
    c = _rand((D,), 23)
    s = 0.45
    o, lse = oracle.attn_fwd(q, k, v, s)
    o2, lse2 = oracle.attn_fwd(q, k + c, v, s)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + s * (q @ c), rtol=0, atol=1e-12)


def test_value_shift_adds_through():
    q, k, v = _qkv((2, 1, 15, 4), seed=29)
    c = _rand((4,), 31)
    o, _ = oracle.attn_fwd(q, k, v, 0.5)
    o2, _ = oracle.attn_fwd(q, k, v + c, 0.5)
    np.testing.assert_allclose(o2, o + c, rtol=0, atol=1e-13)


def test_batch_head_permutation_equivariance():
    B, H, T, D = 3, 4, 9, 3
    q, k, v = _qkv((B, H, T, D), seed=37)
    dO = _rand((B, H, T, D), 41)
    o, lse = oracle.attn_fwd(q, k, v, 0.5)
    dq, dk, dv, de = oracle.attn_bwd(q, k, v, dO, 0.5)
    perm = np.random.default_rng(43).permutation(B * H)
    P = lambda a: a.reshape(B * H, *a.shape[2:])[perm].reshape(a.shape)
    o2, lse2 = oracle.attn_fwd(P(q), P(k), P(v), 0.5)
    dq2, dk2, dv2, de2 = oracle.attn_bwd(P(q), P(k), P(v), P(dO), 0.5)
    for a, b in ((o2, o), (lse2, lse), (dq2, dq), (dk2, dk), (dv2, dv), (de2, de)):
        assert np.array_equal(a, P(b))


# --------------------------------------------------------------------------
# brute force and an independent library routine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", TINY_SHAPES + [(4, 4, 64, 32)])
def test_masked_matrix_brute_force(shape):
    """The explicit matrix form on tiny inputs: S = scale q k^T, -inf strictly
    above the diagonal, row softmax, O = P V."""
    q, k, v = _qkv(shape, seed=47)
    T, D = shape[2], shape[3]
    s = 1 / math.sqrt(D)
    S = s * np.einsum("bhid,bhjd->bhij", q, k)
    S[..., np.triu_indices(T, k=1)[0], np.triu_indices(T, k=1)[1]] = -np.inf
    P = np.exp(S - S.max(axis=-1, keepdims=True))
    P /= P.sum(axis=-1, keepdims=True)
    o, _ = oracle.attn_fwd(q, k, v, s)
    np.testing.assert_allclose(o, P @ v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", TINY_SHAPES + [(4, 4, 64, 32)])
def test_against_torch_sdpa_fp64(shape):
    """PyTorch's fp64 CPU scaled_dot_product_attention with is_causal=True
    (lower-triangular mask for equal query/key lengths), forward and
    autograd backward."""
    q, k, v = _qkv(shape, seed=53)
    dO = _rand(shape, 59)
    s = oracle.widen_scale(1 / math.sqrt(shape[3]))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=s)
    to.backward(torch.tensor(dO))
    o, _ = oracle.attn_fwd(q, k, v, s)
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dO, s)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


# --------------------------------------------------------------------------
# backward: finite differences and identities
# --------------------------------------------------------------------------

def _loss(q, k, v, dO, s, lib=None):
    o, _ = oracle.attn_fwd(q, k, v, s, lib=lib)
    return float(np.sum(o * dO))


def _fd_check(q, k, v, dO, s, idx_per_tensor, h=1e-5, tol=2e-7, lib=None):
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dO, s, lib=lib)
    tensors = {"q": (q, dq), "k": (k, dk), "v": (v, dv)}
    worst = 0.0
    for name, (x, g) in tensors.items():
        for flat in idx_per_tensor(x):
            i = np.unravel_index(flat, x.shape)
            x0 = x[i]
            x[i] = x0 + h
            lp = _loss(q, k, v, dO, s, lib)
            x[i] = x0 - h
            lm = _loss(q, k, v, dO, s, lib)
            x[i] = x0
            fd = (lp - lm) / (2 * h)
            err = abs(fd - g[i]) / max(1.0, abs(g[i]))
            worst = max(worst, err)
            assert err <= tol, f"d{name}{i}: analytic {g[i]!r} vs finite difference {fd!r}"
    return worst


@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_backward_finite_differences_every_element(shape):
    q, k, v = _qkv(shape, seed=61)
    dO = _rand(shape, 67)
    _fd_check(q, k, v, dO, 1 / math.sqrt(shape[3]), lambda x: range(x.size))


def test_backward_finite_differences_tiny_config_sampled():
    """200 random elements per tensor at the tiny config's shape."""
    shape = (4, 4, 64, 32)
    q, k, v = _qkv(shape, seed=71)
    dO = _rand(shape, 73)
    rng = np.random.default_rng(79)
    _fd_check(q, k, v, dO, oracle.widen_scale(1 / math.sqrt(32)),
              lambda x: rng.choice(x.size, 200, replace=False))


def test_backward_identities():
    """Derived closed forms: dq row 0 = 0 (a one-key softmax has no
    gradient); rows of dS sum to 0, so sum_j dk_j = 0; sum_j dv_j = sum_i dO_i;
    Delta_i = dO_i . o_i."""
    B, H, T, D = 2, 3, 40, 8
    q, k, v = _qkv((B, H, T, D), seed=83)
    dO = _rand((B, H, T, D), 89)
    o, _ = oracle.attn_fwd(q, k, v, 0.35)
    dq, dk, dv, delta = oracle.attn_bwd(q, k, v, dO, 0.35)
    assert np.all(dq[:, :, 0, :] == 0.0)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), dO.sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(delta, np.sum(dO * o, axis=-1), atol=1e-12)


def test_backward_causality():
    """dq_i depends only on keys j <= i: perturbing k, v rows > i leaves dq
    rows <= i bit-identical."""
    B, H, T, D = 1, 2, 16, 4
    q, k, v = _qkv((B, H, T, D), seed=97)
    dO = _rand((B, H, T, D), 101)
    dq, _, _, _ = oracle.attn_bwd(q, k, v, dO, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 9:] += 1.0
    v2[:, :, 9:] -= 1.0
    dq2, _, _, _ = oracle.attn_bwd(q, k2, v2, dO, 0.5)
    assert np.array_equal(dq2[:, :, :9], dq[:, :, :9])


# --------------------------------------------------------------------------
# pre-norm attention sublayer
# --------------------------------------------------------------------------

def _sublayer_params(B, T, C, seed=0):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((B, T, C)),
        g=1.0 + 0.1 * r.standard_normal(C),
        bl=0.1 * r.standard_normal(C),
        Wa=0.3 * r.standard_normal((C, 3 * C)),
        ba=0.1 * r.standard_normal(3 * C),
        Wp=0.3 * r.standard_normal((C, C)),
        bp=0.1 * r.standard_normal(C),
    )


def _torch_sublayer(p, H, eps=1e-5):
    """Independent composition from PyTorch fp64 CPU library ops:
    F.layer_norm, F.linear, scaled_dot_product_attention(is_causal=True)."""
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    x = t["x"]
    B, T, C = x.shape
    D = C // H
    u = torch.nn.functional.layer_norm(x, (C,), t["g"], t["bl"], eps)
    qkv = torch.nn.functional.linear(u, t["Wa"].t(), t["ba"])
    q, k, v = qkv.chunk(3, dim=-1)
    heads = lambda z: z.view(B, T, H, D).transpose(1, 2)
    a = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v),
                                                         is_causal=True)
    a = a.transpose(1, 2).reshape(B, T, C)
    y = x + torch.nn.functional.linear(a, t["Wp"].t(), t["bp"])
    return t, y


def test_sublayer_against_torch_library_ops():
    B, T, C, H = 2, 7, 12, 3
    p = _sublayer_params(B, T, C, seed=103)
    dy = np.random.default_rng(107).standard_normal((B, T, C))
    t, y_ref = _torch_sublayer(p, H)
    y_ref.backward(torch.tensor(dy))
    y = oracle.sublayer_fwd(**p, n_head=H)
    grads = oracle.sublayer_bwd(**p, dy=dy, n_head=H)
    np.testing.assert_allclose(y, y_ref.detach().numpy(), rtol=0, atol=1e-12)
    for ours, theirs in (("dx", "x"), ("dg", "g"), ("dbl", "bl"), ("dWa", "Wa"),
                         ("dba", "ba"), ("dWp", "Wp"), ("dbp", "bp")):
        np.testing.assert_allclose(grads[ours], t[theirs].grad.numpy(), rtol=0, atol=1e-11,
                                   err_msg=ours)


def test_sublayer_residual_path():
    """Wp = 0 and bp = 0 switch the attention branch off: y = x exactly (the
    residual path of the pre-norm block)."""
    B, T, C, H = 1, 5, 8, 2
    p = _sublayer_params(B, T, C, seed=109)
    p["Wp"][:] = 0.0
    p["bp"][:] = 0.0
    y = oracle.sublayer_fwd(**p, n_head=H)
    assert np.array_equal(y, p["x"])


def test_sublayer_finite_differences():
    B, T, C, H = 1, 5, 8, 2
    p = _sublayer_params(B, T, C, seed=113)
    dy = np.random.default_rng(127).standard_normal((B, T, C))
    grads = oracle.sublayer_bwd(**p, dy=dy, n_head=H)
    h = 1e-6
    rng = np.random.default_rng(131)
    for name, gname in (("x", "dx"), ("g", "dg"), ("bl", "dbl"), ("Wa", "dWa"),
                        ("ba", "dba"), ("Wp", "dWp"), ("bp", "dbp")):
        arr = p[name]
        for flat in rng.choice(arr.size, min(arr.size, 12), replace=False):
            i = np.unravel_index(flat, arr.shape)
            x0 = arr[i]
            arr[i] = x0 + h
            lp = float(np.sum(oracle.sublayer_fwd(**p, n_head=H) * dy))
            arr[i] = x0 - h
            lm = float(np.sum(oracle.sublayer_fwd(**p, n_head=H) * dy))
            arr[i] = x0
            fd = (lp - lm) / (2 * h)
            g = grads[gname][i]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(g)), f"{gname}{i}: {g} vs {fd}"


def test_layernorm_output_is_standardised():
    """LN with g = 1, b = 0: the q third of c_attn with Wa = [I | 0 | 0] and
    H = 1, q = LN(x); take v = LN(x) too and q = 0 so o_0 = v_0 = LN(x_0):
    mean 0, biased variance 1/(1 + eps/var)."""
    B, T, C = 1, 4, 16
    r = np.random.default_rng(137)
    x = 3.0 + 2.0 * r.standard_normal((B, T, C))
    Wa = np.zeros((C, 3 * C))
    Wa[:, 2 * C:] = np.eye(C)  # v = LN(x); q = k = 0
    Wp = np.eye(C)
    y = oracle.sublayer_fwd(x, np.ones(C), np.zeros(C), Wa, np.zeros(3 * C), Wp, np.zeros(C),
                            n_head=1)
    ln0 = (y - x)[0, 0]  # o_0 = v_0 = LN(x_0)
    var = np.var(x[0, 0])
    assert abs(ln0.mean()) < 1e-14
    np.testing.assert_allclose(np.mean(ln0 ** 2), var / (var + 1e-5), rtol=1e-13)


def test_layernorm_alone_is_standardised_affine_and_shift_invariant():
    """The standalone LayerNorm (class LayerNorm, CS336 section 3.4): with g = 1,
    b = 0 every row has mean 0 and mean square var/(var + eps); the gain and
    bias act elementwise afterwards; a constant added to a row changes
    nothing; scaling a row by s with eps scaled by s^2 changes nothing."""
    r = np.random.default_rng(401)
    N, C = 6, 24
    x = 3.0 + 2.0 * r.standard_normal((N, C))
    g, b = r.standard_normal(C), r.standard_normal(C)
    y0 = oracle.layernorm_fwd(x, np.ones(C), np.zeros(C))
    var = x.var(axis=1)
    assert np.all(np.abs(y0.mean(axis=1)) < 1e-14)
    np.testing.assert_allclose((y0 ** 2).mean(axis=1), var / (var + 1e-5), rtol=1e-13)
    np.testing.assert_allclose(oracle.layernorm_fwd(x, g, b), y0 * g + b, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.layernorm_fwd(x + r.standard_normal((N, 1)), g, b),
                               oracle.layernorm_fwd(x, g, b), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.layernorm_fwd(7.0 * x, g, b, eps=49e-5),
                               oracle.layernorm_fwd(x, g, b), rtol=0, atol=1e-12)


def test_layernorm_backward_finite_differences_and_residual():
    """dx, dg, dbl of sum(du * LN(x)) + sum(dres * x) by central differences;
    without du the gradient is dres itself; and each row's LN part of dx sums
    to zero (LN is invariant to adding a constant to a row)."""
    r = np.random.default_rng(409)
    N, C = 4, 10
    x = r.standard_normal((N, C)) * 1.5 + 0.5
    g, b = r.standard_normal(C), r.standard_normal(C)
    du, dres = r.standard_normal((N, C)), r.standard_normal((N, C))
    dx, dg, db = oracle.layernorm_bwd(x, g, b, du, dres)
    h = 1e-6

    def loss(x_, g_, b_):
        return float(np.sum(du * oracle.layernorm_fwd(x_, g_, b_)) + np.sum(dres * x_))

    for arr, grad in ((x, dx), (g, dg), (b, db)):
        for flat in range(arr.size):
            i = np.unravel_index(flat, arr.shape)
            x0 = arr[i]
            arr[i] = x0 + h
            lp = loss(x, g, b)
            arr[i] = x0 - h
            lm = loss(x, g, b)
            arr[i] = x0
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(grad[i])), (i, grad[i], fd)
    dx0, dg0, db0 = oracle.layernorm_bwd(x, g, b, np.zeros((N, C)), dres)
    assert np.array_equal(dx0, dres) and not dg0.any() and not db0.any()
    dxl, _, _ = oracle.layernorm_bwd(x, g, b, du)
    np.testing.assert_allclose(dxl, dx - dres, rtol=0, atol=1e-13)
    assert np.all(np.abs(dxl.sum(axis=1)) < 1e-12)


def test_colsum_of_a_matrix_with_known_column_sums():
    """Integer entries (exact in fp64): the column sums of the matrix whose row
    n, column j holds (n + 1) * (j - 2) are (j - 2) * N (N + 1) / 2."""
    N, M = 37, 9
    x = np.fromfunction(lambda n, j: (n + 1) * (j - 2), (N, M))
    assert np.array_equal(oracle.colsum(x), (np.arange(M) - 2) * N * (N + 1) / 2)
    assert np.array_equal(oracle.colsum(np.ones((1, 5))), np.ones(5))


# --------------------------------------------------------------------------
# sliding window (query i sees keys i-W < j <= i): nanochat section 9 lists
# sliding-window attention; the band is the causal mask with the W most
# recent keys kept
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 9, 50])
def test_window_at_least_T_is_the_causal_result(window):
    shape = (2, 2, 9, 4)
    q, k, v = _qkv(shape, seed=301)
    dO = _rand(shape, 303)
    o, lse = oracle.attn_fwd(q, k, v, 0.4)
    dq, dk, dv, delta = oracle.attn_bwd(q, k, v, dO, 0.4)
    ow, lsew = oracle.attn_fwd(q, k, v, 0.4, window=window)
    dqw, dkw, dvw, deltaw = oracle.attn_bwd(q, k, v, dO, 0.4, window=window)
    for a, b in ((o, ow), (lse, lsew), (dq, dqw), (dk, dkw), (dv, dvw), (delta, deltaw)):
        assert np.array_equal(a, b)


def test_window_one_is_the_identity():
    """W = 1: each query sees only itself, so o = v, lse = s q_i.k_i, P = 1
    and dS = 0 (dq = dk = 0), dv = dO."""
    shape = (2, 3, 7, 5)
    q, k, v = _qkv(shape, seed=307)
    dO = _rand(shape, 311)
    o, lse = oracle.attn_fwd(q, k, v, 0.3, window=1)
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dO, 0.3, window=1)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * np.sum(q * k, axis=-1), rtol=0, atol=1e-14)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(dv, dO, rtol=0, atol=1e-15)


@pytest.mark.parametrize("window", [2, 3, 5])
def test_window_against_torch_sdpa_band_mask(window):
    """PyTorch fp64 scaled_dot_product_attention with an explicit band mask
    (True where i-W < j <= i), forward and autograd backward."""
    shape = (2, 2, 9, 3)
    q, k, v = _qkv(shape, seed=313)
    dO = _rand(shape, 317)
    s = 0.45
    T = shape[2]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    band = torch.tensor((j <= i) & (j > i - window))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, scale=s)
    to.backward(torch.tensor(dO))
    o, _ = oracle.attn_fwd(q, k, v, s, window=window)
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dO, s, window=window)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def test_window_backward_finite_differences():
    shape = (1, 2, 8, 4)
    q, k, v = _qkv(shape, seed=331)
    dO = _rand(shape, 337)
    W = 3
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dO, 0.5, window=W)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for flat in range(x.size):
            idx = np.unravel_index(flat, x.shape)
            x0 = x[idx]
            x[idx] = x0 + h
            lp = float(np.sum(oracle.attn_fwd(q, k, v, 0.5, window=W)[0] * dO))
            x[idx] = x0 - h
            lm = float(np.sum(oracle.attn_fwd(q, k, v, 0.5, window=W)[0] * dO))
            x[idx] = x0
            assert abs((lp - lm) / (2 * h) - g[idx]) < 2e-7, (name, idx)


# --------------------------------------------------------------------------
# decode against a KV cache (nanochat, section 8: FA3 (B, T, H, D) cache,
# prefill then one token at a time)
# --------------------------------------------------------------------------

def _cache(B, Tmax, H, D, seed):
    return _rand((B, H, D), seed), _rand((B, Tmax, H, D), seed + 1), _rand((B, Tmax, H, D), seed + 2)


@pytest.mark.parametrize("window", [0, 1, 3, 50])
def test_decode_against_torch_sdpa_single_query(window):
    """Each (b, h): PyTorch fp64 SDPA of the one query over the visible cache
    rows, and torch.logsumexp of the scaled scores for lse."""
    B, Tmax, H, D = 4, 12, 3, 5
    q, kc, vc = _cache(B, Tmax, H, D, 401)
    lens = [7, 1, 12, 9]
    s = 0.37
    o, lse = oracle.attn_decode(q, kc, vc, lens, s, window=window)
    for b in range(B):
        n = lens[b]
        j0 = max(0, n - window) if window else 0
        for h in range(H):
            tq = torch.tensor(q[b, h][None, None, None, :])           # [1, 1, 1, D]
            tk = torch.tensor(kc[b, j0:n, h][None, None])             # [1, 1, n-j0, D]
            tv = torch.tensor(vc[b, j0:n, h][None, None])
            to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s)
            np.testing.assert_allclose(o[b, h], to[0, 0, 0].numpy(), rtol=0, atol=1e-13)
            tl = torch.logsumexp(s * (tk[0, 0] @ tq[0, 0, 0]), dim=0)
            assert abs(lse[b, h] - float(tl)) < 1e-13


@pytest.mark.parametrize("window", [0, 4])
def test_decode_is_the_last_row_of_the_causal_forward(window):
    """Prefill and decode agree: the token at position len-1 decoded against
    the cache gets row len-1 of the causal forward over the same sequence."""
    B, H, T, D = 2, 3, 10, 4
    q, k, v = _qkv((B, H, T, D), seed=411)
    o_full, lse_full = oracle.attn_fwd(q, k, v, 0.5, window=window)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))  # [B, T, H, D]
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    for n in (1, 2, 5, T):
        o, lse = oracle.attn_decode(q[:, :, n - 1], kc, vc, [n] * B, 0.5, window=window)
        np.testing.assert_allclose(o, o_full[:, :, n - 1], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, lse_full[:, :, n - 1], rtol=0, atol=1e-14)


def test_decode_closed_forms():
    B, Tmax, H, D = 2, 6, 2, 3
    q, kc, vc = _cache(B, Tmax, H, D, 421)
    # one cached position: the output is that value row, lse its scaled score
    o, lse = oracle.attn_decode(q, kc, vc, [1, 1], 0.7)
    assert np.array_equal(o, vc[:, 0])
    np.testing.assert_allclose(lse, 0.7 * np.einsum("bhd,bhd->bh", q, kc[:, 0]), atol=1e-15)
    # a zero query weighs the visible rows equally
    o, lse = oracle.attn_decode(np.zeros_like(q), kc, vc, [6, 4], 0.7, window=3)
    np.testing.assert_allclose(o[0], vc[0, 3:6].mean(axis=0), atol=1e-15)
    np.testing.assert_allclose(o[1], vc[1, 1:4].mean(axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, math.log(3.0), atol=1e-15)
    # nothing cached
    o, lse = oracle.attn_decode(q, kc, vc, [0, 3], 0.7)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))


def test_decode_reads_only_the_visible_cache_rows():
    """Rows at or past len, and before the window, do not matter; the visible
    rows enter as a set (any order of the positions gives the same result)."""
    B, Tmax, H, D = 2, 9, 2, 4
    q, kc, vc = _cache(B, Tmax, H, D, 431)
    lens, W = [7, 5], 4
    o, lse = oracle.attn_decode(q, kc, vc, lens, 0.5, window=W)
    kc2, vc2 = kc.copy(), vc.copy()
    for b, n in enumerate(lens):
        kc2[b, n:] = 1e3
        vc2[b, n:] = -1e3
        kc2[b, :n - W] = 5e2
        vc2[b, :n - W] = 7e2
    o2, lse2 = oracle.attn_decode(q, kc2, vc2, lens, 0.5, window=W)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    perm = np.array([0, 1, 2, 6, 4, 3, 5, 7, 8])  # positions 3..6 reordered (b = 0)
    o3, lse3 = oracle.attn_decode(q, kc[:, perm], vc[:, perm], lens, 0.5, window=W)
    np.testing.assert_allclose(o3[0], o[0], atol=1e-14)
    np.testing.assert_allclose(lse3[0], lse[0], atol=1e-14)


# --------------------------------------------------------------------------
# RoPE and QK norm (nanochat, section 9); standard forms as the reading
# --------------------------------------------------------------------------

def test_rope_two_columns_is_a_plane_rotation_by_the_position():
    """D = 2: one pair, frequency base^0 = 1, so the row at position p is turned
    by p radians counter-clockwise: (x0, x1) -> (x0 cos p - x1 sin p,
    x0 sin p + x1 cos p)."""
    x = _rand((1, 1, 5, 2), 501)
    y = oracle.rope_qknorm_fwd(x, pos0=3, norm=False)
    for t in range(5):
        p = 3 + t
        c, s = math.cos(p), math.sin(p)
        x0, x1 = x[0, 0, t]
        assert abs(y[0, 0, t, 0] - (x0 * c - x1 * s)) < 1e-15
        assert abs(y[0, 0, t, 1] - (x0 * s + x1 * c)) < 1e-15


def test_rope_four_columns_pairs_and_frequencies():
    """D = 4, base 100: columns (0, 2) turn by p, columns (1, 3) by p / 10
    (100^(-2/4) = 0.1)."""
    x = _rand((1, 1, 4, 4), 503)
    y = oracle.rope_qknorm_fwd(x, base=100.0, norm=False)
    for t in range(4):
        for (a, b), w in (((0, 2), 1.0), ((1, 3), 0.1)):
            c, s = math.cos(w * t), math.sin(w * t)
            assert abs(y[0, 0, t, a] - (x[0, 0, t, a] * c - x[0, 0, t, b] * s)) < 1e-14
            assert abs(y[0, 0, t, b] - (x[0, 0, t, a] * s + x[0, 0, t, b] * c)) < 1e-14


def test_rope_scores_depend_only_on_the_relative_position():
    """q_p . k_s after RoPE is unchanged when both positions move by the same
    amount (pos0), and position 0 is the identity."""
    B, H, T, D = 1, 2, 7, 8
    q, k = _rand((B, H, T, D), 511), _rand((B, H, T, D), 512)
    s0 = np.einsum("bhid,bhjd->bhij", oracle.rope_qknorm_fwd(q, norm=False),
                   oracle.rope_qknorm_fwd(k, norm=False))
    s9 = np.einsum("bhid,bhjd->bhij", oracle.rope_qknorm_fwd(q, pos0=9, norm=False),
                   oracle.rope_qknorm_fwd(k, pos0=9, norm=False))
    np.testing.assert_allclose(s9, s0, atol=1e-12)
    y = oracle.rope_qknorm_fwd(q, norm=False)
    assert np.array_equal(y[:, :, 0], q[:, :, 0])
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(q, axis=-1), atol=1e-13)


@pytest.mark.parametrize("gain,eps", [(1.0, 1e-6), (1.2, 1e-6), (1.2, 0.0), (0.7, 0.5)])
def test_qk_norm_against_torch_rms_norm(gain, eps):
    """Norm only: PyTorch's fp64 rms_norm (no weight) times the gain."""
    x = _rand((2, 3, 5, 16), 521)
    y = oracle.rope_qknorm_fwd(x, rope=False, gain=gain, eps=eps)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (16,), eps=eps).numpy() * gain
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-14)
    if eps == 0.0:
        np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), gain, atol=1e-14)


def test_rope_and_norm_commute():
    x = _rand((1, 2, 6, 8), 531)
    both = oracle.rope_qknorm_fwd(x, pos0=2, gain=1.2)
    rope_then_norm = oracle.rope_qknorm_fwd(oracle.rope_qknorm_fwd(x, pos0=2, norm=False),
                                            rope=False, gain=1.2)
    norm_then_rope = oracle.rope_qknorm_fwd(oracle.rope_qknorm_fwd(x, rope=False, gain=1.2),
                                            pos0=2, norm=False)
    np.testing.assert_allclose(both, rope_then_norm, atol=1e-14)
    np.testing.assert_allclose(both, norm_then_rope, atol=1e-14)


@pytest.mark.parametrize("rope,norm", [(True, False), (False, True), (True, True)])
def test_rope_qknorm_backward_finite_differences(rope, norm):
    B, H, T, D = 1, 2, 4, 6
    x = _rand((B, H, T, D), 541)
    dy = _rand((B, H, T, D), 542)
    kw = dict(pos0=5, base=50.0, rope=rope, norm=norm, gain=1.2, eps=1e-3)
    dx = oracle.rope_qknorm_bwd(x, dy, **kw)
    h = 1e-6
    for flat in range(x.size):
        xp, xm = x.copy(), x.copy()
        xp.flat[flat] += h
        xm.flat[flat] -= h
        fd = (np.sum(dy * oracle.rope_qknorm_fwd(xp, **kw)) -
              np.sum(dy * oracle.rope_qknorm_fwd(xm, **kw))) / (2 * h)
        assert abs(fd - dx.flat[flat]) < 1e-7 * max(1.0, abs(fd)), (flat, fd, dx.flat[flat])


# --------------------------------------------------------------------------
# attention dropout (CS336 section 5.1: att = dropout(att) before att @ v)
# with keep decisions from Philox4x32-10
# --------------------------------------------------------------------------

# Published known-answer vectors of Philox4x32-10 (Random123's kat_vectors,
# the reference implementation of Salmon et al., SC 2011):
# (counter, key) -> output
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def test_philox_known_answer_vectors():
    for ctr, key, out in PHILOX_KAT:
        assert tuple(oracle.philox4x32_10(ctr, key)) == out


def test_dropout_keep_follows_the_stated_draw_and_rate():
    """Element (bh, i, j) reads 16-bit half j % 2 of word (j % 8) / 2 of
    Philox(counter (j/8, i, bh, 0), key = the seed's two halves); over many
    elements the kept fraction is 1 - p16 / 65536 within 5 sigma."""
    seed = 0x0123456789ABCDEF
    p16 = oracle.dropout_threshold(0.3)
    assert p16 == 19661
    kept = n = 0
    for bh in range(3):
        for i in range(0, 40, 7):
            for j in range(0, 64):
                r = oracle.philox4x32_10((j // 8, i, bh, 0), (seed & 0xFFFFFFFF, seed >> 32))
                u = (r[(j % 8) // 2] >> (16 * (j % 2))) & 0xFFFF
                k = oracle.dropout_keep(seed, p16, bh, i, j)
                assert k == (u >= p16)
                kept += k
                n += 1
    rate = 1 - p16 / 65536
    assert abs(kept - n * rate) < 5 * math.sqrt(n * rate * (1 - rate))


def test_dropout_zero_is_the_plain_attention():
    shape = (2, 2, 9, 4)
    q, k, v = _qkv(shape, seed=601)
    dO = _rand(shape, 602)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, window=4)
    od, lsed = oracle.attn_fwd_dropout(q, k, v, 0.5, 0.0, seed=7, window=4)
    assert np.array_equal(o, od) and np.array_equal(lse, lsed)
    g = oracle.attn_bwd(q, k, v, dO, 0.5, window=4)
    gd = oracle.attn_bwd_dropout(q, k, v, dO, 0.5, 0.0, seed=7, window=4)
    for a, b in zip(g, gd):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("p,window", [(0.1, 0), (0.5, 0), (0.3, 3)])
def test_dropout_against_torch_ops_with_the_same_mask(p, window):
    """PyTorch fp64 ops with autograd: masked softmax, times keep / (1 - p16 /
    65536), times v.  lse is that of the undropped weights; Delta equals
    dO . o of the dropped output."""
    B, H, T, D = 2, 2, 10, 3
    q, k, v = _qkv((B, H, T, D), seed=611)
    dO = _rand((B, H, T, D), 612)
    s, seed = 0.6, 0xDEADBEEF12345
    p16 = oracle.dropout_threshold(p)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    vis = (j <= i) & ((j > i - window) if window else True)
    keep = np.array([[[[oracle.dropout_keep(seed, p16, b * H + h, a, c) for c in range(T)]
                       for a in range(T)] for h in range(H)] for b in range(B)], dtype=np.float64)
    mult = torch.tensor(keep * (65536.0 / (65536 - p16)))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    sc = s * tq @ tk.transpose(-1, -2)
    sc = sc.masked_fill(~torch.tensor(vis), float("-inf"))
    to = (torch.softmax(sc, dim=-1) * mult) @ tv
    to.backward(torch.tensor(dO))
    o, lse = oracle.attn_fwd_dropout(q, k, v, s, p, seed, window=window)
    dq, dk, dv, delta = oracle.attn_bwd_dropout(q, k, v, dO, s, p, seed, window=window)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(sc, dim=-1).detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(delta, np.sum(dO * o, axis=-1), atol=1e-12)
    assert 0 < keep[vis[None, None].repeat(B, 0).repeat(H, 1)].mean() < 1


def test_dropout_backward_finite_differences():
    shape = (1, 2, 7, 3)
    q, k, v = _qkv(shape, seed=621)
    dO = _rand(shape, 622)
    kw = dict(p=0.4, seed=99, window=0)
    dq, dk, dv, _ = oracle.attn_bwd_dropout(q, k, v, dO, 0.5, **kw)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for flat in range(x.size):
            xp, xm = x.copy(), x.copy()
            xp.flat[flat] += h
            xm.flat[flat] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fp = np.sum(dO * oracle.attn_fwd_dropout(args_p["q"], args_p["k"], args_p["v"], 0.5,
                                                     **kw)[0])
            fm = np.sum(dO * oracle.attn_fwd_dropout(args_m["q"], args_m["k"], args_m["v"], 0.5,
                                                     **kw)[0])
            fd = (fp - fm) / (2 * h)
            assert abs(fd - g.flat[flat]) < 1e-7 * max(1.0, abs(fd)), (name, flat)


def test_dropout_head_offset_matches_the_full_batch():
    """A (b, h) slice checked alone with bh0 = its global index gets the same
    result as inside the full batch."""
    B, H, T, D = 2, 3, 12, 4
    q, k, v = _qkv((B, H, T, D), seed=631)
    dO = _rand((B, H, T, D), 632)
    o, lse = oracle.attn_fwd_dropout(q, k, v, 0.5, 0.3, 11)
    g = oracle.attn_bwd_dropout(q, k, v, dO, 0.5, 0.3, 11)
    b, h = 1, 2
    sl = (slice(b, b + 1), slice(h, h + 1))
    os_, ls_ = oracle.attn_fwd_dropout(q[sl], k[sl], v[sl], 0.5, 0.3, 11, bh0=b * H + h)
    gs = oracle.attn_bwd_dropout(q[sl], k[sl], v[sl], dO[sl], 0.5, 0.3, 11, bh0=b * H + h)
    assert np.array_equal(os_, o[sl]) and np.array_equal(ls_, lse[sl])
    for a, r in zip(gs, g):
        assert np.array_equal(a, r[sl])
