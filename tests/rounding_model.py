"""A CPU model of the roundings of the bf16 attention pipeline (test
infrastructure; numpy only, shares nothing with the HIP sources).

It computes causal attention and its gradient the way the stated reading of
"bf16 storage / fp32 accumulate" does: every product accumulated in fp32, the
softmax weights P rounded to bf16 before the P V and P^T dO products, dS
rounded to bf16 before the dS K and dS^T Q products, every output stored in
bf16, and Delta formed from the stored bf16 output (CS336 tutorial, section
5.1 for the forward; the backward is the exact gradient the training loop of
its section 5.2 takes).  The forward keeps a running row maximum over 64-key
tiles that is raised only when it grows by more than 2^8 in base-2 exponent,
so the rounded weights are those of an online softmax, not of a two-pass one.

Its purpose is to bound what the rounding model alone costs against the exact
fp64 result, independently of any GPU: a tolerance that an implementation of
these roundings cannot meet is the model's, not the kernel's.  It does not
reproduce the GPU's bits (the summation order inside a matrix product is not
specified), only the size of the errors these roundings produce.
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
TILE = 64
LAZY = 8.0  # base-2 growth of the running max that forces a rescale


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16(x):
    """fp32 -> bf16, round to nearest even, returned as fp64 (exact)."""
    u = f32(x).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _visible(T: int, window: int):
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    vis = j <= i
    if 0 < window < T:
        vis &= j > i - window
    return vis


def head_forward(q, k, v, scale: float, window: int = 0, keep=None, keep_scale: float = 1.0):
    """One head: q, k, v [T, D] (exact bf16 values in fp64).  Returns o (bf16
    values), lse (fp32 values), and the fp32 l and m.  keep: optional [T, T]
    boolean dropout mask (kept weights scaled by keep_scale at the end)."""
    T, _ = q.shape
    c = float(np.float32(scale * LOG2E))  # scale * log2(e) as the fp32 constant
    S = f32(q @ k.T).astype(np.float64)   # fp32 dot products
    vis = _visible(T, window)
    S = np.where(vis, S, -np.inf)
    m = np.full(T, -1e30)
    l = np.zeros(T, dtype=np.float32)
    acc = np.zeros((T, v.shape[1]), dtype=np.float32)
    for j0 in range(0, T, TILE):
        st = S[:, j0:j0 + TILE]
        mt = st.max(axis=1)
        m_new = np.maximum(m, mt)
        # a wave holds 32 query rows; when any of its rows must raise its max,
        # every row of the wave moves to its own new max (factor alpha each)
        grow = np.pad((m_new - m) * c > LAZY, (0, -T % 32))
        raise_ = grow.reshape(-1, 32).any(axis=1).repeat(32)[:T]
        alpha = np.where(raise_, f32(np.exp2(f32((m - m_new) * c))), 1.0)
        m = np.where(raise_, m_new, m)
        l = f32(l * alpha)
        acc = f32(acc * alpha[:, None])
        mc = f32(m * c).astype(np.float64)
        arg = f32(st * c - mc[:, None])
        p = bf16(np.exp2(arg.astype(np.float64)))
        l = f32(l + p.sum(axis=1))
        if keep is not None:
            p = np.where(keep[:, j0:j0 + TILE], p, 0.0)
        acc = f32(acc + p @ v[j0:j0 + TILE])
    o = bf16(acc / l[:, None] * keep_scale)
    lse = f32(m * scale + np.log(l.astype(np.float64))).astype(np.float64)
    return o, lse


def head_backward(q, k, v, o, lse, dO, scale: float, window: int = 0, keep=None,
                  keep_scale: float = 1.0):
    """One head's dq, dk, dv (bf16 values) and Delta (fp32 values) from the
    forward's stored o (bf16) and lse (fp32)."""
    T, _ = q.shape
    c = float(np.float32(scale * LOG2E))
    vis = _visible(T, window)
    S = f32(q @ k.T).astype(np.float64)
    nl = f32(-lse * LOG2E).astype(np.float64)
    P = np.where(vis, f32(np.exp2(f32(S * c + nl[:, None]).astype(np.float64))), 0.0)
    delta = f32((dO * o).sum(axis=1)).astype(np.float64)
    dP = f32(dO @ v.T).astype(np.float64)
    if keep is not None:
        kept = keep & vis
        dS = f32(P * np.where(kept, dP * keep_scale - delta[:, None], -delta[:, None]))
        Pd = np.where(kept, P, 0.0)
    else:
        dS = f32(P * (dP - delta[:, None]))
        Pd = P
    dS = np.where(vis, dS, 0.0)
    Pb, dSb = bf16(Pd), bf16(dS)
    dv = bf16(f32(Pb.T @ dO) * keep_scale)
    dk = bf16(f32(dSb.T @ q) * np.float32(scale))
    dq = bf16(f32(dSb @ k) * np.float32(scale))
    return dq, dk, dv, delta


_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 (Salmon et al., SC 2011) on arrays of 32-bit words held
    in uint64: ten rounds of the two 32 x 32 -> 64-bit products with the
    published multipliers, the key bumped by the published Weyl constants."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(k0) & _MASK, np.uint64(k1) & _MASK
    for _ in range(10):
        p0 = np.uint64(0xD2511F53) * c[0]
        p1 = np.uint64(0xCD9E8D57) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & _MASK,
             (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & _MASK]
        k0 = (k0 + np.uint64(0x9E3779B9)) & _MASK
        k1 = (k1 + np.uint64(0xBB67AE85)) & _MASK
    return c


def keep_mask(B: int, H: int, T: int, seed: int, p16: int, bh0: int = 0):
    """[B, H, T, T] keep decisions of the dropout reading: weight (bh, i, j) is
    kept iff 16-bit half j % 2 of word (j % 8) / 2 of Philox4x32-10(counter
    (j / 8, i, bh, 0), key = the 64-bit seed) is >= p16."""
    nb = (T + 7) // 8
    blk = np.arange(nb, dtype=np.uint64)[None, :]
    row = np.arange(T, dtype=np.uint64)[:, None]
    out = np.zeros((B, H, T, nb * 8), dtype=bool)
    for bh in range(B * H):
        r = philox4x32_10(blk + 0 * row, row + 0 * blk, np.uint64(bh0 + bh), 0,
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
        for t in range(8):
            half = (r[t >> 1] >> np.uint64(16 * (t & 1))) & np.uint64(0xFFFF)
            out[bh // H, bh % H, :, t::8] = half >= np.uint64(p16)
    return out[..., :T]


def attention(q, k, v, dO, scale: float, window: int = 0, keep=None, keep_scale: float = 1.0):
    """[B, H, T, D] inputs (numpy fp64 of bf16 values, or torch tensors);
    keep: optional [B, H, T, T] boolean mask.  Returns a dict of o, lse, dq,
    dk, dv, delta as the rounding model produces them."""
    arrs = [np.asarray(t.double().numpy() if hasattr(t, "double") else t, dtype=np.float64)
            for t in (q, k, v, dO)]
    q, k, v, dO = arrs
    B, H, T, D = q.shape
    out = {n: np.zeros((B, H, T, D)) for n in ("o", "dq", "dk", "dv")}
    out["lse"] = np.zeros((B, H, T))
    out["delta"] = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            kp = None if keep is None else keep[b, h]
            o, lse = head_forward(q[b, h], k[b, h], v[b, h], scale, window, kp, keep_scale)
            dq, dk, dv, dl = head_backward(q[b, h], k[b, h], v[b, h], o, lse, dO[b, h], scale,
                                           window, kp, keep_scale)
            out["o"][b, h], out["lse"][b, h] = o, lse
            out["dq"][b, h], out["dk"][b, h], out["dv"][b, h] = dq, dk, dv
            out["delta"][b, h] = dl
    return out


def dropout_scale(p16: int) -> float:
    return 65536.0 / (65536.0 - p16)


def lazy(q, k, v, dO, scale: float, window: int = 0, p: float = 0.0, seed: int = 0,
         bh0: int = 0):
    """A zero-argument callable that computes attention(...) once, when first
    called (dropout p > 0: keep decisions of pairs bh0 + b * H + h)."""
    memo = {}

    def get():
        if "out" not in memo:
            kw = {}
            if p > 0:
                p16 = min(int(np.floor(p * 65536.0 + 0.5)), 65535)
                B, H, T, _ = q.shape
                kw = dict(keep=keep_mask(B, H, T, seed, p16, bh0), keep_scale=dropout_scale(p16))
            memo["out"] = attention(q, k, v, dO, scale, window, **kw)
        return memo["out"]
    return get
