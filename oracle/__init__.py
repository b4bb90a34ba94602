"""fp64 CPU oracle for causal multi-head self-attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this package; the product library never does.  It
shares no code with the HIP path (see ``oracle.c`` for the definition it
implements and the passages it follows).

All functions take and return float64 NumPy arrays in the [B, H, T, D] layout
(lse and delta are [B, H, T]).  ``scale`` is widened from the float32 value the
GPU receives, so both sides compute the same function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_libs: dict = {}

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def compile_source(src: str, out: str) -> str:
    """gcc -O2 (no fast-math) with OpenMP: the one way the oracle is built."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", src, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    lib.oracle_attn_fwd.argtypes = [_dp] * 5 + [_i64] * 4 + [ctypes.c_double, _i64, _i64]
    lib.oracle_attn_fwd.restype = None
    lib.oracle_attn_bwd.argtypes = [_dp] * 8 + [_i64] * 4 + [ctypes.c_double, _i64, _i64]
    lib.oracle_attn_bwd.restype = None
    lib.oracle_sublayer_fwd.argtypes = [_dp] * 8 + [_i64] * 4 + [ctypes.c_double, _i64]
    lib.oracle_sublayer_fwd.restype = ctypes.c_int
    lib.oracle_sublayer_bwd.argtypes = [_dp] * 15 + [_i64] * 4 + [ctypes.c_double, _i64]
    lib.oracle_sublayer_bwd.restype = ctypes.c_int
    lib.oracle_attn_decode.argtypes = ([_dp] * 3 + [ctypes.POINTER(ctypes.c_int64)] + [_dp] * 2 +
                                       [_i64] * 4 + [ctypes.c_double, _i64, _i64])
    lib.oracle_attn_decode.restype = None
    lib.oracle_rope_qknorm_fwd.argtypes = [_dp] * 2 + [_i64] * 5 + [ctypes.c_double, _i64, _i64,
                                                                    ctypes.c_double, ctypes.c_double]
    lib.oracle_rope_qknorm_fwd.restype = None
    lib.oracle_rope_qknorm_bwd.argtypes = [_dp] * 3 + [_i64] * 5 + [ctypes.c_double, _i64, _i64,
                                                                    ctypes.c_double, ctypes.c_double]
    lib.oracle_rope_qknorm_bwd.restype = None
    _u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_dropout_keep.argtypes = [ctypes.c_uint64, _i64, _i64, _i64, _i64]
    lib.oracle_dropout_keep.restype = ctypes.c_int
    lib.oracle_attn_fwd_dropout.argtypes = ([_dp] * 5 + [_i64] * 4 +
                                            [ctypes.c_double, _i64, _i64, ctypes.c_uint64, _i64,
                                             _i64])
    lib.oracle_attn_fwd_dropout.restype = None
    lib.oracle_attn_bwd_dropout.argtypes = ([_dp] * 8 + [_i64] * 4 +
                                            [ctypes.c_double, _i64, _i64, ctypes.c_uint64, _i64,
                                             _i64])
    lib.oracle_attn_bwd_dropout.restype = None
    lib.oracle_layernorm_fwd.argtypes = [_dp] * 4 + [_i64] * 2 + [ctypes.c_double, _i64]
    lib.oracle_layernorm_fwd.restype = ctypes.c_int
    lib.oracle_layernorm_bwd.argtypes = [_dp] * 8 + [_i64] * 2 + [ctypes.c_double, _i64]
    lib.oracle_layernorm_bwd.restype = ctypes.c_int
    lib.oracle_colsum.argtypes = [_dp, _dp, _i64, _i64]
    lib.oracle_colsum.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


_override: list = []


class use_library:
    """Context manager: route every call to another build of the oracle source
    (the planted-mistake tests use it to show that the pins catch slips)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        _override.append(self.path)
        return self

    def __exit__(self, *exc):
        _override.pop()
        return False


def _load(path: str | None = None):
    """The compiled oracle (built on first use).  ``path`` selects another
    build of the same source, e.g. a copy with a planted mistake in a test."""
    if path is None and _override:
        path = _override[-1]
    if path is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        path = _LIB
    if path not in _libs:
        _libs[path] = _bind(path)
    return _libs[path]


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def widen_scale(scale: float) -> float:
    """The float32 value the GPU receives, widened exactly to float64."""
    return float(np.float32(scale))


def attn_fwd(q, k, v, scale: float, nthreads: int = 0, lib: str | None = None,
             window: int = 0):
    """Returns (o [B,H,T,D], lse [B,H,T]) in float64.  window = W > 0 restricts
    query i to keys i-W < j <= i (sliding window); 0 is the full causal mask."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    _load(lib).oracle_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, T, D,
                            float(scale), int(window), int(nthreads))
    return o, lse


def attn_bwd(q, k, v, dO, scale: float, nthreads: int = 0, lib: str | None = None,
             window: int = 0):
    """Returns (dq, dk, dv, delta) in float64 for the upstream gradient dO
    (window as in attn_fwd)."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, T, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dO.shape == q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    delta = np.empty((B, H, T), dtype=np.float64)
    _load(lib).oracle_attn_bwd(_p(q), _p(k), _p(v), _p(dO), _p(dq), _p(dk), _p(dv),
                            _p(delta), B, H, T, D, float(scale), int(window), int(nthreads))
    return dq, dk, dv, delta


def attn_decode(q, k_cache, v_cache, lens, scale: float, window: int = 0, nthreads: int = 0,
                lib: str | None = None):
    """One new token per sequence against its KV cache.  q: [B, H, D];
    k_cache, v_cache: [B, Tmax, H, D]; lens: [B] cached positions per sequence
    (the token itself is the last).  Returns (o [B, H, D], lse [B, H]) in
    float64; a sequence with len 0 gets o = 0, lse = -inf."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Tmax, H, D = kc.shape
    assert q.shape == (B, H, D) and vc.shape == kc.shape
    ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int64))
    assert ln.shape == (B,) and np.all(ln >= 0) and np.all(ln <= Tmax)
    o = np.empty((B, H, D), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    _load(lib).oracle_attn_decode(_p(q), _p(kc), _p(vc), ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                               _p(o), _p(lse), B, H, Tmax, D, float(scale), int(window),
                               int(nthreads))
    return o, lse


def dropout_threshold(p: float) -> int:
    """p16 = round(p * 65536), the integer threshold of a 16-bit draw (0 <= p < 1)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout p must be in [0, 1)")
    return min(int(np.floor(p * 65536.0 + 0.5)), 65535)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter under a 2-word key -> 4 words."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    kk = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    _load().oracle_philox4x32_10(c, kk, out)
    return [int(x) for x in out]


def dropout_keep(seed: int, p16: int, bh: int, i: int, j: int) -> bool:
    return bool(_load().oracle_dropout_keep(int(seed), int(p16), int(bh), int(i), int(j)))


def attn_fwd_dropout(q, k, v, scale: float, p: float, seed: int, window: int = 0,
                     nthreads: int = 0, lib: str | None = None, bh0: int = 0):
    """Forward with attention dropout (see oracle.c): returns (o, lse).  bh0 is
    the global (batch, head) index of the first pair given."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, D = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    _load(lib).oracle_attn_fwd_dropout(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, T, D,
                                    float(scale), int(window), dropout_threshold(p),
                                    int(seed) & (2 ** 64 - 1), int(bh0), int(nthreads))
    return o, lse


def attn_bwd_dropout(q, k, v, dO, scale: float, p: float, seed: int, window: int = 0,
                     nthreads: int = 0, lib: str | None = None, bh0: int = 0):
    """Backward with attention dropout: returns (dq, dk, dv, delta)."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, T, D = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    delta = np.empty((B, H, T), dtype=np.float64)
    _load(lib).oracle_attn_bwd_dropout(_p(q), _p(k), _p(v), _p(dO), _p(dq), _p(dk), _p(dv),
                                    _p(delta), B, H, T, D, float(scale), int(window),
                                    dropout_threshold(p), int(seed) & (2 ** 64 - 1), int(bh0),
                                    int(nthreads))
    return dq, dk, dv, delta


def rope_qknorm_fwd(x, pos0: int = 0, base: float = 10000.0, rope: bool = True,
                    norm: bool = True, gain: float = 1.0, eps: float = 1e-6,
                    lib: str | None = None):
    """RoPE (pairs (i, i + D/2), angle (pos0 + t) * base^(-2i/D)) and QK norm
    (x / sqrt(mean(x^2) + eps) * gain) of every row of x [B, H, T, D]."""
    x = _f64(x)
    B, H, T, D = x.shape
    y = np.empty_like(x)
    _load(lib).oracle_rope_qknorm_fwd(_p(x), _p(y), B, H, T, D, int(pos0), float(base),
                                   int(bool(rope)), int(bool(norm)), float(gain), float(eps))
    return y


def rope_qknorm_bwd(x, dy, pos0: int = 0, base: float = 10000.0, rope: bool = True,
                    norm: bool = True, gain: float = 1.0, eps: float = 1e-6,
                    lib: str | None = None):
    """Gradient with respect to x of sum(dy * rope_qknorm_fwd(x))."""
    x, dy = _f64(x), _f64(dy)
    B, H, T, D = x.shape
    dx = np.empty_like(x)
    _load(lib).oracle_rope_qknorm_bwd(_p(x), _p(dy), _p(dx), B, H, T, D, int(pos0), float(base),
                                   int(bool(rope)), int(bool(norm)), float(gain), float(eps))
    return dx


def sublayer_fwd(x, g, bl, Wa, ba, Wp, bp, n_head: int, eps: float = 1e-5,
                 nthreads: int = 0, lib: str | None = None):
    """Pre-norm attention sublayer forward.  x: [B,T,C]; Wa: [C,3C]; Wp: [C,C]."""
    x, g, bl, Wa, ba, Wp, bp = map(_f64, (x, g, bl, Wa, ba, Wp, bp))
    B, T, C = x.shape
    y = np.empty_like(x)
    rc = _load(lib).oracle_sublayer_fwd(_p(x), _p(g), _p(bl), _p(Wa), _p(ba), _p(Wp), _p(bp),
                                     _p(y), B, T, C, int(n_head), float(eps), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_sublayer_fwd failed ({rc})")
    return y


def sublayer_bwd(x, g, bl, Wa, ba, Wp, bp, dy, n_head: int, eps: float = 1e-5,
                 nthreads: int = 0, lib: str | None = None):
    """Gradients of sum(dy * y): returns dict dx, dg, dbl, dWa, dba, dWp, dbp."""
    x, g, bl, Wa, ba, Wp, bp, dy = map(_f64, (x, g, bl, Wa, ba, Wp, bp, dy))
    B, T, C = x.shape
    out = {
        "dx": np.empty_like(x), "dg": np.empty_like(g), "dbl": np.empty_like(bl),
        "dWa": np.empty_like(Wa), "dba": np.empty_like(ba), "dWp": np.empty_like(Wp),
        "dbp": np.empty_like(bp),
    }
    rc = _load(lib).oracle_sublayer_bwd(
        _p(x), _p(g), _p(bl), _p(Wa), _p(ba), _p(Wp), _p(bp), _p(dy),
        _p(out["dx"]), _p(out["dg"]), _p(out["dbl"]), _p(out["dWa"]), _p(out["dba"]),
        _p(out["dWp"]), _p(out["dbp"]), B, T, C, int(n_head), float(eps), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_sublayer_bwd failed ({rc})")
    return out


def layernorm_fwd(x, g, bl, eps: float = 1e-5, nthreads: int = 0, lib: str | None = None):
    """LayerNorm over the last dimension of x [N, C] (biased variance, eps under
    the square root), times g [C] plus bl [C]."""
    x, g, bl = map(_f64, (x, g, bl))
    N, C = x.shape
    y = np.empty_like(x)
    rc = _load(lib).oracle_layernorm_fwd(_p(x), _p(g), _p(bl), _p(y), N, C, float(eps),
                                         int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_layernorm_fwd failed ({rc})")
    return y


def layernorm_bwd(x, g, bl, du, dres=None, eps: float = 1e-5, nthreads: int = 0,
                  lib: str | None = None):
    """Gradients of sum(du * layernorm_fwd(x)) + sum(dres * x): (dx, dg, dbl)."""
    x, g, bl, du = map(_f64, (x, g, bl, du))
    N, C = x.shape
    dr = None if dres is None else _f64(dres)
    dx = np.empty_like(x)
    dg, dbl = np.empty_like(g), np.empty_like(bl)
    rc = _load(lib).oracle_layernorm_bwd(_p(x), _p(g), _p(bl), _p(du),
                                         None if dr is None else _p(dr), _p(dx), _p(dg),
                                         _p(dbl), N, C, float(eps), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_layernorm_bwd failed ({rc})")
    return dx, dg, dbl


def colsum(x, lib: str | None = None):
    """Column sums of x [N, M]: the gradient of a bias added to every row."""
    x = _f64(x)
    N, M = x.shape
    out = np.empty(M, dtype=np.float64)
    _load(lib).oracle_colsum(_p(x), _p(out), N, M)
    return out
