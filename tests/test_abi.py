"""C ABI contract tests that need no GPU.

The library must load, export every symbol include/causal_attn.h declares, and
reject every bad argument with its status code before any HIP call.  The
pointers below are never dereferenced: each call returns during validation.
"""
import ctypes
import os
import re

import pytest
import torch

import causal_head_self_amd as cat
from causal_head_self_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "causal_attn.h")

# Fake, distinct, 16-byte-aligned addresses far apart (never dereferenced).
P = [0x10000000 * (i + 1) for i in range(14)]

# Every call below hands fake device pointers to the library and expects a
# status from its argument checks.  If one of those checks regressed, a call
# would reach a kernel launch at those addresses; on a host without a GPU that
# launch can only fail, so the module runs only where no GPU is visible.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake device pointers: run where no GPU is visible")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_python_exports():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = cat.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_lds_poison_library_loads_with_the_same_abi():
    """The LDS-poisoning debug build (same sources, -DCATTN_LDS_POISON) is a
    drop-in copy of the release library: same exports, same ABI version."""
    from causal_head_self_amd import build as hip_build
    lib = _lib.load_library(hip_build.LIB_POISON)
    for name in _declared_functions():
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value, name
    assert lib.attn_abi_version() == _lib.ABI_VERSION


def test_abi_version_and_status_strings():
    lib = cat.load_library()
    assert lib.attn_abi_version() == _lib.ABI_VERSION
    seen = set()
    for code in range(0, 14):
        s = cat.attn_status_str(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 14
    assert cat.attn_status_str(1234) == "unknown status"
    assert cat.attn_status_str(-1) == "unknown status"


def _fwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=3, T=17, D=64, scale=0.125,
             dtype=1, stream=None)
    a.update(kw)
    return cat.load_library().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                       a["T"], a["D"], a["scale"], a["dtype"], a["stream"])


def _bwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], dO=P[5], dq=P[6], dk=P[7], dv=P[8],
             delta=P[9], B=2, H=3, T=17, D=64, scale=0.125, dtype=1, stream=None)
    a.update(kw)
    return cat.load_library().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"],
                                       a["dq"], a["dk"], a["dv"], a["delta"], a["B"], a["H"],
                                       a["T"], a["D"], a["scale"], a["dtype"], a["stream"])


def _dq(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[5], lse=P[4], delta=P[9], dq=P[6], B=2, H=3,
             T=17, D=64, scale=0.125, dtype=1, stream=None)
    a.update(kw)
    return cat.load_library().attn_bwd_dq(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"],
                                          a["delta"], a["dq"], a["B"], a["H"], a["T"], a["D"],
                                          a["scale"], a["dtype"], a["stream"])


def _dkdv(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], dO=P[5], lse=P[4], delta=P[9], dk=P[7], dv=P[8], B=2, H=3,
             T=17, D=64, scale=0.125, dtype=1, stream=None)
    a.update(kw)
    return cat.load_library().attn_bwd_dkdv(a["q"], a["k"], a["v"], a["dO"], a["lse"],
                                            a["delta"], a["dk"], a["dv"], a["B"], a["H"],
                                            a["T"], a["D"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("call,names", [
    (_dq, ["q", "k", "v", "o", "dO", "lse", "delta", "dq"]),
    (_dkdv, ["q", "k", "v", "dO", "lse", "delta", "dk", "dv"]),
])
def test_stage_null_pointers(call, names):
    for name in names:
        assert call(**{name: None}) == 1, name


@pytest.mark.parametrize("call", [_dq, _dkdv])
def test_stage_validation(call):
    assert call(T=0) == 2
    assert call(dtype=3) == 4
    assert call(D=96) == 3
    assert call(D=128, dtype=0) == 3
    assert call(T=2 ** 30) == 6


def test_stage_alignment_and_aliasing():
    assert _dq(delta=P[9] + 2) == 5
    assert _dq(o=P[3] + 8) == 5
    assert _dq(delta=P[5]) == 8               # delta inside dO
    assert _dq(delta=P[6]) == 8               # delta inside dq
    assert _dq(dq=P[2]) == 8                  # dq is v
    assert _dq(dq=P[6] + 4) == 5
    assert _dq(scale=-2.0) == 7
    assert _dkdv(dk=P[8]) == 8                # dk is dv
    assert _dkdv(dv=P[9]) == 8                # dv overlaps delta
    assert _dkdv(scale=float("nan")) == 7
    assert _dkdv(lse=P[4] + 1) == 5


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null_pointer(name):
    assert _fwd(**{name: None}) == 1


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "dO", "dq", "dk", "dv", "delta"])
def test_bwd_null_pointer(name):
    assert _bwd(**{name: None}) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0), dict(B=-1), dict(T=-5)])
def test_bad_shape(kw):
    assert _fwd(**kw) == 2
    assert _bwd(**kw) == 2


@pytest.mark.parametrize("D", [0, 1, 16, 48, 96, 256])
def test_unsupported_head_dim(D):
    assert _fwd(D=D) == 3
    assert _bwd(D=D) == 3


def test_head_dim_128_is_bf16_only():
    # fp32 has no D = 128 kernels; in bf16 the D check passes and the next
    # check in order (alignment of a misaligned lse) is the one that fires
    assert _fwd(D=128, dtype=0) == 3
    assert _bwd(D=128, dtype=0) == 3
    assert _fwd(D=128, dtype=1, lse=P[4] + 1) == 5
    assert _bwd(D=128, dtype=1, lse=P[4] + 1) == 5
    assert _dq(D=128, dtype=1, lse=P[4] + 1) == 5
    assert _dkdv(D=128, dtype=1, lse=P[4] + 1) == 5


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_bad_dtype(dtype):
    assert _fwd(dtype=dtype) == 4
    assert _bwd(dtype=dtype) == 4


@pytest.mark.parametrize("name", ["q", "k", "v", "o"])
def test_fwd_misaligned(name):
    base = {"q": P[0], "k": P[1], "v": P[2], "o": P[3]}[name]
    assert _fwd(**{name: base + 8}) == 5


def test_lse_alignment():
    assert _fwd(lse=P[4] + 2) == 5
    assert _bwd(delta=P[9] + 1) == 5


@pytest.mark.parametrize("name", ["dO", "dq", "dk", "dv"])
def test_bwd_misaligned(name):
    base = {"dO": P[5], "dq": P[6], "dk": P[7], "dv": P[8]}[name]
    assert _bwd(**{name: base + 4}) == 5


def test_overflow():
    assert _fwd(T=2 ** 30, D=64) == 6
    assert _fwd(B=2 ** 20, H=2 ** 10, T=2 ** 10, D=32) == 6
    assert _bwd(T=2 ** 26, D=64) == 6


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_bad_scale(scale):
    assert _fwd(scale=scale) == 7
    assert _bwd(scale=scale) == 7


def test_fwd_aliasing():
    assert _fwd(o=P[0]) == 8          # o is q
    assert _fwd(lse=P[2] + 64) == 8   # lse inside v
    assert _fwd(lse=P[3] + 16) == 8   # lse inside o


def test_bwd_aliasing():
    assert _bwd(dq=P[0]) == 8         # dq is q
    assert _bwd(dk=P[6]) == 8         # dk is dq
    assert _bwd(delta=P[4]) == 8      # delta is lse
    assert _bwd(dv=P[5] + 32) == 8    # dv overlaps dO


def test_checks_run_in_documented_order():
    """NULL is reported before shape, shape before dtype, dtype before D."""
    assert _fwd(q=None, B=0, dtype=9, D=7) == 1
    assert _fwd(B=0, dtype=9, D=7) == 2
    assert _fwd(dtype=9, D=7) == 4
    assert _fwd(D=7, scale=-1.0) == 3


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        cat.attn_fwd(q, q, q, q.clone(), torch.zeros(1, 1, 4))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load_library(str(tmp_path / "libcausal_attn.so"))


# ---------------------------------------------------------------------------
# strided views (attn_fwd_strided / attn_bwd_strided): every call below holds
# an invalid argument, so it returns during validation
# ---------------------------------------------------------------------------

B_, H_, T_, D_ = 2, 3, 17, 64
C_ = H_ * D_


def _v(ptr, sb=H_ * T_ * D_, sh=T_ * D_, st=D_):
    return _lib.AttnView(ptr, sb, sh, st)


def _qkv_views(base, elem=2):
    """q, k, v views of one [B][T][3][H][D] buffer at `base`."""
    sb, sh, st = T_ * 3 * C_, D_, 3 * C_
    return [_v(base + i * C_ * elem, sb, sh, st) for i in range(3)]


def _fwd_s(views=None, lse=P[4], B=B_, H=H_, T=T_, D=D_, scale=0.125, dtype=1, window=0,
           dropout_p=0.0):
    v = views or [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3])]
    return cat.load_library().attn_fwd_strided(v[0], v[1], v[2], v[3], lse, B, H, T, D, window,
                                               dropout_p, 0, scale, dtype, None)


def _bwd_s(views=None, lse=P[4], delta=P[9], B=B_, H=H_, T=T_, D=D_, scale=0.125, dtype=1,
           window=0, dropout_p=0.0):
    v = views or [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3]), _v(P[5]), _v(P[6]), _v(P[7]),
                  _v(P[8])]
    return cat.load_library().attn_bwd_strided(v[0], v[1], v[2], v[3], lse, v[4], v[5], v[6],
                                               v[7], delta, B, H, T, D, window, dropout_p, 0,
                                               scale, dtype, None)


def test_strided_null_shape_scale():
    assert _fwd_s(views=[_v(0), _v(P[1]), _v(P[2]), _v(P[3])]) == 1
    assert _fwd_s(lse=0) == 1
    assert _bwd_s(delta=0) == 1
    assert _fwd_s(T=0) == 2
    assert _bwd_s(H=0) == 2
    assert _fwd_s(scale=0.0) == 7
    assert _bwd_s(scale=float("nan")) == 7


# The window and dropout_p checks come after every other check, so a call whose
# only fault is one of them would reach a kernel launch (with the fake pointers
# above) if that check were missing.  Without a GPU such a launch can only fail;
# with one it must not be attempted, so these run on GPU-less hosts only.
_last_check = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="would launch with fake pointers if the check were missing")


@_last_check
def test_strided_negative_window_is_a_shape_error():
    assert _fwd_s(window=-1) == 2
    assert _bwd_s(window=-5) == 2


@_last_check
def test_strided_dropout_probability_range():
    for p in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        assert _fwd_s(dropout_p=p) == 12, p
        assert _bwd_s(dropout_p=p) == 12, p


def test_dropout_keep_bytes():
    kb = cat.load_library().attn_dropout_keep_bytes
    assert kb(2, 3, 17) == 2 * 3 * 1 * 17 * 4
    assert kb(8, 12, 1024) == 8 * 12 * 32 * 1024 * 4
    assert kb(1, 1, 33) == 2 * 33 * 4
    assert kb(0, 1, 1) == 0 and kb(1, 0, 1) == 0 and kb(1, 1, 0) == 0 and kb(-1, 2, 3) == 0


KEEP = P[11]
KEEP_BYTES = 2 * 3 * 1 * 17 * 4


def _fwd_k(keep=KEEP, keep_bytes=KEEP_BYTES, T=T_, dropout_p=0.1, views=None):
    v = views or [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3])]
    return cat.load_library().attn_fwd_strided_keep(v[0], v[1], v[2], v[3], P[4], B_, H_, T, D_, 0,
                                                    dropout_p, 0, 0.125, 1, keep, keep_bytes, None)


def _bwd_k(keep=KEEP, keep_bytes=KEEP_BYTES, T=T_, dropout_p=0.1):
    v = [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3]), _v(P[5]), _v(P[6]), _v(P[7]), _v(P[8])]
    return cat.load_library().attn_bwd_strided_keep(v[0], v[1], v[2], v[3], P[4], v[4], v[5], v[6],
                                                    v[7], P[9], B_, H_, T, D_, 0, dropout_p, 0.125,
                                                    1, keep, keep_bytes, None)


def test_keep_entry_points_check_the_strided_arguments_first():
    assert _fwd_k(T=0, keep=0) == 2        # shape before the keep buffer
    assert _bwd_k(T=0, keep=0) == 2
    assert _fwd_k(dropout_p=1.5, keep=0) == 12
    assert _bwd_k(dropout_p=-1.0, keep=0) == 12


@_last_check
def test_keep_buffer_checks():
    for call in (_fwd_k, _bwd_k):
        assert call(keep=0) == 1                               # null
        assert call(keep=KEEP + 2) == 5                        # not 4-byte aligned
        assert call(keep_bytes=KEEP_BYTES - 4) == 11           # too small
        assert call(keep=P[1] + 64) == 8                       # inside k
        assert call(keep=P[4]) == 8                            # on lse
    assert _bwd_k(keep=P[9] - 4, keep_bytes=KEEP_BYTES) == 8   # overlaps delta


def test_strided_supports_only_bf16_d64_d128():
    assert _fwd_s(dtype=0) == 10
    assert _bwd_s(dtype=0) == 10
    assert _fwd_s(D=32) == 10
    assert _fwd_s(D=48) == 3
    assert _fwd_s(D=128, dtype=0) == 3
    v128 = [_v(P[i], H_ * T_ * 128, T_ * 128, 128) for i in range(4)]
    assert _fwd_s(views=v128, D=128, lse=P[4] + 1) == 5  # D=128 passes the layout check
    assert _fwd_s(D=128, lse=P[4] + 1) == 10              # stride_t 64 < D
    assert _fwd_s(dtype=7) == 4


def test_strided_stride_rules():
    base = [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3])]
    bad = [_v(P[0], st=60), _v(P[0], st=68), _v(P[0], sh=4), _v(P[0], sb=-64),
           _v(P[0], st=1 << 27)]  # stride_t < D, not /8, not /8, negative, T*st*2 >= 2^32
    for b in bad:
        assert _fwd_s(views=[b] + base[1:]) == 10, (b.stride_b, b.stride_h, b.stride_t)
    assert _fwd_s(views=base[:3] + [_v(P[3] + 8)]) == 5  # o not 16-byte aligned
    assert _fwd_s(lse=P[4] + 2) == 5


def test_strided_alias_rules():
    q, k, v = _qkv_views(P[0])
    # inputs may share memory (q, k, v of one qkv buffer); o may not overlap them
    assert _fwd_s(views=[q, k, v, _v(P[0] + 64)]) == 8
    # o equal to an input lattice translate that meets it
    assert _fwd_s(views=[q, k, v, _qkv_views(P[0] + 2 * 64)[0]]) == 8
    # lse inside an input
    assert _fwd_s(views=[q, k, v, _v(P[3])], lse=P[0] + 256) == 8
    # dq, dk, dv interleaved in one [B][T][3][H][D] buffer pass the view check; the
    # call then fails on delta overlapping lse, which is checked after it
    dq, dk, dv = _qkv_views(P[6])
    assert _bwd_s(views=[q, k, v, _v(P[3]), _v(P[5]), dq, dk, dv], delta=P[4]) == 8
    # two outputs at the same address
    assert _bwd_s(views=[q, k, v, _v(P[3]), _v(P[5]), dq, dq, dv]) == 8
    # outputs of one lattice whose token footprints meet (offset 32 elements, footprint 192)
    sb, sh, st = T_ * 3 * C_, D_, 3 * C_
    near = _lib.AttnView(P[6] + 64, sb, sh, st)
    assert _bwd_s(views=[q, k, v, _v(P[3]), _v(P[5]), dq, near, dv]) == 8


# ---------------------------------------------------------------------------
# decode against a KV cache (attn_decode): every call below holds an invalid
# argument, so it returns during validation
# ---------------------------------------------------------------------------

DB, DH, DT, DD = 2, 3, 17, 64


def _ws(B=DB, H=DH, T=DT, D=DD):
    return cat.load_library().attn_decode_workspace_bytes(B, H, T, D)


def _dec(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], lens=P[3], o=P[4], lse=P[5], ws=P[6], ws_bytes=_ws(),
             B=DB, H=DH, T=DT, D=DD, window=0, scale=0.125, dtype=1)
    a.update(kw)
    return cat.load_library().attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"],
                                          a["ws"], a["ws_bytes"], a["B"], a["H"], a["T"],
                                          a["D"], a["window"], a["scale"], a["dtype"], None)


def test_decode_workspace_bytes():
    # one (D + 4)-float partial per (b, h, 64-position slice)
    assert _ws(8, 12, 1024, 64) == 8 * 12 * 16 * 68 * 4
    assert _ws(2, 16, 4097, 128) == 2 * 16 * 65 * 132 * 4
    assert _ws(1, 1, 1, 64) == 68 * 4
    assert _ws(0, 1, 1, 64) == 0 and _ws(1, 1, 0, 64) == 0


@pytest.mark.parametrize("name", ["q", "k", "v", "lens", "o", "lse", "ws"])
def test_decode_null_pointer(name):
    assert _dec(**{name: None}) == 1


@_last_check
def test_decode_validation_order_and_codes():
    assert _dec(B=0) == 2 and _dec(H=0) == 2 and _dec(T=0) == 2 and _dec(window=-1) == 2
    assert _dec(dtype=0) == 4 and _dec(dtype=5) == 4
    assert _dec(D=32) == 3 and _dec(D=96) == 3
    assert _dec(scale=0.0) == 7 and _dec(scale=float("inf")) == 7
    assert _dec(B=2 ** 16, H=2 ** 10, T=2 ** 12, ws_bytes=2 ** 62) == 6
    assert _dec(q=P[0] + 8) == 5 and _dec(o=P[4] + 2) == 5 and _dec(ws=P[6] + 4) == 5
    assert _dec(lse=P[5] + 2) == 5 and _dec(lens=P[3] + 1) == 5
    assert _dec(ws_bytes=_ws() - 1) == 11 and _dec(ws_bytes=0) == 11
    assert _dec(o=P[0]) == 8                      # o is q
    assert _dec(ws=P[1]) == 8                     # workspace is the key cache
    assert _dec(lse=P[6] + 64) == 8               # lse inside the workspace
    assert _dec(o=P[3]) == 8                      # o over cache_lens
    # D = 128 passes the head-dim check (the misaligned q is what fires)
    assert _dec(D=128, ws_bytes=_ws(D=128), q=P[0] + 8) == 5


# ---------------------------------------------------------------------------
# RoPE / QK norm (attn_rope_qknorm_fwd / _bwd): invalid arguments only
# ---------------------------------------------------------------------------

def _rope(fwd=True, views=None, B=B_, H=H_, T=T_, D=D_, pos0=0, base=10000.0, qg=1.2, kg=1.0,
          eps=1e-6, flags=3, dtype=1):
    lib = cat.load_library()
    if fwd:
        v = views or [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3])]
        return lib.attn_rope_qknorm_fwd(*v, B, H, T, D, pos0, base, qg, kg, eps, flags, dtype, None)
    v = views or [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3]), _v(P[4]), _v(P[5])]
    return lib.attn_rope_qknorm_bwd(*v, B, H, T, D, pos0, base, qg, kg, eps, flags, dtype, None)


@_last_check
@pytest.mark.parametrize("fwd", [True, False])
def test_rope_qknorm_validation(fwd):
    n = 4 if fwd else 6
    for i in range(n):  # a NULL view
        views = [_v(P[j]) for j in range(n)]
        views[i] = _v(None)
        assert _rope(fwd, views=views) == 1
    assert _rope(fwd, B=0) == 2
    assert _rope(fwd, dtype=0) == 10 and _rope(fwd, D=32) == 10 and _rope(fwd, D=48) == 3
    for kw in (dict(flags=4), dict(flags=-1), dict(pos0=-1), dict(pos0=2 ** 24), dict(base=0.0),
               dict(base=float("inf")), dict(qg=float("nan")), dict(kg=float("inf")),
               dict(eps=-1e-3), dict(eps=float("nan"))):
        assert _rope(fwd, **kw) == 12, kw
    views = [_v(P[j]) for j in range(n)]
    views[n - 1] = _v(P[0])                       # an output on an input
    assert _rope(fwd, views=views) == 8
    views = [_v(P[j]) for j in range(n)]
    views[n - 1] = _v(P[n - 2])                   # the two outputs on each other
    assert _rope(fwd, views=views) == 8


# ---------------------------------------------------------------------------
# outputs that address one element twice
# ---------------------------------------------------------------------------

def test_self_overlapping_output_views_are_rejected():
    B, H, T, D = B_, H_, T_, D_
    # stride_h = 0 with H > 1: every head writes the same rows
    bad = cat.AttnView(P[3], H * T * D, 0, D)
    assert _fwd_s(views=[_v(P[0]), _v(P[1]), _v(P[2]), bad]) == 8
    # 0 < stride_h < D: neighbouring heads overlap
    bad = cat.AttnView(P[3], H * T * D, 8, T * D)
    assert _fwd_s(views=[_v(P[0]), _v(P[1]), _v(P[2]), bad]) == 8
    # stride_b below one batch's footprint
    bad = cat.AttnView(P[3], T * D, T * D, D)
    assert _fwd_s(views=[_v(P[0]), _v(P[1]), _v(P[2]), bad]) == 8
    # the same for gradients of the backward (dq of the [B, T, 3C] layout is fine,
    # a dk view with stride_t < H * D across heads is not)
    C = H * D
    v = [_v(P[0]), _v(P[1]), _v(P[2]), _v(P[3]), _v(P[5]), _v(P[6]), _v(P[7]), _v(P[8])]
    v[6] = cat.AttnView(P[7], T * C, D, D)
    assert _bwd_s(views=v) == 8


# ---------------------------------------------------------------------------
# attention with the fused RoPE / QK-norm prologue: invalid arguments only
# ---------------------------------------------------------------------------

def _frope(views=None, lse=P[12], B=B_, H=H_, T=T_, D=D_, window=0, scale=0.125, pos0=0,
           base=10000.0, qg=1.2, kg=1.0, eps=1e-6, flags=3, dtype=1):
    v = views or [_v(P[j]) for j in (0, 1, 2, 3, 4, 5)]
    return cat.load_library().attn_fwd_strided_rope(v[0], v[1], v[2], v[3], lse, v[4], v[5], B, H,
                                                    T, D, window, scale, pos0, base, qg, kg, eps,
                                                    flags, dtype, None)


def _brope(views=None, lse=P[12], delta=P[13], B=B_, H=H_, T=T_, D=D_, window=0, scale=0.125,
           pos0=0, base=10000.0, qg=1.2, kg=1.0, eps=1e-6, flags=3, dtype=1):
    v = views or [_v(P[j]) for j in range(10)]
    return cat.load_library().attn_bwd_strided_rope(v[0], v[1], v[2], v[3], v[4], v[5], lse, v[6],
                                                    v[7], v[8], v[9], delta, B, H, T, D, window,
                                                    scale, pos0, base, qg, kg, eps, flags, dtype,
                                                    None)


@pytest.mark.parametrize("fwd", [True, False])
def test_fused_prologue_validation(fwd):
    call, n = (_frope, 6) if fwd else (_brope, 10)
    for i in range(n):  # a NULL view
        views = [_v(P[j]) for j in range(n)]
        views[i] = _v(None)
        assert call(views=views) == 1, i
    assert call(lse=0) == 1
    if not fwd:
        assert call(delta=0) == 1
    assert call(T=0) == 2 and call(window=-1) == 2
    assert call(dtype=0) == 10 and call(D=32) == 10 and call(D=48) == 3
    assert call(scale=0.0) == 7
    for kw in (dict(flags=4), dict(pos0=-1), dict(pos0=2 ** 24), dict(base=0.0),
               dict(qg=float("nan")), dict(eps=-1.0)):
        assert call(**kw) == 12, kw
    views = [_v(P[j]) for j in range(n)]
    views[n - 1] = _v(P[0])                       # an output on an input
    assert call(views=views) == 8
    views = [_v(P[j]) for j in range(n)]
    views[n - 1] = _v(P[n - 2])                   # two outputs on each other
    assert call(views=views) == 8
    if fwd:
        assert call(lse=P[1] + 64) == 8           # lse (an output) inside an input view
    else:
        assert call(delta=P[1] + 64) == 8         # delta (an output) inside an input view
        assert call(delta=P[12]) == 8             # delta on lse


# ---------------------------------------------------------------------------
# row passes (attn_layernorm_fwd / _bwd, attn_colsum): invalid arguments only
# ---------------------------------------------------------------------------

N_, C_ = 64, 768


def _ln_fwd(x=P[0], g=P[1], b=P[2], y=P[3], N=N_, C=C_, stride=C_, eps=1e-5, dtype=1):
    return cat.load_library().attn_layernorm_fwd(x, g, b, y, N, C, stride, eps, dtype, None)


def _ln_ws(N=N_, C=C_):
    return cat.load_library().attn_layernorm_workspace_bytes(N, C)


def _ln_bwd(x=P[0], g=P[1], dy=P[2], dres=P[3], dx=P[4], dg=P[5], db=P[6], ws=P[7],
            ws_bytes=None, N=N_, C=C_, stride=C_, eps=1e-5, dtype=1):
    ws_bytes = _ln_ws(N, C) if ws_bytes is None else ws_bytes
    return cat.load_library().attn_layernorm_bwd(x, g, dy, dres, dx, dg, db, ws, ws_bytes, N, C,
                                                 stride, eps, dtype, None)


def _cs_ws(N=N_, M=C_):
    return cat.load_library().attn_colsum_workspace_bytes(N, M)


def _cs(x=P[0], out=P[1], ws=P[2], ws_bytes=None, N=N_, M=C_, stride=C_, dtype=1):
    ws_bytes = _cs_ws(N, M) if ws_bytes is None else ws_bytes
    return cat.load_library().attn_colsum(x, out, ws, ws_bytes, N, M, stride, dtype, None)


def test_row_pass_workspace_bytes():
    # LayerNorm gradient: [dg | db] partials per 16 rows; column sums: per block
    # of max(8, ceil(N / 128)) rows
    assert _ln_ws(8192, 768) == 512 * 2 * 768 * 4
    assert _ln_ws(17, 8) == 2 * 2 * 8 * 4
    assert _cs_ws(8192, 2304) == 128 * 2304 * 4
    assert _cs_ws(8200, 8) == 127 * 8 * 4 and _cs_ws(33, 8) == 5 * 8 * 4
    assert _ln_ws(0, 768) == 0 and _cs_ws(1, 0) == 0


@pytest.mark.parametrize("name", ["x", "g", "b", "y"])
def test_layernorm_fwd_null_pointer(name):
    assert _ln_fwd(**{name: None}) == 1


@pytest.mark.parametrize("name", ["x", "g", "dy", "dx", "dg", "db", "ws"])
def test_layernorm_bwd_null_pointer(name):
    assert _ln_bwd(**{name: None}) == 1


@_last_check
def test_row_pass_validation_order_and_codes():
    # shape: N >= 1, 8 <= C <= 4096 (LayerNorm), C % 8 == 0
    assert _ln_fwd(N=0) == 2 and _ln_fwd(C=4) == 2 and _ln_fwd(C=12, stride=16) == 2
    assert _ln_fwd(C=4104, stride=4104) == 2 and _ln_bwd(C=0) == 2 and _cs(M=12, stride=16) == 2
    assert _ln_fwd(dtype=0) == 4 and _ln_bwd(dtype=0) == 4 and _cs(dtype=2) == 4
    assert _ln_fwd(stride=760) == 10 and _ln_fwd(stride=772) == 10 and _cs(stride=100) == 10
    assert _ln_fwd(eps=-1.0) == 12 and _ln_fwd(eps=float("nan")) == 12
    assert _ln_bwd(eps=float("inf")) == 12
    assert _ln_fwd(x=P[0] + 8) == 5 and _ln_fwd(g=P[1] + 2) == 5 and _ln_fwd(y=P[3] + 4) == 5
    assert _ln_bwd(dres=P[3] + 8) == 5 and _ln_bwd(ws=P[7] + 4) == 5 and _cs(out=P[1] + 2) == 5
    assert _ln_bwd(ws_bytes=_ln_ws() - 1) == 11 and _cs(ws_bytes=_cs_ws() - 4) == 11
    assert _ln_fwd(y=P[0]) == 8                    # y is x
    assert _ln_fwd(y=P[1] - 64) == 8               # y runs into g
    assert _ln_bwd(dx=P[2]) == 8                   # dx is dy
    assert _ln_bwd(dx=P[3] + 16) == 8              # dx inside dres
    assert _ln_bwd(dg=P[4] + 32) == 8              # dg inside dx
    assert _ln_bwd(ws=P[6]) == 8                   # workspace over db
    assert _cs(out=P[0] + 64) == 8 and _cs(ws=P[1]) == 8
    # no residual term is allowed
    assert _ln_bwd(dres=None, dx=P[0]) == 8
    # fp32 rows (split-K partials): no workspace needed, the other checks as for bf16
    assert _cs(ws=None) == 1
    assert _cs(dtype=0, ws=None, M=12, stride=16) == 2 and _cs(dtype=0, ws=None, stride=100) == 10
    assert _cs(dtype=0, ws=None, x=P[0] + 8) == 5 and _cs(dtype=0, ws=None, out=P[0] + 64) == 8
