"""Host AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

* The fp64 oracle (oracle/oracle.c) is built with gcc and
  -fsanitize=address,undefined and driven over ragged shapes, windows and
  dropout, forward and backward, decode, the RoPE / QK-norm prologue and the
  sublayer, in a child process with the sanitizer runtime preloaded.
* The library's host code (attn_api.hip: argument checks, view-overlap tests,
  size arithmetic) is recompiled with the sanitizers on its host pass only and
  linked with the release kernel objects; tests/test_abi.py then runs against
  that library, every call ending in its argument checks (no GPU is used).

Any out-of-bounds access, use after free or undefined operation (signed
overflow, misaligned load, bad shift) aborts the child with a report.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "causal_head_self_amd")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only sanitizer runs (fake device pointers)")


def _run(script: str, preload: str, *args) -> subprocess.CompletedProcess:
    env = dict(os.environ, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-c", script, *args], env=env, cwd=ROOT,
                          capture_output=True, text=True, timeout=600)


def _gcc_asan() -> str:
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's libasan is not installed")
    return asan


def _sanitized_oracle(src: str, lib: str) -> str:
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fopenmp", "-fPIC", "-shared", "-Wall", src, "-o", lib, "-lm"], check=True)
    return lib


ORACLE_SCRIPT = textwrap.dedent("""
        import sys
        import numpy as np
        import oracle
        rng = np.random.default_rng(0)
        with oracle.use_library(sys.argv[1]):
            for (B, H, T, D, W) in ((1, 2, 37, 16, 0), (2, 1, 70, 32, 9), (1, 1, 1, 8, 0)):
                q, k, v, g = (rng.standard_normal((B, H, T, D)) for _ in range(4))
                o, lse = oracle.attn_fwd(q, k, v, 0.25, window=W)
                oracle.attn_bwd(q, k, v, g, 0.25, window=W)
                oracle.attn_fwd_dropout(q, k, v, 0.25, 0.3, 7, window=W)
                oracle.attn_bwd_dropout(q, k, v, g, 0.25, 0.3, 7, window=W)
            for D in (16, 64):
                x, dy = (rng.standard_normal((1, 2, 19, D)) for _ in range(2))
                oracle.rope_qknorm_fwd(x, pos0=3, gain=1.2)
                oracle.rope_qknorm_bwd(x, dy, pos0=3, gain=1.2)
            qd = rng.standard_normal((3, 2, 16))
            kc, vc = (rng.standard_normal((3, 40, 2, 16)) for _ in range(2))
            oracle.attn_decode(qd, kc, vc, np.array([0, 17, 40]), 0.25)
            oracle.attn_decode(qd, kc, vc, np.array([5, 40, 1]), 0.25, window=6)
            B, T, C, nh = 2, 9, 16, 2
            x, dy = rng.standard_normal((B, T, C)), rng.standard_normal((B, T, C))
            w = (rng.standard_normal(C), rng.standard_normal(C),
                 rng.standard_normal((C, 3 * C)) * 0.1, rng.standard_normal(3 * C) * 0.1,
                 rng.standard_normal((C, C)) * 0.1, rng.standard_normal(C))
            oracle.sublayer_fwd(x, *w, n_head=nh)
            oracle.sublayer_bwd(x, *w, dy, n_head=nh)
            x2 = x.reshape(B * T, C)
            oracle.layernorm_fwd(x2, w[0], w[1])
            oracle.layernorm_bwd(x2, w[0], w[1], dy.reshape(B * T, C), x2)
            oracle.layernorm_bwd(x2, w[0], w[1], dy.reshape(B * T, C))
            oracle.colsum(x2)
        print("sanitized oracle: ok")
    """)


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan = _gcc_asan()
    lib = _sanitized_oracle(os.path.join(ROOT, "oracle", "oracle.c"),
                            str(tmp_path / "liboracle_san.so"))
    r = _run(ORACLE_SCRIPT, asan, lib)
    assert r.returncode == 0 and "sanitized oracle: ok" in r.stdout, r.stdout[-3000:] + r.stderr[-6000:]


def test_sanitized_oracle_run_catches_a_planted_overflow(tmp_path):
    """The same run on a copy of the oracle that writes each lse one row too
    far must stop with an AddressSanitizer report (the check is live)."""
    asan = _gcc_asan()
    text = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "lse[bh * T + i] = m + log(Z);"
    assert text.count(good) == 1
    src = tmp_path / "oracle_planted.c"
    src.write_text(text.replace(good, "lse[bh * T + i + 1] = m + log(Z);"))
    lib = _sanitized_oracle(str(src), str(tmp_path / "liboracle_planted.so"))
    r = _run(ORACLE_SCRIPT, asan, lib)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-3000:]


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    from causal_head_self_amd import build as hip_build
    objs = [os.path.join(PKG, "_build", os.path.splitext(n)[0] + ".o") for n in hip_build.SOURCES
            if n != "attn_api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    assert not missing, f"build the library first (python -m causal_head_self_amd.build): {missing}"
    api_o = str(tmp_path / "attn_api_san.o")
    lib = str(tmp_path / "libcausal_attn_san.so")
    # the sanitizers instrument the host pass only (each flag after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hip_build.HIPCC, *hip_build.FLAGS, "-O1", "-g", *san, "-c",
                    os.path.join(PKG, "csrc", "attn_api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([hip_build.HIPCC, f"--offload-arch={hip_build.ARCH}", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    api_o, *objs, "-o", lib], check=True, capture_output=True)
    script = textwrap.dedent("""
        import ctypes, sys
        import pytest
        from causal_head_self_amd import _lib
        _lib.LIB_PATH = sys.argv[1]
        assert _lib.load_library()._name == sys.argv[1]
        assert hasattr(ctypes.CDLL(None), "__asan_init"), "the ASan runtime is not loaded"
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py"]))
    """)
    r = _run(script, rt[-1], lib)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert " passed" in r.stdout
