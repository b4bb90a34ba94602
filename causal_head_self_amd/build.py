"""Build libcausal_attn.so (the gfx950 HIP kernels plus the C ABI) in-tree.

    python -m causal_head_self_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (``-Xclang -target-feature -Xclang -packed-fp32-ops``).

A second library, libcausal_attn_lds_poison.so, is the same sources compiled
with -DCATTN_LDS_POISON: each kernel fills its LDS arrays with NaN words
before first use, so a read of LDS the kernel never wrote changes its results
(tests/test_gpu_lds_poison.py compares the two libraries bit for bit).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcausal_attn.so")
LIB_POISON = os.path.join(PKG, "libcausal_attn_lds_poison.so")
POISON_FLAGS = ["-DCATTN_LDS_POISON"]
SOURCES = ["attn_api.hip", "attn_bf16.hip", "attn_bf16_d64.hip", "attn_bwd_plain.hip", "attn_decode.hip", "attn_f32.hip",
           "attn_norm.hip", "attn_rope.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Kernel-only sources: NaN inputs are outside the contract (results unspecified),
# so fmax needs no NaN canonicalisation.  Not used for attn_api.hip, whose
# argument checks must see NaN.
KERNEL_ONLY_FLAGS = {
    "attn_bf16_d64.hip": ["-fno-honor-nans"],
    # the one-launch backward without dropout alone, under LLVM's iterative ILP
    # machine scheduler (see the head of that file)
    "attn_bwd_plain.hip": ["-fno-honor-nans", "-mllvm", "--amdgpu-sched-strategy=iterative-ilp"],
}


def _compile(job) -> str:
    src, poison = job
    tag = "_lds_poison" if poison else ""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *KERNEL_ONLY_FLAGS.get(src, []), *(POISON_FLAGS if poison else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, lds_poison: bool = True) -> str:
    """Compile and link libcausal_attn.so (and, unless lds_poison is False,
    the LDS-poisoning debug library beside it).  Returns the release path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, False) for src in SOURCES]
    if lds_poison:
        jobs += [(src, True) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    if lds_poison:
        _link(objs[len(SOURCES):], LIB_POISON)
    if verbose:
        print(f"built {LIB}" + (f" and {LIB_POISON}" if lds_poison else ""))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
