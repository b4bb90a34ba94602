"""Host-side logic of bench.py (no GPU): the work convention and the refusal
of multi-GPU runs."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("T", [1, 2, 7, 64, 300, 1024])
def test_causal_pairs_follow_the_half_square_convention(T):
    exact = sum(i + 1 for i in range(T))  # keys 0..i for query i
    assert bench.visible_pairs(T) == T * T / 2
    assert bench.visible_pairs(T) + T / 2 == exact
    for W in (T, T + 1, 10 * T):  # a window of at least T keys is the causal mask
        assert bench.visible_pairs(T, W) == bench.visible_pairs(T)


@pytest.mark.parametrize("T,W", [(2, 1), (10, 3), (300, 64), (1024, 256), (1024, 1023)])
def test_window_pairs_match_a_brute_count_less_the_diagonal_half(T, W):
    exact = sum(1 for i in range(T) for j in range(T) if i - W < j <= i)
    # same convention as the causal case: the half of the diagonal is not counted
    assert bench.visible_pairs(T, W) + W / 2 == exact


def test_kernel_work_is_seven_gemms_over_the_causal_half():
    c = workloads.ATTN_CONFIGS["gpt2s"]
    w = bench.kernel_work(c)
    g = c.B * c.H * c.T * c.T * c.D
    assert w["fwd"]["flops"] == 2 * g and w["bwd"]["flops"] == 5 * g
    ww = bench.kernel_work(c, 256)
    assert ww["fwd"]["flops"] == 2 * c.B * c.H * c.D * 2 * (c.T * 256 - 256 * 256 / 2)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
