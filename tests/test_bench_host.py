"""Host-side logic of bench.py (no GPU): the work convention and the refusal
of multi-GPU runs, and the seeded input generators."""
import os
import subprocess
import sys

import pytest
import torch

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


def test_device_input_generators_follow_the_host_recipe():
    """The device-side generators (used for tensors too large to draw on the
    host) give bf16 tensors of the stated shapes, reproducible per seed, with
    q, k, v, dO drawn from different streams and unit-variance values.  Run
    here on the CPU device."""
    q, k, v, dO = workloads.device_attention_inputs(2, 3, 40, 64, "cpu", seed=5)
    again = workloads.device_attention_inputs(2, 3, 40, 64, "cpu", seed=5)
    for a, b in zip((q, k, v, dO), again):
        assert a.shape == (2, 3, 40, 64) and a.dtype == torch.bfloat16
        assert torch.equal(a, b)
    assert not torch.equal(q, k) and not torch.equal(v, dO)
    x = torch.cat([t.float().flatten() for t in (q, k, v, dO)])
    assert abs(float(x.mean())) < 0.05 and abs(float(x.std()) - 1.0) < 0.05
    # with one batch the device recipe is the host recipe on the CPU device
    q1, _, _, _ = workloads.device_attention_inputs(1, 3, 40, 64, "cpu", seed=5)
    assert torch.equal(q1, workloads.attention_inputs(1, 3, 40, 64, "bf16", 5)[0])
    qd, kc, vc = workloads.device_decode_inputs(3, 2, 50, 64, "cpu", seed=9)
    assert qd.shape == (3, 2, 64) and kc.shape == vc.shape == (3, 50, 2, 64)
    assert qd.dtype == kc.dtype == vc.dtype == torch.bfloat16
    assert torch.equal(kc, workloads.device_decode_inputs(3, 2, 50, 64, "cpu", seed=9)[1])
