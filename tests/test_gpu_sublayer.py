"""GPU parity of the pre-norm attention sublayer (LayerNorm -> c_attn -> causal
MHA (HIP kernels) -> c_proj + residual) against the fp64 oracle sublayer.

x, y and dx keep the plain bf16 tolerance 2e-2.  Tensors that are not unit
variance (weight and bias gradients, summed over B*T rows, and the LN-weight
gradient) are compared as |gpu - ref| <= 2e-2 * max(1, rms(ref)).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _run(cfg, B):
    from causal_head_self_amd.sublayer import attention_sublayer
    print(f"[sublayer] B={B} T={cfg.T} C={cfg.C} H={cfg.H}", flush=True)
    sys.stdout.flush()
    inp = workloads.sublayer_inputs(cfg, B=B)
    names = ["x", "g", "bl", "Wa", "ba", "Wp", "bp"]
    dev = {n: inp[n].cuda().requires_grad_(True) for n in names}
    y = attention_sublayer(dev["x"], dev["g"], dev["bl"], dev["Wa"], dev["ba"], dev["Wp"],
                           dev["bp"], cfg.H)
    y.backward(inp["dy"].cuda())
    torch.cuda.synchronize()
    got = {"y": y.detach().float().cpu().numpy()}
    for n in names:
        got["d" + n] = dev[n].grad.float().cpu().numpy()
    args = [inp[n] for n in names]
    ref = {"y": oracle.sublayer_fwd(*args, n_head=cfg.H)}
    ref.update(oracle.sublayer_bwd(*args, dy=inp["dy"], n_head=cfg.H))
    return got, ref


def _compare(got, ref):
    plain = {"y", "dx"}
    for name, r in ref.items():
        g = got[name]
        assert np.all(np.isfinite(g)), name
        err = float(np.max(np.abs(g - r)))
        tol = TOL if name in plain else TOL * max(1.0, float(np.sqrt(np.mean(r ** 2))))
        print(f"  {name}: max abs err {err:.3e} (tol {tol:.3e}, rms(ref) "
              f"{float(np.sqrt(np.mean(r ** 2))):.3e})", flush=True)
        assert err <= tol, f"{name}: max abs err {err:.3e} > {tol:.3e}"


def test_sublayer_small():
    cfg = workloads.SublayerConfig("small", B=2, T=77, C=128, H=2, n_layer=12, dtype="bf16")
    got, ref = _run(cfg, cfg.B)
    _compare(got, ref)


def test_sublayer_full_config():
    cfg = workloads.SUBLAYER_CONFIG
    got, ref = _run(cfg, cfg.B)
    _compare(got, ref)
