"""The attention step and the decode step captured in HIP graphs (through
torch.cuda.CUDAGraph, which captures the launches the C ABI enqueues on the
current stream) and replayed.  Every replay is compared with the eager result,
bit for bit (the kernels are deterministic), with eager work and
synchronisations between the replays.  The kernels record no memset and
allocate nothing, so they are capturable.  The cases cover the plain and the
strided entry points (with a window and dropout, and the two-launch backward at
D = 128), the entry points with stored dropout keep bits, and both decode
paths."""
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,H,T,D,window,p,keep_bits", [
    (2, 3, 300, 64, 0, 0.0, False),     # attn_fwd / attn_bwd (one backward launch)
    (2, 2, 300, 128, 100, 0.1, False),  # strided entry points: window, dropout, two backward launches
    (1, 3, 200, 64, 70, 0.2, False),    # strided, window and dropout at D = 64
    (2, 3, 300, 64, 0, 0.1, True),      # dropout with stored keep bits
    (1, 2, 260, 128, 90, 0.2, True),    # stored keep bits, window, two backward launches
])
def test_attention_step_graph_replays_match_eager(B, H, T, D, window, p, keep_bits):
    """With stored keep bits the keep buffer starts zeroed for the eager step and
    is set to all ones (every weight kept) before each replay, so a word of a
    visible pair that the replayed forward did not rewrite would change the
    backward's outputs."""
    import causal_head_self_amd as cat
    _note(f"[graph] attention fwd+bwd B={B} H={H} T={T} D={D} window={window} p={p} "
          f"keep_bits={keep_bits}")
    dev = torch.device("cuda")
    q, k, v, dO = (t.to(dev) for t in workloads.attention_inputs(B, H, T, D, "bf16", 501))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    keep = (torch.zeros(cat.dropout_keep_bytes(B, H, T) // 4, dtype=torch.int32, device=dev)
            if keep_bits else None)

    def step():
        if keep_bits:
            cat.attn_fwd_strided_keep(q, k, v, o, lse, keep, window=window, dropout_p=p, seed=99)
            cat.attn_bwd_strided_keep(q, k, v, o, lse, dO, dq, dk, dv, delta, keep,
                                      window=window, dropout_p=p)
        elif window == 0 and p == 0.0:
            cat.attn_fwd(q, k, v, o, lse)
            cat.attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta)
        else:
            cat.attn_fwd_strided(q, k, v, o, lse, window=window, dropout_p=p, seed=99)
            cat.attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, window=window,
                                 dropout_p=p, seed=99)

    step()
    torch.cuda.synchronize()
    outs = (o, lse, dq, dk, dv, delta)
    names = ("o", "lse", "dq", "dk", "dv", "delta")
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the stream before capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv, delta):
            t.fill_(float("nan"))  # eager work between replays
        if keep_bits:
            keep.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, r in zip(names, outs, ref):
            assert torch.equal(a, r), f"replay {rep}: {name}"


@pytest.mark.parametrize("B,H,T_max,D,lens,step", [
    (4, 6, 700, 64, [700, 1, 350, 64], [0, 1, 1, 1]),   # one launch
    (2, 2, 1500, 64, [1500, 700], [0, 1]),              # two launches (split-K and merge)
])
def test_decode_graph_replays_match_eager(B, H, T_max, D, lens, step):
    import causal_head_self_amd as cat
    _note(f"[graph] decode B={B} H={H} T_max={T_max} D={D} lens={lens}")
    dev = torch.device("cuda")
    q, kc, vc = (t.to(dev) for t in workloads.decode_inputs(B, H, T_max, D, seed=777))
    lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(cat.decode_workspace_bytes(B, H, T_max, D), dtype=torch.uint8, device=dev)
    cat.attn_decode(q, kc, vc, lens, o, lse, ws)
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cat.attn_decode(q, kc, vc, lens, o, lse, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cat.attn_decode(q, kc, vc, lens, o, lse, ws)
    for rep in range(3):
        o.fill_(0)
        lse.fill_(0)
        ws.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
    # the lengths are read on the device at run time: a replay after they change
    # computes the new step (the next token of each sequence)
    lens.add_(torch.tensor(step, dtype=torch.int32, device=dev))
    cat.attn_decode(q, kc, vc, lens, ref_o, ref_l, ws)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


def test_sublayer_training_step_graph_replays_match_eager():
    """The pre-norm sublayer's forward + backward (LayerNorm, the c_attn and
    c_proj GEMMs, the attention kernels on strided views, the residual, every
    parameter gradient) captured as one graph, as the benchmark times it.  Each
    replay must give the eager step's gradients bit for bit; the gradient
    buffers are filled with NaN and eager GEMM work runs between replays."""
    from causal_head_self_amd.sublayer import attention_sublayer
    _note("[graph] sublayer fwd+bwd B=2 T=256 C=768 H=12")
    cfg = workloads.SUBLAYER_CONFIG
    inp = workloads.sublayer_inputs(cfg, B=2)
    names = ["x", "g", "bl", "Wa", "ba", "Wp", "bp"]
    T = 256
    inp = {n: (t[:, :T].contiguous() if n in ("x", "dy") else t) for n, t in inp.items()}
    dy = inp["dy"].cuda()

    def leaves():
        return {n: inp[n].cuda().requires_grad_(True) for n in names}

    def run(d):
        for n in names:
            d[n].grad = None
        attention_sublayer(d["x"], d["g"], d["bl"], d["Wa"], d["ba"], d["Wp"], d["bp"],
                           cfg.H).backward(dy)

    eager = leaves()
    run(eager)
    torch.cuda.synchronize()
    ref = {n: eager[n].grad.clone() for n in names}

    d = leaves()
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for _ in range(3):
            run(d)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    for n in names:
        d[n].grad = None
    with torch.cuda.graph(graph):
        attention_sublayer(d["x"], d["g"], d["bl"], d["Wa"], d["ba"], d["Wp"], d["bp"],
                           cfg.H).backward(dy)
    torch.cuda.synchronize()
    grads = {n: d[n].grad for n in names}
    junk = torch.randn(1024, 1024, device="cuda")
    for rep in range(4):
        for n in names:
            grads[n].fill_(float("nan"))
        junk = junk @ junk.T * 1e-3
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(grads[n], ref[n]), f"replay {rep}: grad of {n}"
