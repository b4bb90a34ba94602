#!/usr/bin/env python3
"""Benchmark: causal multi-head self-attention forward + backward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
attn_fwd (tiled forward, lse out) followed by attn_bwd (Delta, dQ, dK/dV in
one launch), all through the C ABI of libcausal_attn.so, inputs resident in
HBM.

Default workload: GPT-2-small attention (B=8, H=12, T=1024, D=64, bf16 storage,
fp32 accumulation; q, k, v, dO iid N(0, 1), seeds 42+idx).  Metric: causal
fwd+bwd TFLOP/s with work = 7 * B * H * T^2 * D (forward 2 GEMMs and backward
5 GEMMs over the causal half), also as a fraction of the bf16 dense MFMA peak.

Prints ONE JSON line.  Extra keys: pct_of_peak, fwd_tflops, per-kernel times
(each kernel timed on its own, launches back to back), the roofline of the
dominant kernel, the CPU-oracle baseline (every host core this process may
use, forward alone and forward + backward) and, for the default workload,
"configs": every configuration of the contract timed in the same run (the tiny
fp32 one, GPT-2 small, the ~400M shape, the long context and the whole
pre-norm sublayer), forward and forward + backward, with the oracle's seconds
beside each.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s at GPT-2-small shape; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/CU/clk
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")
# the sources each family of kernels is built from (a profile summary is valid
# only for the source it was taken on)
KERNEL_SOURCES = {
    "attention": ["causal_head_self_amd/csrc/attn_bf16.hip",
                  "causal_head_self_amd/csrc/attn_bf16_d64.hip",
                  "causal_head_self_amd/csrc/attn_bwd_plain.hip",
                  "causal_head_self_amd/csrc/attn_device.h",
                  "causal_head_self_amd/build.py"],  # per-file compiler flags
    "decode": ["causal_head_self_amd/csrc/attn_decode.hip",
               "causal_head_self_amd/csrc/attn_device.h"],
    "rope": ["causal_head_self_amd/csrc/attn_rope.hip",
             "causal_head_self_amd/csrc/attn_device.h"],
    "norm": ["causal_head_self_amd/csrc/attn_norm.hip",
             "causal_head_self_amd/csrc/attn_device.h",
             "causal_head_self_amd/sublayer.py"],
}


def kernel_source_sha(family: str = "attention") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(T: int, window: int = 0) -> float:
    """(query, key) pairs that take part, by the causal convention: T^2 / 2
    for the causal mask (the diagonal not counted separately), T*W - W^2/2
    for a sliding window of W < T keys (the same formula at W = T)."""
    if window <= 0 or window >= T:
        return T * T / 2.0
    return T * window - window * window / 2.0


def kernel_work(cfg, window: int = 0):
    """Algorithmic work per launch, per kernel (causal-adjusted).  One GEMM
    over the causal half of one head is T^2 * D flops (2 D flops per visible
    pair).  The forward credits 2 GEMMs (S, PV); the backward 5: its dK/dV
    work is credited with S, dP, dV and dK, its dQ work with the dQ product
    (their recomputed S and dP are not credited again).  Delta (a row sum of
    dO * o) is not credited."""
    B, H, T, D = cfg.B, cfg.H, cfg.T, cfg.D
    g = float(B * H * D) * 2.0 * visible_pairs(T, window)
    return {
        "fwd": {"flops": 2 * g},
        "bwd": {"flops": 5 * g},
    }


MIN_WARMUP_SECONDS = 0.25


def warm_up(body, n: int) -> None:
    """n untimed calls of body, then more in groups of 10 until at least
    MIN_WARMUP_SECONDS of wall time has passed.  The GPU's clock follows its
    load: right after host-side work (the oracle timings) a warm-up of a few
    milliseconds has left a whole timed region several times slower than the
    same steps a moment later."""
    import torch
    t_end = time.perf_counter() + MIN_WARMUP_SECONDS
    for _ in range(n):
        body()
    torch.cuda.synchronize()
    while time.perf_counter() < t_end:
        for _ in range(10):
            body()
        torch.cuda.synchronize()


def read_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_src_sha") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info() -> dict:
    """The host the oracle runs on: CPU model, the cores this process may use,
    the machine's logical CPUs and OMP_NUM_THREADS as set."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "affinity_cores": affinity, "os_cpu_count": os.cpu_count(),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def oracle_attention_seconds(cfg, inputs, threads: int, window: int = 0):
    """The fp64 oracle, as it stands: (forward seconds, backward seconds) over
    the given inputs, wall clock."""
    import oracle
    q, k, v, dO = inputs
    s = oracle.widen_scale(cfg.scale)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, s, window=window, nthreads=threads)
    t1 = time.perf_counter()
    oracle.attn_bwd(q, k, v, dO, s, window=window, nthreads=threads)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def cpu_baseline(cfg, inputs, window: int = 0):
    """The fp64 oracle, as it stands, on every host core this process may use:
    the forward alone and then the backward, over all heads of the workload."""
    info = host_info()
    threads = info["affinity_cores"]
    tf, tb = oracle_attention_seconds(cfg, inputs, threads, window)
    work_f = 2.0 * cfg.B * cfg.H * cfg.D * 2.0 * visible_pairs(cfg.T, window)
    work = 3.5 * work_f
    return {
        "value": round(work / (tf + tb) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"one fp64 forward then backward pass over all {cfg.B * cfg.H} heads of the "
                   f"same workload (B={cfg.B}, H={cfg.H}, T={cfg.T}, D={cfg.D}); "
                   f"{tf:.2f} s + {tb:.2f} s wall on {threads} threads"),
        "seconds": round(tf + tb, 3),
        "fwd_seconds": round(tf, 3),
        "fwd_value": round(work_f / tf / 1e12, 6),
        "host": info,
    }


def sublayer_measure(args, with_oracle: bool = True) -> dict:
    """The pre-norm attention sublayer around the GPT-2-small shape: LayerNorm,
    c_attn, causal attention on strided views of the c_attn output (the HIP
    kernels), c_proj, residual; forward and backward through torch autograd.
    The step is timed twice: eagerly (every launch enqueued from Python and the
    autograd engine) and as one HIP-graph replay of the captured forward +
    backward (the same kernels, without the host's launch gaps between them);
    the graph replay is the reported value.  Work per step: the c_attn and
    c_proj GEMMs (2*N*C*3C + 2*N*C*C forward, 3x that forward plus backward)
    plus the attention's 7*B*H*T^2*D (2*B*H*T^2*D forward).  The attention
    share is the time of attn_fwd + attn_bwd alone at the same shape over the
    step time.  The oracle baseline is one of the eight sequences (fp64
    sublayer forward and backward), scaled to the whole batch."""
    import torch
    import causal_head_self_amd as cat
    from causal_head_self_amd.sublayer import attention_sublayer
    import workloads

    cfg = workloads.SUBLAYER_CONFIG
    inp = workloads.sublayer_inputs(cfg)
    names = ["x", "g", "bl", "Wa", "ba", "Wp", "bp"]
    dev = {n: inp[n].cuda().requires_grad_(True) for n in names}
    dy = inp["dy"].cuda()
    stream = torch.cuda.current_stream()

    def forward():
        return attention_sublayer(dev["x"], dev["g"], dev["bl"], dev["Wa"], dev["ba"], dev["Wp"],
                                  dev["bp"], cfg.H)

    def step():
        for n in names:
            dev[n].grad = None
        forward().backward(dy)

    def fwd_only():
        with torch.no_grad():
            forward()

    def timed(body, n):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(n):
            body()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    warm_up(step, args.warmup)
    eager_ms = timed(step, args.steps)
    fwd_ms = timed(fwd_only, args.steps)

    # The same step captured in a HIP graph (torch.cuda.CUDAGraph records the
    # launches the C ABI and the torch ops enqueue on the capturing stream).
    # Fresh leaves, warmed up on a side stream as capture requires, so that
    # their gradient-accumulation nodes belong to the capturing stream.
    gdev = {n: inp[n].cuda().requires_grad_(True) for n in names}

    def gstep():
        for n in names:
            gdev[n].grad = None
        attention_sublayer(gdev["x"], gdev["g"], gdev["bl"], gdev["Wa"], gdev["ba"],
                           gdev["Wp"], gdev["bp"], cfg.H).backward(dy)

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _ in range(3):
            gstep()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    for n in names:
        gdev[n].grad = None
    with torch.cuda.graph(graph):
        attention_sublayer(gdev["x"], gdev["g"], gdev["bl"], gdev["Wa"], gdev["ba"], gdev["Wp"],
                           gdev["bp"], cfg.H).backward(dy)
    warm_up(graph.replay, args.warmup)
    ms = timed(graph.replay, args.steps)

    # attention alone at the same shape (the gpt2s inputs)
    B, T, C, H = cfg.B, cfg.T, cfg.C, cfg.H
    D = C // H
    a = measure_attention(workloads.ATTN_CONFIGS["gpt2s"],
                          workloads.config_inputs(workloads.ATTN_CONFIGS["gpt2s"]),
                          args.steps, args.warmup)
    attn_ms = a["step_ms"]
    N = B * T
    gemm_fwd = 2.0 * N * C * 3 * C + 2.0 * N * C * C
    attn = 7.0 * B * H * T * T * D
    work = 3.0 * gemm_fwd + attn
    work_f = gemm_fwd + 2.0 * B * H * T * T * D
    out = {
        "value": round(work / (ms * 1e-3) / 1e12, 3), "ms_per_step": round(ms, 5),
        "step": "one HIP-graph replay of the captured forward + backward",
        "eager_value": round(work / (eager_ms * 1e-3) / 1e12, 3),
        "eager_ms_per_step": round(eager_ms, 5),
        "fwd_tflops": round(work_f / (fwd_ms * 1e-3) / 1e12, 3), "fwd_ms": round(fwd_ms, 5),
        "attention_ms": round(attn_ms, 5), "attention_share": round(attn_ms / ms, 4),
        "attention_tflops": round(a["tflops"], 3),
        "shape": {"B": B, "T": T, "C": C, "H": H, "dtype": cfg.dtype},
    }
    if with_oracle:
        import oracle
        one = workloads.sublayer_inputs(cfg, B=1)
        args_ = [one[n] for n in names]
        threads = host_info()["affinity_cores"]
        c0 = time.perf_counter()
        oracle.sublayer_fwd(*args_, n_head=H, nthreads=threads)
        c1 = time.perf_counter()
        oracle.sublayer_bwd(*args_, dy=one["dy"], n_head=H, nthreads=threads)
        c2 = time.perf_counter()
        out["oracle"] = {"fwd_seconds": round(c1 - c0, 4), "fwd_bwd_seconds": round(c2 - c0, 4),
                         "fwd_bwd_tflops": round(work / B / (c2 - c0) / 1e12, 6),
                         "threads": threads,
                         "sample": "one of the 8 sequences (B=1), TFLOP/s scaled per sequence"}
    return out


def sublayer_bench(args) -> int:
    import torch
    import causal_head_self_amd as cat
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cat.load_library()
    cfg = workloads.SUBLAYER_CONFIG
    m = sublayer_measure(args, with_oracle=not args.no_cpu_baseline)
    cpu = None
    if "oracle" in m:
        o = m.pop("oracle")
        cpu = {"value": o["fwd_bwd_tflops"], "unit": "TFLOP/s", "cores": o["threads"],
               "kind": "oracle", "sample": (f"fp64 sublayer forward and backward of one of the 8 "
                                            f"sequences: {o['fwd_bwd_seconds']} s wall"),
               "host": host_info()}
    out = {
        "metric": "causal attention sublayer fwd+bwd TFLOP/s (LN, c_attn, attention, c_proj, residual)",
        "value": m["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": m["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": (f"pre-norm attention sublayer, B={cfg.B} T={cfg.T} C={cfg.C} "
                                f"H={cfg.H} {cfg.dtype}; x, dy N(0,1), GPT-2 init weights, "
                                "seeds 42+idx"),
                   "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "single GPU"},
        "step": m["step"], "eager_value": m["eager_value"],
        "eager_ms_per_step": m["eager_ms_per_step"],
        "fwd_tflops": m["fwd_tflops"], "fwd_ms": m["fwd_ms"],
        "attention_ms": m["attention_ms"], "attention_share": m["attention_share"],
        "attention_tflops": m["attention_tflops"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def decode_bench(args) -> int:
    """One decode step against a full KV cache (nanochat, section 8: (B, T, H, D)
    cache, one new token per sequence): one attn_decode call, which is one
    launch (a workgroup per head) or, for few heads with long caches, a
    per-slice partial launch and a merge launch.  The op streams the visible
    cache once, so the metric is bytes per second against the HBM peak.
    Algorithmic bytes per call: the visible K and V rows
    (2 * sum_b len_b * H * D * 2), q and o (B * H * D * 2 each), lse (B * H * 4)
    and the lengths (B * 4); the workspace round trip of the two-launch path
    (B * H * slices * (D + 4) * 4 twice) is not counted."""
    import torch
    import causal_head_self_amd as cat
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cat.load_library()
    cfg = workloads.DECODE_CONFIGS[args.config]
    B, H, T_max, D = cfg.B, cfg.H, cfg.T_max, cfg.D
    dev = torch.device("cuda:0")
    host = workloads.decode_inputs(B, H, T_max, D)
    q, kc, vc = (t.to(dev) for t in host)
    lens = cfg.lens()
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(cat.decode_workspace_bytes(B, H, T_max, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(s=stream):
        cat.attn_decode(q, kc, vc, ln, o, lse, ws, cfg.scale, 0, s)

    warm_up(step, args.warmup)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps

    # the same steps captured once in a HIP graph and replayed (launch cost of
    # the two small kernels per step amortised by the graph)
    graph_ms = None
    if args.graph:
        per = 16
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()  # the capturing stream
            for _ in range(per):
                step(cap)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // per)
        t0.record(stream)
        for _ in range(reps):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        graph_ms = t0.elapsed_time(t1) / (reps * per)

    if args.copy_calibration_mib > 0:  # a plain device copy of known size (counter scaling)
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # the path attn_decode takes (the library's rule): one launch when every wave
    # of a workgroup has at most one 64-position slice, or when B*H reaches half
    # the compute units
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    one_launch = -(-T_max // 64) <= (8 if D == 128 else 16) or 2 * B * H >= n_cu
    kernel_name = ("attn_decode (one launch: decode_fused_kernel)" if one_launch else
                   "attn_decode (decode_partial_kernel + decode_combine_kernel launches)")
    kv_bytes = 2.0 * sum(lens) * H * D * 2
    alg_bytes = kv_bytes + 2.0 * B * H * D * 2 + B * H * 4 + B * 4
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        info = host_info()
        threads = info["affinity_cores"]
        c0 = time.perf_counter()
        oracle.attn_decode(host[0], host[1], host[2], lens, oracle.widen_scale(cfg.scale),
                           nthreads=threads)
        dt = time.perf_counter() - c0
        cpu = {"value": round(alg_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": (f"one fp64 decode step over the whole workload ({B * H} heads, "
                          f"{sum(lens)} cached positions); {dt:.3f} s wall on {threads} threads"),
               "seconds": round(dt, 4), "host": info}
    out = {
        "metric": "decode attention against a KV cache: algorithmic bytes per second",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: one token per sequence against a full "
                                f"[B={B}][T={T_max}][H={H}][D={D}] bf16 cache, fp32 arithmetic; "
                                "q, k, v iid N(0,1) seeds 42+idx"),
                   "B": B, "H": H, "T_max": T_max, "D": D, "cached_positions": lens,
                   "global_batch": B, "seq_len": T_max, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kernel_name,
                     "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic("decode", f"{cfg.name}_B{B}_H{H}_T{T_max}_D{D}",
                                             kernel_source_sha("decode")),
                     "algorithmic_bytes_per_call": alg_bytes},
        "cpu_baseline": cpu,
        "l2_flushed": False,
    }
    if graph_ms is not None:
        out["graph"] = {"ms_per_step": round(graph_ms, 6),
                        "GB_per_s": round(alg_bytes / (graph_ms * 1e-3) / 1e9, 2),
                        "note": "16 decode steps per captured graph, replayed"}
    print(json.dumps(out), flush=True)
    return 0


def rope_bench(args) -> int:
    """RoPE + QK norm on q and k of the gpt2s shape, read from the c_attn output
    layout [B, T, 3C] (as causal_attention_qkv does): the forward launch (read
    q, k; write the results) and the gradient launch (read q, k and the two
    incoming gradients; write dq, dk into the q and k thirds of dqkv).  Both are
    bound by HBM bandwidth; algorithmic bytes per step = 10 * B*H*T*D * 2."""
    import torch
    import causal_head_self_amd as cat
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cat.load_library()
    c = workloads.ATTN_CONFIGS["gpt2s"]
    B, H, T, D = c.B, c.H, c.T, c.D
    dev = torch.device("cuda:0")
    q, k, v, g = (t.to(dev) for t in workloads.config_inputs(c))
    qkv = torch.cat([t.permute(0, 2, 1, 3).reshape(B, T, H * D) for t in (q, k, v)], dim=-1)
    qv, kv, _ = cat.qkv_heads(qkv, H)
    qo, ko = torch.empty_like(q), torch.empty_like(q)
    dqkv = torch.empty_like(qkv)
    dq, dk, _ = cat.qkv_heads(dqkv, H)
    p = cat.Prologue()
    stream = torch.cuda.current_stream()
    names = ["rope_fwd", "rope_bwd"]

    # the incoming gradients of q and k: two distinct N(0, 1) tensors (v is not
    # otherwise used here), so that the gradient launch reads both from memory
    gq, gk = g, v
    launch = {"rope_fwd": lambda: cat.rope_qknorm_fwd(qv, kv, qo, ko, p, stream),
              "rope_bwd": lambda: cat.rope_qknorm_bwd(qv, kv, gq, gk, dq, dk, p, stream)}

    def run(n, which=names):
        for _ in range(n):
            for name in which:
                launch[name]()

    warm_up(lambda: run(1), args.warmup)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    run(args.steps)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    # per launch: each kind back to back on its own (events around single
    # launches of this length would also time the host's enqueue gaps)
    kern = {}
    for name in names:
        t0.record(stream)
        run(args.steps, [name])
        t1.record(stream)
        torch.cuda.synchronize()
        kern[name] = t0.elapsed_time(t1) / args.steps
    elem = B * H * T * D
    byt = {"rope_fwd": 4.0 * elem * 2, "rope_bwd": 6.0 * elem * 2}
    gbs = (byt["rope_fwd"] + byt["rope_bwd"]) / (ms * 1e-3) / 1e9
    dom = max(names, key=lambda n: kern[n])
    ach = byt[dom] / (kern[dom] * 1e-3) / 1e9
    if args.copy_calibration_mib > 0:  # a plain device copy of known size (counter scaling)
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    sha = kernel_source_sha("rope")

    # The whole attention step with the prologue, both ways: fused into the
    # attention kernels (the key pass, the forward turning the queries in
    # registers, the backward applying the prologue's gradient in registers),
    # and as separate passes around the strided attention.
    y = torch.empty((B, T, H * D), dtype=torch.bfloat16, device=dev)
    ov = y.view(B, T, H, D).permute(0, 2, 1, 3)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dqkv2 = torch.empty_like(qkv)
    dq2, dk2, dv2 = cat.qkv_heads(dqkv2, H)
    vv = cat.qkv_heads(qkv, H)[2]
    qr, kr, dqa, dka = (torch.empty_like(q) for _ in range(4))
    gO = g  # the incoming gradient of the attention output, as [B, H, T, D]

    def fused():
        cat.attn_fwd_strided_rope(qv, kv, vv, ov, lse, qr, kr, p, stream=stream)
        cat.attn_bwd_strided_rope(qv, kv, qr, kr, vv, ov, lse, gO, dq2, dk2, dv2, delta, p,
                                  stream=stream)

    def two_pass():
        cat.rope_qknorm_fwd(qv, kv, qr, kr, p, stream)
        cat.attn_fwd_strided(qr, kr, vv, ov, lse, stream=stream)
        cat.attn_bwd_strided(qr, kr, vv, ov, lse, gO, dqa, dka, dv2, delta, stream=stream)
        cat.rope_qknorm_bwd(qv, kv, dqa, dka, dq2, dk2, p, stream)

    e2e = {}
    for name, body in (("fused", fused), ("two_pass", two_pass)):
        warm_up(body, args.warmup)
        t0.record(stream)
        for _ in range(args.steps):
            body()
        t1.record(stream)
        torch.cuda.synchronize()
        e2e[name] = t0.elapsed_time(t1) / args.steps
    attn_flops = 7.0 * B * H * T * T * D
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle (one host thread) over the whole workload: forward and
        # gradient of q and k
        import oracle
        hq, hk, hgq, hgk = (t.cpu() for t in (q, k, gq, gk))
        c0 = time.perf_counter()
        oracle.rope_qknorm_fwd(hq, p.pos0, p.base, p.rope, p.qk_norm, p.q_gain, p.eps)
        oracle.rope_qknorm_fwd(hk, p.pos0, p.base, p.rope, p.qk_norm, p.k_gain, p.eps)
        oracle.rope_qknorm_bwd(hq, hgq, p.pos0, p.base, p.rope, p.qk_norm, p.q_gain, p.eps)
        oracle.rope_qknorm_bwd(hk, hgk, p.pos0, p.base, p.rope, p.qk_norm, p.k_gain, p.eps)
        dt = time.perf_counter() - c0
        cpu = {"value": round((byt["rope_fwd"] + byt["rope_bwd"]) / dt / 1e9, 4), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": (f"one fp64 forward and gradient over the whole workload ({B * H * T} "
                          f"q rows and as many k rows); {dt:.3f} s wall on one thread"),
               "seconds": round(dt, 4), "host": host_info()}
    out = {
        "metric": "RoPE + QK-norm prologue (forward + gradient): algorithmic bytes per second",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"rope_gpt2s: RoPE (base 1e4) + QK norm (gain 1.2 / 1.0) on q, k "
                                f"views of a [B={B}, T={T}, 3C={3 * H * D}] bf16 c_attn output, "
                                f"H={H} D={D}"),
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "kernel_ms": {n: round(v_, 5) for n, v_ in kern.items()},
        "attention_step_ms": {"fused": round(e2e["fused"], 5), "two_pass": round(e2e["two_pass"], 5),
                              "note": ("causal attention forward + backward with RoPE + QK norm "
                                       "on the gpt2s shape: the prologue fused into the kernels, "
                                       "or as separate passes")},
        "attention_step_tflops": {n: round(attn_flops / (v_ * 1e-3) / 1e12, 3)
                                  for n, v_ in e2e.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(dom, f"rope_gpt2s_B{B}_H{H}_T{T}_D{D}", sha),
                     "algorithmic_bytes_per_launch": byt[dom]},
        "cpu_baseline": cpu,
        "kernel_src_sha": sha,
        "l2_flushed": False,
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="gpt2s",
                    choices=["tiny", "gpt2s", "gpt400m", "long", "gpt2s_d128", "sublayer",
                             "decode_gpt2s", "decode_gpt2s_b64", "decode_long", "rope_gpt2s"])
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window W (bf16, D 64/128): query i sees keys i-W < j <= i")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="attention dropout probability (bf16, D 64/128; Philox seed 42)")
    ap.add_argument("--keep-bits", action="store_true",
                    help="with --dropout: the forward stores its keep bits and the backward "
                         "loads them (attn_*_strided_keep) instead of drawing them again")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-configs", action="store_true",
                    help="default workload: skip timing the other configurations in the same run")
    ap.add_argument("--graph", action="store_true",
                    help="decode configs: also time the steps replayed from a captured HIP graph")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(every (batch, head) pair is independent, so more GPUs would each run their "
              "own shard of the batch with no exchange).", file=sys.stderr)
        return 2

    if args.config == "sublayer":
        return sublayer_bench(args)
    if args.config.startswith("decode_"):
        return decode_bench(args)
    if args.config == "rope_gpt2s":
        return rope_bench(args)

    import torch
    import causal_head_self_amd as cat
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cat.load_library()  # raises if the HIP library is missing
    torch.manual_seed(42)
    cfg = workloads.ATTN_CONFIGS[args.config]
    W, P = args.window, args.dropout
    if W < 0 or not 0.0 <= P < 1.0 or ((W or P) and (cfg.dtype != "bf16" or cfg.D not in (64, 128))):
        print("bench.py: --window needs W >= 0, --dropout 0 <= p < 1, and either a bf16 "
              "workload with D 64 or 128", file=sys.stderr)
        return 2
    host_inputs = workloads.config_inputs(cfg)
    m = measure_attention(cfg, host_inputs, args.steps, args.warmup, W, P,
                          args.keep_bits and P > 0, args.copy_calibration_mib)
    B, H, T, D = cfg.B, cfg.H, cfg.T, cfg.D
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    work = kernel_work(cfg, W)
    kern_ms = m["kernel_ms"]
    dominant = max(kern_ms, key=lambda n: kern_ms[n])
    achieved = work[dominant]["flops"] / (kern_ms[dominant] * 1e-3) / 1e12
    sha = kernel_source_sha()
    workload_name = (f"{cfg.name}_B{B}_H{H}_T{T}_D{D}_{cfg.dtype}" + (f"_W{W}" if W else "")
                     + (f"_drop{P:g}" if P else ""))
    roofline = {
        "bound": "mfma",
        "kernel": dominant,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": read_traffic(dominant, workload_name, sha),
        "algorithmic_flops_per_launch": work[dominant]["flops"],
    }
    cpu = None
    if not args.no_cpu_baseline and not P:
        cpu = cpu_baseline(cfg, host_inputs, W)
    out = {
        "metric": METRIC,
        "value": round(m["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"causal MHA fwd+bwd, {cfg.name}: B={B} H={H} T={T} D={D} {cfg.dtype} "
                         "storage / fp32 accumulate, q,k,v,dO iid N(0,1) seeds 42+idx"
                         + (f", sliding window W={W}" if W else "")
                         + (f", attention dropout p={P:g} (Philox seed 42)" if P else "")
                         + (", keep bits stored by the forward" if m["keep_bits"] else "")),
            "B": B, "H": H, "T": T, "D": D, "window": W, "dropout": P,
            "keep_bits": m["keep_bits"], "global_batch": B,
            "seq_len": T,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * m["tflops"] / peak, 2),
        "fwd_tflops": round(m["fwd_tflops"], 3),
        "fwd_pct_of_peak": round(100.0 * m["fwd_tflops"] / peak, 2),
        # each kernel timed on its own, K launches back to back
        "kernel_ms": {n: round(v_, 5) for n, v_ in kern_ms.items()},
        "kernel_src_sha": sha,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "l2_flushed": False,
    }
    if args.config == "gpt2s" and not (W or P) and not args.no_all_configs:
        out["configs"] = all_configs(args, cat, workloads)
    print(json.dumps(out), flush=True)
    return 0


def measure_attention(cfg, host_inputs, steps, warmup, W=0, P=0.0, keep_bits=False,
                      copy_calibration_mib=0):
    """One workload on the GPU.  step_ms: K whole steps (forward + backward)
    between two events on the launch stream, nothing else in the region.
    kernel_ms: each call timed on its own, K launches back to back (the
    forward's outputs from one call feed every backward)."""
    import torch
    import causal_head_self_amd as cat
    dev = torch.device("cuda:0")
    q, k, v, dO = (t.to(dev) for t in host_inputs)
    B, H, T, D = cfg.B, cfg.H, cfg.T, cfg.D
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)
    scale = cfg.scale
    stream = torch.cuda.current_stream()
    strided = bool(W or P)
    keep = None
    if keep_bits:
        keep = torch.empty((cat.dropout_keep_bytes(B, H, T) // 4,), dtype=torch.int32, device=dev)

    def fwd():
        if keep is not None:
            cat.attn_fwd_strided_keep(q, k, v, o, lse, keep, scale, stream, window=W, dropout_p=P,
                                      seed=42)
        elif strided:
            cat.attn_fwd_strided(q, k, v, o, lse, scale, stream, window=W, dropout_p=P, seed=42)
        else:
            cat.attn_fwd(q, k, v, o, lse, scale, stream)

    def bwd():
        if keep is not None:
            cat.attn_bwd_strided_keep(q, k, v, o, lse, dO, dq, dk, dv, delta, keep, scale, stream,
                                      window=W, dropout_p=P)
        elif strided:
            cat.attn_bwd_strided(q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stream, window=W,
                                 dropout_p=P, seed=42)
        else:
            cat.attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stream)

    def timed(body, n):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(n):
            body()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    warm_up(lambda: (fwd(), bwd()), warmup)
    step_ms = timed(lambda: (fwd(), bwd()), steps)
    kern = {"fwd": timed(fwd, steps), "bwd": timed(bwd, steps)}
    if copy_calibration_mib > 0:  # a plain device copy of known size (counter scaling)
        n = copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    work = kernel_work(cfg, W)
    flops_f = work["fwd"]["flops"]
    flops_fb = flops_f + work["bwd"]["flops"]
    return {"step_ms": step_ms, "kernel_ms": kern, "tflops": flops_fb / (step_ms * 1e-3) / 1e12,
            "fwd_tflops": flops_f / (kern["fwd"] * 1e-3) / 1e12, "keep_bits": keep is not None}


def all_configs(args, cat, workloads) -> dict:
    """Every configuration of the contract in the same run: GPU forward and
    forward + backward TFLOP/s (K steps each), and the fp64 oracle's seconds
    beside them (all heads of each attention workload; one of the sublayer's
    eight sequences)."""
    threads = host_info()["affinity_cores"]
    res = {}
    for name in ("tiny", "gpt2s", "gpt400m", "long"):
        c = workloads.ATTN_CONFIGS[name]
        inputs = workloads.config_inputs(c)
        m = measure_attention(c, inputs, args.steps, args.warmup)
        peak = PEAK_BF16_TFLOPS if c.dtype == "bf16" else PEAK_F32_TFLOPS
        entry = {
            "shape": {"B": c.B, "H": c.H, "T": c.T, "D": c.D, "dtype": c.dtype},
            "fwd_bwd_tflops": round(m["tflops"], 3), "fwd_tflops": round(m["fwd_tflops"], 3),
            "pct_of_peak": round(100.0 * m["tflops"] / peak, 2), "peak_tflops": peak,
            "step_ms": round(m["step_ms"], 5), "kernel_ms": {n: round(x, 5) for n, x in
                                                            m["kernel_ms"].items()},
        }
        if not args.no_cpu_baseline:
            tf, tb = oracle_attention_seconds(c, inputs, threads)
            wf = 2.0 * c.B * c.H * c.D * 2.0 * visible_pairs(c.T)
            entry["oracle"] = {"fwd_seconds": round(tf, 4), "fwd_bwd_seconds": round(tf + tb, 4),
                               "fwd_bwd_tflops": round(3.5 * wf / (tf + tb) / 1e12, 6),
                               "threads": threads, "sample": "all heads"}
        res[name] = entry
    res["sublayer"] = sublayer_measure(args, with_oracle=not args.no_cpu_baseline)
    return res


if __name__ == "__main__":
    sys.exit(main())
