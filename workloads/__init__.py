"""Workload shapes and seeded synthetic inputs.

This module is shared by the oracle side and the GPU side, so it holds no
attention arithmetic: only shapes, seeds and random draws.

Shapes follow the pages' model configurations:
  * tiny      -- the CPU config of "Train Your Own LLM from Scratch" (section 3:
                 block_size 64, n_head 4, n_embd 128, so D = 32), fp32;
  * gpt2s     -- GPTConfig defaults of the same page (n_head 12, n_embd 768,
                 block_size 1024), bf16;
  * gpt400m   -- the ~400M config of the train-llm-from-scratch hub page
                 (n_embed 1024, n_head 16, context 1024), bf16;
  * long      -- the same head shape at a 4096-token context, bf16;
  * gpt2s_d128 -- the gpt2s width (768) and context in 6 heads of 128, bf16
                 (head dim 128 is not one of the pages' shapes);
  * sublayer  -- the GPT-2-small pre-norm attention sublayer (LayerNorm ->
                 c_attn -> causal MHA -> c_proj + residual), bf16;
  * decode_*  -- one decode step against a full KV cache in the (B, T, H, D)
                 layout (nanochat, section 8) at the gpt2s and long head
                 shapes, bf16.

Seeding follows the set_seed(42) convention of the CS336 tutorial (section
9.3): tensor number idx is drawn from its own generator seeded 42 + idx, as
float32 N(0, 1), multiplied by its standard deviation, then rounded to the
workload dtype (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

SEED = 42


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str  # "f32" | "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return torch_dtype(self.dtype)


@dataclass(frozen=True)
class SublayerConfig:
    name: str
    B: int
    T: int
    C: int
    H: int
    n_layer: int
    dtype: str

    @property
    def D(self) -> int:
        return self.C // self.H


ATTN_CONFIGS = {
    "tiny": AttnConfig("tiny", B=4, H=4, T=64, D=32, dtype="f32"),
    "gpt2s": AttnConfig("gpt2s", B=8, H=12, T=1024, D=64, dtype="bf16"),
    "gpt400m": AttnConfig("gpt400m", B=8, H=16, T=1024, D=64, dtype="bf16"),
    "long": AttnConfig("long", B=2, H=16, T=4096, D=64, dtype="bf16"),
    "gpt2s_d128": AttnConfig("gpt2s_d128", B=8, H=6, T=1024, D=128, dtype="bf16"),
}

@dataclass(frozen=True)
class DecodeConfig:
    """One decode step: B sequences, each adding one token to a [T_max] cache
    of H heads of width D; every sequence holds `fill` cached positions
    (T_max when fill is None)."""
    name: str
    B: int
    H: int
    T_max: int
    D: int
    fill: int | None = None

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def lens(self):
        return [self.T_max if self.fill is None else self.fill] * self.B


# decode steps at the pages' head shapes with a full cache: GPT-2-small
# (context 1024) at the training batch and at a serving batch of 64 sequences,
# and the long-context shape (4096)
DECODE_CONFIGS = {
    "decode_gpt2s": DecodeConfig("decode_gpt2s", B=8, H=12, T_max=1024, D=64),
    "decode_gpt2s_b64": DecodeConfig("decode_gpt2s_b64", B=64, H=12, T_max=1024, D=64),
    "decode_long": DecodeConfig("decode_long", B=2, H=16, T_max=4096, D=64),
}

SUBLAYER_CONFIG = SublayerConfig("sublayer", B=8, T=1024, C=768, H=12, n_layer=12, dtype="bf16")


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _draw(shape, idx: int, std: float, dtype, seed: int = SEED) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed + idx)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def attention_inputs(B: int, H: int, T: int, D: int, dtype="bf16", seed: int = SEED):
    """q, k, v, dO as CPU tensors [B, H, T, D], iid N(0, 1), seeds seed+0..3."""
    dt = torch_dtype(dtype) if isinstance(dtype, str) else dtype
    shape = (B, H, T, D)
    return tuple(_draw(shape, i, 1.0, dt, seed) for i in range(4))


def device_attention_inputs(B: int, H: int, T: int, D: int, device, seed: int = SEED):
    """q, k, v, dO as bf16 [B, H, T, D] tensors drawn on `device` (for shapes too
    large to draw on the host): the same recipe as attention_inputs (float32
    N(0, 1) from a generator seeded seed + idx, rounded to bf16), but from the
    device generator, so the values differ from the host draws of that shape."""
    out = []
    for idx in range(4):
        g = torch.Generator(device=device).manual_seed(seed + idx)
        x = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=device)
        for b in range(B):  # one batch at a time keeps the float32 temporary small
            x[b] = torch.randn((H, T, D), generator=g, dtype=torch.float32, device=device)
        out.append(x)
    return tuple(out)


def device_decode_inputs(B: int, H: int, T_max: int, D: int, device, seed: int = SEED):
    """q [B, H, D] and k_cache, v_cache [B, T_max, H, D] as bf16 tensors drawn on
    `device`: the decode_inputs recipe from the device generator."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn((B, H, D), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    out = [q]
    for idx in (1, 2):
        g = torch.Generator(device=device).manual_seed(seed + idx)
        x = torch.empty((B, T_max, H, D), dtype=torch.bfloat16, device=device)
        for b in range(B):
            x[b] = torch.randn((T_max, H, D), generator=g, dtype=torch.float32, device=device)
        out.append(x)
    return tuple(out)


def config_inputs(cfg: AttnConfig, seed: int = SEED):
    return attention_inputs(cfg.B, cfg.H, cfg.T, cfg.D, cfg.dtype, seed)


def decode_inputs(B: int, H: int, T_max: int, D: int, seed: int = SEED):
    """q [B, H, D] and k_cache, v_cache [B, T_max, H, D] as bf16 CPU tensors,
    iid N(0, 1), seeds seed+0..2 (the cache rows past a sequence's length are
    drawn too; they must not matter)."""
    dt = torch.bfloat16
    return (_draw((B, H, D), 0, 1.0, dt, seed), _draw((B, T_max, H, D), 1, 1.0, dt, seed),
            _draw((B, T_max, H, D), 2, 1.0, dt, seed))


def sublayer_inputs(cfg: SublayerConfig = SUBLAYER_CONFIG, seed: int = SEED, B: int | None = None):
    """x [B,T,C] N(0,1); W_attn [C,3C] N(0,0.02); W_proj [C,C] N(0, 0.02/sqrt(2 n_layer));
    dy [B,T,C] N(0,1); LayerNorm weight 1, bias 0; linear biases 0 (the pages'
    _init_weights).  Weights are drawn in fp32 and rounded once to the dtype.
    Seeds: 0 = x, 1 = W_attn, 2 = W_proj, 3 = dy."""
    dt = torch_dtype(cfg.dtype)
    B = cfg.B if B is None else B
    C = cfg.C
    x = _draw((B, cfg.T, C), 0, 1.0, dt, seed)
    Wa = _draw((C, 3 * C), 1, 0.02, dt, seed)
    Wp = _draw((C, C), 2, 0.02 / math.sqrt(2 * cfg.n_layer), dt, seed)
    dy = _draw((B, cfg.T, C), 3, 1.0, dt, seed)
    g = torch.ones(C, dtype=dt)
    bl = torch.zeros(C, dtype=dt)
    ba = torch.zeros(3 * C, dtype=dt)
    bp = torch.zeros(C, dtype=dt)
    return dict(x=x, g=g, bl=bl, Wa=Wa, ba=ba, Wp=Wp, bp=bp, dy=dy)


def causal_flops_fwd(B: int, H: int, T: int, D: int) -> float:
    """Causal-adjusted forward work: 2 GEMMs x 2*T*T*D x 1/2 per head."""
    return 2.0 * B * H * T * T * D


def causal_flops_fwd_bwd(B: int, H: int, T: int, D: int) -> float:
    """Forward plus backward (backward = 2.5 x forward, 5 GEMMs)."""
    return 7.0 * B * H * T * T * D
