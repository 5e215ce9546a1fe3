"""Seeded synthetic inputs for the MoE-layer hot path.

This module only draws inputs; it holds none of the layer's arithmetic.  The
GPU path and the CPU oracle both take their inputs from here, as plain numpy
arrays (float32 logits, bfloat16 values as uint16 bit patterns).

Workloads (sizes and distributions as stated for each):
  tiny     T=64,    H=256,  E=8,   top-2, I=128
  balanced T=512,   H=2048, E=64,  top-8, I=1024  (the shape of the MoonEP
           page's larger validation run and of OLMoE's layer)
  skewed   as balanced, +ln 8 on 8 randomly chosen experts' logits
  deepseek T=4096,  H=7168, E=256, top-8, I=2048, one shared expert
           (I=2048), FP8 combine-row fake-quant with a calibrated constant
           per-tensor scale
  prefill  T=16384 of which 10 % padding rows, H=4096, E=128, top-8,
           I=1536, FP8 dispatch fake-quant in 1x128 blocks, power-of-two
           segment buckets
Hidden states ~ N(0,1), expert weights ~ N(0,1)*0.02, router logits
~ N(0,1), all rounded to bfloat16 (logits stay float32).

Every stream has its own torch CPU generator, seeded
``1000*(config_index+1) + stream``: 0 logits, 1 hidden, 2 hot experts or
padding rows, 15 the shared expert, 16+2e / 17+2e expert e's w13 / w2.  One
expert's weights can therefore be regenerated on its own.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    index: int           # seed namespace
    T: int
    H: int
    E: int
    K: int
    I: int
    shared_I: int = 0            # 0: no shared expert
    hot_experts: int = 0         # experts whose logits get +ln(8)
    pad_rows: int = 0            # padding tokens (topk_idx = -1 in all slots)
    dispatch_block: int = 0      # 0: no dispatch fake-quant
    combine_qdq: bool = False    # per-tensor FP8 fake-quant of combine rows
    pad_pow2: bool = False       # power-of-two segment buckets

    @property
    def T_valid(self) -> int:
        return self.T - self.pad_rows

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": MoEConfig("tiny", 0, T=64, H=256, E=8, K=2, I=128),
    "balanced": MoEConfig("balanced", 1, T=512, H=2048, E=64, K=8, I=1024),
    "skewed": MoEConfig("skewed", 2, T=512, H=2048, E=64, K=8, I=1024, hot_experts=8),
    "deepseek": MoEConfig("deepseek", 3, T=4096, H=7168, E=256, K=8, I=2048,
                          shared_I=2048, combine_qdq=True),
    "prefill": MoEConfig("prefill", 4, T=16384, H=4096, E=128, K=8, I=1536,
                         pad_rows=1638, dispatch_block=128, pad_pow2=True),
}


def _gen(cfg: MoEConfig, stream: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(1000 * (cfg.index + 1) + stream)


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    """torch float32 -> bfloat16 (torch's cast) -> uint16 bit patterns."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def logits(cfg: MoEConfig) -> np.ndarray:
    """Router logits, float32 [T, E]."""
    x = torch.randn(cfg.T, cfg.E, generator=_gen(cfg, 0), dtype=torch.float32)
    if cfg.hot_experts:
        hot = torch.randperm(cfg.E, generator=_gen(cfg, 2))[: cfg.hot_experts]
        x[:, hot] += torch.tensor(math.log(8.0), dtype=torch.float32)
    return x.numpy().copy()


def hot_experts(cfg: MoEConfig) -> np.ndarray:
    if not cfg.hot_experts:
        return np.zeros(0, dtype=np.int64)
    return torch.randperm(cfg.E, generator=_gen(cfg, 2))[: cfg.hot_experts].numpy()


def row_valid(cfg: MoEConfig):
    """uint8 [T] (1 = real token, 0 = padding), or None with no padding."""
    if not cfg.pad_rows:
        return None
    v = np.ones(cfg.T, dtype=np.uint8)
    pad = torch.randperm(cfg.T, generator=_gen(cfg, 2))[: cfg.pad_rows].numpy()
    v[pad] = 0
    return v


def hidden(cfg: MoEConfig) -> np.ndarray:
    """Hidden states, bfloat16 bits uint16 [T, H]."""
    return _bf16_bits(torch.randn(cfg.T, cfg.H, generator=_gen(cfg, 1), dtype=torch.float32))


def expert_weights(cfg: MoEConfig, e: int):
    """Expert ``e``'s ``(w13 [2I, H], w2 [H, I])`` as bfloat16 bits."""
    w13 = torch.randn(2 * cfg.I, cfg.H, generator=_gen(cfg, 16 + 2 * e), dtype=torch.float32)
    w2 = torch.randn(cfg.H, cfg.I, generator=_gen(cfg, 17 + 2 * e), dtype=torch.float32)
    return _bf16_bits(w13 * 0.02), _bf16_bits(w2 * 0.02)


def shared_weights(cfg: MoEConfig):
    """The shared expert's ``(w13 [2Is, H], w2 [H, Is])``, or None."""
    if not cfg.shared_I:
        return None
    g = _gen(cfg, 15)
    w13 = torch.randn(2 * cfg.shared_I, cfg.H, generator=g, dtype=torch.float32)
    w2 = torch.randn(cfg.H, cfg.shared_I, generator=g, dtype=torch.float32)
    return _bf16_bits(w13 * 0.02), _bf16_bits(w2 * 0.02)


def for_each_expert(cfg: MoEConfig, fn, experts=None, threads: int = 8):
    """Call ``fn(e, w13, w2)`` for each expert, generating in a thread pool.

    Generation runs ahead of ``fn`` by at most ``threads`` experts so that
    host memory stays bounded even for the 22 GB deepseek weights.
    """
    experts = list(range(cfg.E)) if experts is None else list(experts)
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for i in range(0, len(experts), threads):
            chunk = experts[i:i + threads]
            futs = [pool.submit(expert_weights, cfg, e) for e in chunk]
            for e, f in zip(chunk, futs):
                w13, w2 = f.result()
                fn(e, w13, w2)
