"""Helpers for the GPU parity tests: numpy <-> device tensors, seeded inputs.

bfloat16 data travels as uint16 bit patterns on the host and as
torch.bfloat16 on the device (same bits).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def stacked_weights(cfg: workloads.MoEConfig, experts=None):
    """All experts' weights on the device as [E, 2I, H] and [E, H, I] bf16,
    plus a host dict expert -> (w13, w2) bit arrays for the oracle."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    w13 = torch.empty(len(experts), 2 * cfg.I, cfg.H, dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty(len(experts), cfg.H, cfg.I, dtype=torch.bfloat16, device="cuda")
    host_w = {}
    pos = {e: i for i, e in enumerate(experts)}

    def put(e, a, b):
        w13[pos[e]] = dev_bf16(a)
        w2[pos[e]] = dev_bf16(b)
        host_w[e] = (a, b)

    workloads.for_each_expert(cfg, put, experts)
    return w13, w2, host_w


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))
