"""Helpers for the GPU parity tests: device checks and oracle-side inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle

DEV = "cuda:0"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_58_amd as kda
    kda.lib()  # raises if libkda.so is missing: there is no fallback


def say(*a):
    """Flush a line naming the case before a GPU step (so a lost box still says which)."""
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_gate_f32(dr, heads=None):
    """g, beta from the fp64 oracle gate, rounded to fp32 (torch CPU tensors)."""
    idx = slice(None) if heads is None else heads
    x = dr.x[:, idx].cpu()
    b = dr.b[:, idx].cpu()
    g, beta = oracle.gate(x, b, dr.A_log[idx].cpu(), dr.dt_bias[idx].cpu())
    return torch.from_numpy(g).float(), torch.from_numpy(beta).float()


def oracle_gate_f64(dr, heads):
    x = dr.x[:, heads].cpu()
    b = dr.b[:, heads].cpu()
    return oracle.gate(x, b, dr.A_log[heads].cpu(), dr.dt_bias[heads].cpu())


def sample_heads(H, n, seed):
    r = np.random.default_rng(seed)
    return sorted(r.choice(H, size=min(n, H), replace=False).tolist())
