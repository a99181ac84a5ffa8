"""Seeded input recipes for the KDA core workloads.

Distributions follow the Kimi-K3 artifact audit ("Kimi K3 第三轮：开放工件、权重元数据与
可复现实验审计", §5.1 KDA layer 1 parameter table): A_log has median about -0.15 and
range -0.75..2.47, dt_bias median about -4.6.  The five workload recipes draw
  A_log   ~ U(-0.75, 0.5)            per head            [H]
            (the per-channel variant: U(-0.75, 1.0) per (head, channel) [H, d])
  dt_bias ~ N(-4.6, 1.2)             per channel         [H, d]
  q, k    ~ N(0, 1), then L2-normalised over d per (token, head)
  v       ~ N(0, 1)
  x       ~ N(0, 1)   raw gate logits                    [T, H, d]
  b       ~ N(0, 1)   raw beta logits                    [T, H]
  S0      ~ N(0, 0.02**2) (standard deviation 0.02) where an initial state is used.

Draw order for one workload, from one torch.Generator seeded with `seed`:
A_log, dt_bias, then q, k, v, x, b, then the initial states.  Values drawn on a
CUDA generator differ from CPU draws; a test uses one device for one case.
q/k/v are rounded to bf16 (round-to-nearest-even, torch's cast) after the L2
normalisation when the workload asks for bf16; consumers upcast exactly.

Nothing here computes the gate or the recurrence.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

D = 128

# name, T (or per-sequence lengths), H, qkv dtype, initial state, seed
CONFIGS = {
    0: dict(name="kda-core-T256-H2-fp32", lengths=[256], H=2, dtype=torch.float32,
            init_state=False, seed=1000),
    1: dict(name="k3-layer-prefill-T4096-H96-bf16", lengths=[4096], H=96,
            dtype=torch.bfloat16, init_state=False, seed=1001),
    2: dict(name="varlen-8seq-T32768-H96-bf16", lengths="varlen8", H=96,
            dtype=torch.bfloat16, init_state=True, seed=1002),
    3: dict(name="long-prefill-T131072-H96-bf16", lengths=[131072], H=96,
            dtype=torch.bfloat16, init_state=False, seed=1003),
    4: dict(name="decode-N256-H96-64steps-bf16", N=256, H=96, steps=64,
            dtype=torch.bfloat16, seed=1004),
}


@dataclasses.dataclass
class KdaDraw:
    """One prefill workload: raw draws, packed varlen layout [T_tot, H, d]."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    x: torch.Tensor          # raw gate logits, fp32 [T, H, d]
    b: torch.Tensor          # raw beta logits, fp32 [T, H]
    A_log: torch.Tensor      # fp32 [H]
    dt_bias: torch.Tensor    # fp32 [H, d]
    cu_seqlens: torch.Tensor  # int32 [N+1], on CPU
    initial_state: Optional[torch.Tensor]  # fp32 [N, H, d, d] or None
    lengths: List[int]


@dataclasses.dataclass
class DecodeDraw:
    q: torch.Tensor          # [N, H, d]
    k: torch.Tensor
    v: torch.Tensor
    x: torch.Tensor          # fp32 [N, H, d]
    b: torch.Tensor          # fp32 [N, H]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(t: torch.Tensor) -> torch.Tensor:
    """L2-normalise over the last dimension (input recipe, not part of the core)."""
    n = torch.linalg.vector_norm(t, dim=-1, keepdim=True)
    return t / n.clamp_min(1e-30)


def varlen_lengths(seed: int, n: int = 8, total: int = 32768, lo: int = 512,
                   hi: int = 8192) -> List[int]:
    """Seeded rejection draw of n lengths in [lo, hi] summing to `total`.

    Draw n-1 lengths uniformly from the integers in [lo, hi]; the last one is
    total - sum; accept when it also lies in [lo, hi], else draw again.  Always
    drawn on the CPU so that the lengths do not depend on the device.
    """
    g = _gen(seed, "cpu")
    while True:
        first = torch.randint(lo, hi + 1, (n - 1,), generator=g).tolist()
        last = total - sum(first)
        if lo <= last <= hi:
            return first + [last]


def _params(g, H, device):
    A_log = torch.rand(H, generator=g, device=device, dtype=torch.float32) * 1.25 - 0.75
    dt_bias = torch.randn(H, D, generator=g, device=device, dtype=torch.float32) * 1.2 - 4.6
    return A_log, dt_bias


def _tokens(g, n_tok, H, dtype, device):
    shape = (n_tok, H, D)
    q = _unit_rows(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
    k = _unit_rows(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    b = torch.randn((n_tok, H), generator=g, device=device, dtype=torch.float32)
    if dtype != torch.float32:
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    return q, k, v, x, b


def draw_prefill(lengths: List[int], H: int, dtype=torch.float32, init_state: bool = False,
                 seed: int = 0, device="cpu", init_std: float = 0.02) -> KdaDraw:
    """Draw one packed varlen prefill workload with the recipe above."""
    g = _gen(seed, device)
    A_log, dt_bias = _params(g, H, device)
    T = int(sum(lengths))
    q, k, v, x, b = _tokens(g, T, H, dtype, device)
    S0 = None
    if init_state:
        S0 = torch.randn((len(lengths), H, D, D), generator=g, device=device,
                         dtype=torch.float32) * init_std
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return KdaDraw(q, k, v, x, b, A_log, dt_bias, cu, S0, list(lengths))


def draw_config(idx: int, device="cpu") -> KdaDraw:
    """The prefill workloads 0..3 at their full sizes."""
    c = CONFIGS[idx]
    if idx == 4:
        raise ValueError("workload 4 is decode: use draw_decode_params/draw_decode_step")
    lengths = varlen_lengths(c["seed"]) if c["lengths"] == "varlen8" else c["lengths"]
    return draw_prefill(lengths, c["H"], c["dtype"], c["init_state"], c["seed"], device)


def draw_decode_params(N: int, H: int, seed: int, device="cpu", init_std: float = 0.02):
    """A_log, dt_bias and the initial state [N, H, d, d] of a decode workload."""
    g = _gen(seed, device)
    A_log, dt_bias = _params(g, H, device)
    S0 = torch.randn((N, H, D, D), generator=g, device=device, dtype=torch.float32) * init_std
    return A_log, dt_bias, S0


def draw_decode_step(N: int, H: int, step: int, seed: int, dtype=torch.bfloat16,
                     device="cpu") -> DecodeDraw:
    """Fresh one-token inputs of decode step `step` (its own generator: seed*1000+1+step)."""
    g = _gen(seed * 1000 + 1 + step, device)
    q, k, v, x, b = _tokens(g, N, H, dtype, device)
    return DecodeDraw(q, k, v, x, b)


def draw_alog_per_channel(H: int, seed: int, device="cpu", lo: float = -0.75,
                          hi: float = 1.0) -> torch.Tensor:
    """A_log per (head, channel), [H, d] fp32 ~ U(lo, hi): the channel-wise
    variant of the gate (inside the audit's observed A_log range), from its own
    generator seeded with seed * 1000 + 999."""
    g = _gen(seed * 1000 + 999, device)
    return torch.rand(H, D, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def orthonormal_keys_pm_quarter(n: int, d: int = D) -> torch.Tensor:
    """n <= d orthonormal rows with entries in {0, +-1/4} (exact in bf16 and fp16).

    Rows are the rows of a 16x16 Sylvester-Hadamard matrix scaled by 1/4, placed
    in successive 16-channel blocks.
    """
    if n > d or d % 16:
        raise ValueError("need n <= d and d a multiple of 16")
    i = torch.arange(16)
    bits = (i[:, None] & i[None, :])
    pop = torch.zeros_like(bits)
    for s in range(4):
        pop += (bits >> s) & 1
    h16 = (1 - 2 * (pop % 2)).to(torch.float32) * 0.25
    out = torch.zeros(n, d)
    for r in range(n):
        blk, row = divmod(r, 16)
        out[r, blk * 16:(blk + 1) * 16] = h16[row]
    return out
