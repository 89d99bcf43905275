"""Seeded synthetic inputs shaped like the HyperQuant workloads.

Synthetic stand-ins for the pages' evaluation (Llama-3.1-8B-Instruct weights
and KV cache, a 70B-class MLP weight), which are not available here.  Every
generator is seeded and deterministic for a given device; nothing here
performs any step of the codec.  Shapes and distributions:

  c1  fp32 [4096, 128] weight, N(0, 0.02^2), 1% of entries x20 (seeded mask)
  c2  bf16 [4096, 4096] weight, per-row sigma ~ LogUniform(0.005, 0.05) times
      Student-t(4) entries (t = Z / sqrt(chi2_4 / 4))
  c3  bf16 K and V [8, 8, 32768, 128], N(0, 1), 4 seeded channels per KV head
      scaled x50 (K and V each), plus 4096 fp32 queries N(0, I)
  c4  bf16 [8192, 28672] weight, N(0, 0.015^2), 0.1% of entries x30
  c5  bf16 K and V [1, 8, 131072, 128], N(0, 1), 2% of K entries x100, plus
      32 fp32 query heads N(0, I) (4 per KV head)

``scale`` shrinks the leading dimension (rows, batch or sequence) for tests.
"""
from __future__ import annotations

import math

import torch

PLAN_SEED = 0x5EED0001
DATA_SEEDS = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5": 1005}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def c1(device="cpu", rows: int = 4096, seed: int = DATA_SEEDS["c1"]) -> torch.Tensor:
    g = _gen(device, seed)
    x = torch.randn(rows, 128, generator=g, device=device) * 0.02
    mask = torch.rand(rows, 128, generator=g, device=device) < 0.01
    return torch.where(mask, x * 20.0, x).contiguous()


def c1_sigma_eff() -> float:
    """RMS of the c1 distribution: 0.02 * sqrt(0.99 + 0.01 * 400)."""
    return 0.02 * math.sqrt(0.99 + 0.01 * 400.0)


def c2(device="cpu", rows: int = 4096, cols: int = 4096, seed: int = DATA_SEEDS["c2"]) -> torch.Tensor:
    g = _gen(device, seed)
    lo, hi = math.log(0.005), math.log(0.05)
    sigma = torch.exp(lo + (hi - lo) * torch.rand(rows, 1, generator=g, device=device))
    z = torch.randn(rows, cols, generator=g, device=device)
    chi2 = torch.zeros(rows, cols, device=device)
    for _ in range(4):
        chi2 += torch.randn(rows, cols, generator=g, device=device) ** 2
    t = z / torch.sqrt(chi2 / 4.0)
    return (sigma * t).to(torch.bfloat16).contiguous()


def c3(device="cpu", batch: int = 8, heads: int = 8, seq: int = 32768, n_queries: int = 4096,
       seed: int = DATA_SEEDS["c3"]):
    g = _gen(device, seed)
    out = []
    for _ in range(2):  # K then V, each with its own outlier channels
        x = torch.randn(batch, heads, seq, 128, generator=g, device=device)
        ch = torch.stack([torch.randperm(128, generator=g, device=device)[:4] for _ in range(heads)])
        scale = torch.ones(heads, 128, device=device)
        scale.scatter_(1, ch, 50.0)
        x *= scale.view(1, heads, 1, 128)
        out.append(x.to(torch.bfloat16).contiguous())
        del x
    q = torch.randn(n_queries, 128, generator=g, device=device)
    return out[0], out[1], q


def c4(device="cpu", rows: int = 8192, cols: int = 28672, seed: int = DATA_SEEDS["c4"]) -> torch.Tensor:
    g = _gen(device, seed)
    x = torch.randn(rows, cols, generator=g, device=device) * 0.015
    mask = torch.rand(rows, cols, generator=g, device=device) < 0.001
    x = torch.where(mask, x * 30.0, x)
    return x.to(torch.bfloat16).contiguous()


def c5(device="cpu", heads: int = 8, seq: int = 131072, q_per_head: int = 4, seed: int = DATA_SEEDS["c5"]):
    g = _gen(device, seed)
    k = torch.randn(1, heads, seq, 128, generator=g, device=device)
    mask = torch.rand(1, heads, seq, 128, generator=g, device=device) < 0.02
    k = torch.where(mask, k * 100.0, k).to(torch.bfloat16).contiguous()
    v = torch.randn(1, heads, seq, 128, generator=g, device=device).to(torch.bfloat16).contiguous()
    q = torch.randn(heads * q_per_head, 128, generator=g, device=device)
    return k, v, q
