"""Seeded synthetic inputs shaped like the pages' workloads.

Random numbers only -- nothing of the method's arithmetic lives here.  The
same tensor is handed to the HIP path and to the CPU oracle by the tests and
the benchmark.  Each recipe stands in for KV activations of real models
(Llama-3.1-8B-shaped heads: 8 KV heads x head_dim 128, 32 query heads), which
need trained weights and are not available.

Recipes (d = head dimension):
  tiny     n x d float32 N(0,1), 4 fixed outlier channels (0, 17, 64, 127) x 20
  llama    [heads][seq][d]: N(0,1) * exp(N(0,1)) per-channel scale (one per head
           and channel), 2% of channels per head (round(0.02 d) = 3 at d = 128)
           chosen without replacement and scaled x 20; bfloat16
  sweep    n x d float32: Gaussian direction normalised, times exp(0.5 N(0,1))
  highdim  n x d float32 N(0,1), 1% of channels (round(0.01 d)) x 10
  queries  float32 N(0,1)
"""
from __future__ import annotations

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def tiny_keys(n: int = 4096, d: int = 128, seed: int = 1, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn((n, d), generator=g, device=device, dtype=torch.float32)
    for ch in (0, 17, 64, 127):
        if ch < d:
            x[:, ch] *= 20.0
    return x


def llama_keys(heads: int = 8, seq: int = 32768, d: int = 128, seed: int = 1, device="cpu",
               dtype=torch.bfloat16, batch: int = 1) -> torch.Tensor:
    """[batch * heads * seq, d], vector (b * heads + h) * seq + pos."""
    g = _gen(seed, device)
    scale = torch.exp(torch.randn((batch, heads, 1, d), generator=g, device=device))
    n_out = max(1, round(0.02 * d))
    for b in range(batch):
        for h in range(heads):
            ch = torch.randperm(d, generator=g, device=device)[:n_out]
            scale[b, h, 0, ch] *= 20.0
    out = torch.empty((batch, heads, seq, d), dtype=dtype, device=device)
    for b in range(batch):
        for h in range(heads):
            out[b, h] = (torch.randn((seq, d), generator=g, device=device) * scale[b, h]).to(dtype)
    return out.reshape(batch * heads * seq, d)


def sweep_keys(n: int = 65536, d: int = 128, seed: int = 1, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn((n, d), generator=g, device=device)
    x = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
    return x * torch.exp(0.5 * torch.randn((n, 1), generator=g, device=device))


def highdim_keys(n: int, d: int = 1024, seed: int = 1, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn((n, d), generator=g, device=device)
    ch = torch.randperm(d, generator=_gen(seed + 1000, "cpu"))[: max(1, round(0.01 * d))].to(device)
    x[:, ch] *= 10.0
    return x


def queries(n: int, d: int = 128, seed: int = 5, device="cpu") -> torch.Tensor:
    return torch.randn((n, d), generator=_gen(seed, device), device=device, dtype=torch.float32)
