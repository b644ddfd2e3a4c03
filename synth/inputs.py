"""Seeded generators: random numbers and layout only (see package docstring)."""

import math

import numpy as np
import torch

# Chunked generation keeps host memory bounded for very large tensors.
_CHUNK = 1 << 24


ROLES = {"x": 0, "w": 1, "dy": 2, "a": 3, "b": 4}


def tensor_seed(seed, role):
    """Distinct generator seed per tensor role.  Two tensors drawn from the
    same seed are correlated (the same underlying stream), which would bias
    every product of them; each role therefore gets its own seed."""
    return int(seed) * 16 + ROLES[role]


def _generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, seed=0, device="cpu"):
    """N(0,1) drawn in float32 with a seeded generator, rounded to bf16."""
    g = _generator(seed, device)
    numel = math.prod(shape)
    out = torch.empty(numel, dtype=torch.bfloat16, device=device)
    for s in range(0, numel, _CHUNK):
        e = min(numel, s + _CHUNK)
        out[s:e] = torch.randn(e - s, generator=g, dtype=torch.float32,
                               device=device).to(torch.bfloat16)
    return out.view(*shape)


def linear_weight_bf16(n_out, k_in, seed=0, device="cpu"):
    """nn.Linear(k_in, n_out) weight distribution U(+-1/sqrt(k_in)), bf16."""
    g = _generator(seed, device)
    bound = 1.0 / math.sqrt(k_in)
    numel = n_out * k_in
    out = torch.empty(numel, dtype=torch.bfloat16, device=device)
    for s in range(0, numel, _CHUNK):
        e = min(numel, s + _CHUNK)
        t = torch.empty(e - s, dtype=torch.float32, device=device)
        t.uniform_(-bound, bound, generator=g)
        out[s:e] = t.to(torch.bfloat16)
    return out.view(n_out, k_in)


def bf16_bits(t):
    """A bf16 torch tensor -> numpy uint16 array of its bit patterns (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_device(t, device="cuda"):
    return t.to(device=device, copy=True).contiguous()
