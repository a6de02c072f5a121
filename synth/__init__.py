"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the arithmetic of the method (no matmul, GeLU, softmax, sums).
Both sides receive the exact same bits from here and nothing else.

Recipe: tensor ``sub`` of workload ``seed`` is drawn from
``torch.Generator('cpu').manual_seed(seed * 16 + sub)`` as ``torch.randn`` in
float32, multiplied by ``sigma`` and rounded (round-to-nearest-even) to the
requested dtype.  The sub-seed numbering is fixed by ``SUB``.
"""
from __future__ import annotations

import math

import torch

SUB = {"x": 0, "A": 1, "B": 2, "Wqkv": 3, "Wo": 4, "bias": 5, "partials": 6,
       "gamma": 7, "beta": 8, "residual": 9, "dZ": 10, "preact": 11, "tokens": 12,
       "targets": 13, "E": 14}


def normal(shape, sigma: float, seed: int, sub, dtype=torch.bfloat16):
    """N(0, sigma^2) tensor of ``shape`` on the CPU, rounded to ``dtype``."""
    if isinstance(sub, str):
        sub = SUB[sub]
    g = torch.Generator(device="cpu").manual_seed(int(seed) * 16 + int(sub))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(float(sigma))
    return t.to(dtype)


def fan_in_sigma(fan_in: int) -> float:
    """Standard deviation 1/sqrt(fan_in) used for every weight matrix."""
    return 1.0 / math.sqrt(fan_in)


def rank_seed(seed: int, rank: int) -> int:
    """Seed for rank ``rank``'s weights when several ranks are drawn."""
    return int(seed) * 64 + int(rank)


def token_ids(n: int, vocab: int, seed: int, sub) -> torch.Tensor:
    """n token ids uniform on [0, vocab) as int32, on the CPU."""
    if isinstance(sub, str):
        sub = SUB[sub]
    g = torch.Generator(device="cpu").manual_seed(int(seed) * 16 + int(sub))
    return torch.randint(0, int(vocab), (int(n),), generator=g, dtype=torch.int64).to(torch.int32)
