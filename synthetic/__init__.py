"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers; it holds none of the quantization
arithmetic.  Every tensor is produced on the CPU with a ``torch.Generator``
seeded explicitly, in float32, and then rounded to bfloat16 by torch.

Workloads follow the linear-layer shapes the pages train with (Llama-3-8B and
Qwen3-8B feed-forward projections; torchtitan PR #3914 "Add an NVFP4
quantization converter", Numerical and performance validation / Table 1):
activations ~ N(0, 1), weights ~ N(0, 0.02^2), output gradients ~ N(0, 1e-4^2).
The pages train on the C4 dataset; these Gaussian tensors stand in for it.
"""
from __future__ import annotations

import torch

# Seeds of the standard workloads.
SEED_X = 1234
SEED_W = 1235
SEED_DY = 1236
SEED_OUTLIER_MASK = 1237
SEED_SR_KEY = 42
SEED_SIGNS = 7

STD_X = 1.0
STD_W = 0.02
STD_DY = 1e-4


def gaussian_bf16(shape, std: float, seed: int) -> torch.Tensor:
    """bf16 CPU tensor of N(0, std^2) samples (float32 draw, then bf16 RNE by torch)."""
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(float(std))
    return t.to(torch.bfloat16)


def outlier_bf16(shape, seed: int = SEED_X, mask_seed: int = SEED_OUTLIER_MASK,
                 frac: float = 0.01, factor: float = 100.0) -> torch.Tensor:
    """N(0,1) bf16 tensor in which a random ``frac`` of the entries is multiplied by ``factor``.

    The mask is ``U(0,1) < frac`` drawn from its own generator, so a block of 16
    contains an outlier with probability 1 - (1 - frac)^16 (about 15 % at 1 %).
    """
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    gm = torch.Generator().manual_seed(int(mask_seed))
    mask = torch.rand(tuple(shape), generator=gm, dtype=torch.float32) < frac
    t[mask] *= factor
    return t.to(torch.bfloat16)


def rht_signs(seed: int = SEED_SIGNS, n: int = 16) -> torch.Tensor:
    """int8 vector of n random +-1 entries (the Hadamard sign vector)."""
    g = torch.Generator().manual_seed(int(seed))
    bits = torch.randint(0, 2, (n,), generator=g, dtype=torch.int64)
    return (bits * 2 - 1).to(torch.int8)


def uniform_f32(shape, lo: float, hi: float, seed: int) -> torch.Tensor:
    """float32 CPU tensor of U(lo, hi) samples."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.rand(tuple(shape), generator=g, dtype=torch.float32) * (hi - lo) + lo


def bf16_bits(t: torch.Tensor):
    """The raw 16-bit patterns of a bf16 CPU tensor, as a contiguous numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


# Workload descriptions (shapes and distributions) used by tests and the bench.
WORKLOADS = {
    "tiny": dict(x=(128, 256), w=(256, 256)),
    "quant": dict(x=(8192, 4096)),
    "fwd": dict(x=(16384, 4096), w=(14336, 4096)),
    "wgrad": dict(dy=(16384, 14336), x=(16384, 4096)),
    "hybrid": dict(x=(65536, 4096), w=(12288, 4096), dy=(65536, 12288)),
}
