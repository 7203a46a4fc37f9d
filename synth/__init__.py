"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds raw random draws only: Gaussian and uniform floats, uniform
integer symbols, random sign bits and rare outliers.  It contains none of the
method's arithmetic (no quantizer, packer, rotation, hash or dot product), so
the CPU oracle and the HIP library each turn these draws into codes on their
own.

Seeds are lists of small integers fed to numpy's SeedSequence; a draw is a
pure function of (seed list, shape, parameters).  Large draws that must live on
the GPU use torch's device generator seeded from the same SeedSequence; those
values differ from the numpy ones, so a test always hands one materialised
copy of the inputs to both sides.
"""
from __future__ import annotations

import numpy as np

# Output rows N and input columns K of the seven weight matrices of one layer
# of the 27B-shaped model: 24 query heads and 4 key/value heads of dim 256
# over a 5120-wide residual stream, a 17408-wide FFN.
LAYER_SHAPES = (
    ("q", 6144, 5120),
    ("k", 1024, 5120),
    ("v", 1024, 5120),
    ("o", 5120, 6144),
    ("gate", 17408, 5120),
    ("up", 17408, 5120),
    ("down", 5120, 17408),
)
# The same layer with q, k and v fused into one 8192-row matrix.
LAYER_SHAPES_FUSED = (
    ("qkv", 8192, 5120),
    ("o", 5120, 6144),
    ("gate", 17408, 5120),
    ("up", 17408, 5120),
    ("down", 5120, 17408),
)
N_LAYERS = 64
ATTN = ("q", "k", "v", "o", "qkv")


def rng(*seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(s) for s in seed])))


def seed64(*seed) -> int:
    """A 63-bit integer derived from the seed list (for torch generators)."""
    return int(np.random.SeedSequence([int(s) for s in seed]).generate_state(2, np.uint64)[0] >> np.uint64(1))


def gauss(seed, shape, sigma: float = 1.0) -> np.ndarray:
    g = rng(*seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def uniform(seed, shape, lo: float, hi: float) -> np.ndarray:
    g = rng(*seed)
    return (g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """Store float data as IEEE fp16 bit patterns (numpy round-to-nearest-even)."""
    return np.ascontiguousarray(np.asarray(x, np.float32).astype(np.float16)).view(np.uint16)


def uniform_f16(seed, shape, lo: float, hi: float) -> np.ndarray:
    return f16_bits(uniform(seed, shape, lo, hi))


def trits(seed, shape) -> np.ndarray:
    """Values in {-1, 0, 1}, each with probability 1/3."""
    return (rng(*seed).integers(0, 3, size=shape, dtype=np.int8) - 1).astype(np.int8)


def symbols(seed, shape, n: int) -> np.ndarray:
    """Uniform integer symbols 0..n-1 (int8)."""
    return rng(*seed).integers(0, n, size=shape, dtype=np.int8)


def integers(seed, shape, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in [lo, hi] (int32)."""
    return rng(*seed).integers(lo, hi + 1, size=shape, dtype=np.int32)


def u16(seed, shape) -> np.ndarray:
    return rng(*seed).integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)


def sign_bits(seed, K: int) -> np.ndarray:
    """K random sign bits packed 32 per uint32 word (bit k%32 of word k/32)."""
    assert K % 32 == 0
    return rng(*seed).integers(0, 1 << 32, size=K // 32, dtype=np.uint64).astype(np.uint32)


def with_outliers(x: np.ndarray, seed, p: float = 0.001, factor: float = 20.0) -> np.ndarray:
    """Each entry independently, with probability p, multiplied by factor."""
    m = rng(*seed).random(size=x.shape) < p
    y = x.copy()
    y[m] *= np.float32(factor)
    return y


# -- device-side draws (torch is only plumbing here) ---------------------------

def gauss_torch(seed, shape, sigma: float = 1.0, device: str = "cuda"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed64(*seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x


def _torch_gen(seed, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed64(*seed))
    return g


def bytes_torch(seed, shape, device: str = "cuda"):
    """Uniform random bytes (uint8) drawn on the device."""
    import torch

    return torch.randint(0, 256, shape, generator=_torch_gen(seed, device), device=device, dtype=torch.uint8)


def u16_torch(seed, shape, device: str = "cuda"):
    """Uniform 16-bit words drawn on the device, stored as int16 bit patterns."""
    import torch

    x = torch.randint(0, 1 << 16, shape, generator=_torch_gen(seed, device), device=device, dtype=torch.int32)
    return x.to(torch.int16)


def uniform_f16_torch(seed, shape, lo: float, hi: float, device: str = "cuda"):
    """U[lo, hi) fp32 draws on the device stored as fp16 bit patterns (int16),
    rounded to nearest even."""
    import torch

    x = torch.rand(shape, generator=_torch_gen(seed, device), device=device, dtype=torch.float32)
    return (x * (hi - lo) + lo).to(torch.float16).view(torch.int16)
