"""Seeded synthetic inputs for the codec workloads.

This module draws random inputs and nothing else: it holds none of the
codec's arithmetic (no statistics, rounding, quantization or packing), so
the GPU path and the CPU oracle can both be fed from it.

Two families:

* ``host_*`` functions return numpy arrays drawn with
  ``numpy.random.Generator(PCG64(seed))``; used for sizes a test can hold
  on the host comfortably.
* ``device_*`` functions return torch tensors drawn on a GPU with a seeded
  ``torch.Generator`` (deterministic for a given seed and torch build); used
  for the full-size workloads, where host generation would dominate.

Distributions follow the workloads the codec is measured on: gradients
~ N(0, sigma) (sigma is the standard deviation), Laplace(0, b) gradients
(b is the scale), embedding rows ~ N(0, sigma) with a fraction of rows
scaled up (heavy tail), gradients with Bernoulli outlier entries scaled up,
bf16 gradients rounded from fp32, and random 1-bit sign words.
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------ host


def host_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def host_normal(n: int, sigma: float, seed: int) -> np.ndarray:
    """float32[n] ~ N(0, sigma)."""
    g = host_rng(seed)
    x = g.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    return x


def host_laplace(n: int, b: float, seed: int) -> np.ndarray:
    """float32[n] ~ Laplace(0, b)."""
    return host_rng(seed).laplace(0.0, b, n).astype(np.float32)


def host_embedding_rows(rows: int, dim: int, sigma: float, heavy_frac: float, heavy_mult: float,
                        seed: int) -> np.ndarray:
    """float32[rows*dim]: N(0, sigma) rows; round(heavy_frac*rows) rows, chosen
    without replacement, are multiplied by heavy_mult."""
    g = host_rng(seed)
    x = g.standard_normal(rows * dim, dtype=np.float32)
    x *= np.float32(sigma)
    nheavy = int(round(heavy_frac * rows))
    if nheavy:
        idx = g.choice(rows, size=nheavy, replace=False)
        x2 = x.reshape(rows, dim)
        x2[idx] *= np.float32(heavy_mult)
    return x


def host_outlier_grad(n: int, sigma: float, p: float, mult: float, seed: int) -> np.ndarray:
    """float32[n] ~ N(0, sigma); each entry independently (prob p) times mult."""
    g = host_rng(seed)
    x = g.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    mask = g.random(n) < p
    x[mask] *= np.float32(mult)
    return x


def host_bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of x rounded to bfloat16 (round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_words(count: int, seed: int) -> np.ndarray:
    """uint32[count] of independent uniformly random bits."""
    return host_rng(seed).integers(0, 2**32, size=count, dtype=np.uint32)


# ------------------------------------------------------------------ device


def _gen(seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_normal(n: int, sigma: float, seed: int, device="cuda"):
    import torch

    x = torch.empty(n, dtype=torch.float32, device=device)
    x.normal_(0.0, sigma, generator=_gen(seed, device))
    return x


def device_laplace(n: int, b: float, seed: int, device="cuda"):
    """Laplace(0, b) by inverse CDF of a uniform draw on (-1/2, 1/2)."""
    import torch

    u = torch.empty(n, dtype=torch.float32, device=device)
    u.uniform_(-0.5, 0.5, generator=_gen(seed, device))
    # x = -b * sign(u) * log(1 - 2|u|); clamp keeps log finite at |u| -> 1/2
    mag = torch.log1p(-2.0 * u.abs()).clamp_min_(-80.0)
    x = torch.sign(u).mul_(mag).mul_(-b)
    del u, mag
    return x


def device_embedding_rows(rows: int, dim: int, sigma: float, heavy_frac: float, heavy_mult: float,
                          seed: int, device="cuda"):
    import torch

    g = _gen(seed, device)
    x = torch.empty(rows * dim, dtype=torch.float32, device=device)
    x.normal_(0.0, sigma, generator=g)
    nheavy = int(round(heavy_frac * rows))
    if nheavy:
        idx = torch.randperm(rows, generator=g, device=device)[:nheavy]
        x.view(rows, dim)[idx] *= heavy_mult
    return x


def device_outlier_grad(n: int, sigma: float, p: float, mult: float, seed: int, device="cuda"):
    import torch

    g = _gen(seed, device)
    x = torch.empty(n, dtype=torch.float32, device=device)
    x.normal_(0.0, sigma, generator=g)
    u = torch.empty(n, dtype=torch.float32, device=device)
    u.uniform_(0.0, 1.0, generator=g)
    x = torch.where(u < p, x * mult, x)
    return x


def device_bf16_normal(n: int, sigma: float, seed: int, device="cuda"):
    import torch

    return device_normal(n, sigma, seed, device).to(torch.bfloat16)


def device_words(count: int, seed: int, device="cuda"):
    """int32[count] tensor of uniformly random bit patterns."""
    import torch

    w = torch.empty(count, dtype=torch.int32, device=device)
    w.random_(-(2**31), 2**31, generator=_gen(seed, device))
    return w
