"""Seeded synthetic inputs for the compressed-attention path.

This module only draws numbers: counter-based Philox streams keyed by
(seed, tensor name), standard-normal / uniform draws, and rounding of those
draws to the input dtypes (fp32, bf16).  It holds none of the method's
arithmetic (no pooling, norm, RoPE, quantisation, scoring or attention) and
is shared by the tests, the oracle side and the benchmark as plain input.

Arrays are numpy: float32, or uint16 bit patterns for bf16.
"""
from __future__ import annotations

import zlib

import numpy as np
import torch


def stream(seed: int, name: str) -> np.random.Generator:
    """Independent counter-based stream for one named tensor."""
    return np.random.Generator(np.random.Philox(key=[int(seed), zlib.crc32(name.encode())]))


def normal(seed: int, name: str, shape, scale: float = 1.0) -> np.ndarray:
    x = stream(seed, name).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def uniform(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    return stream(seed, name).uniform(lo, hi, size=shape).astype(np.float32)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (nearest even, via torch's conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bf16(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(seed: int, name: str, c: int, frac: float = 0.01) -> np.ndarray:
    """A fixed seeded set of round(frac*c) channels (at least one)."""
    n = max(1, int(round(frac * c)))
    return np.sort(stream(seed, name).choice(c, size=n, replace=False))


def activations(seed: int, name: str, shape, outlier_frac: float = 0.01,
                outlier_gain: float = 20.0) -> np.ndarray:
    """N(0,1) activations whose last axis has a seeded 1% of channels scaled x20."""
    x = normal(seed, name, shape)
    if outlier_frac > 0:
        ch = outlier_channels(seed, name + "/outliers", shape[-1], outlier_frac)
        x[..., ch] *= np.float32(outlier_gain)
    return x


def block_scaled(seed: int, name: str, b: int, rows: int, c: int, lo: float = 0.1,
                 hi: float = 10.0) -> np.ndarray:
    """Sequence b's rows: N(0,1)^c times a per-row scale drawn log-uniform in [lo, hi].

    Each sequence has its own streams, so one sequence can be rebuilt alone.
    """
    sig = np.exp(stream(seed, f"{name}/{b}/sigma").uniform(np.log(lo), np.log(hi), size=rows))
    x = normal(seed, f"{name}/{b}", (rows, c))
    x *= sig.astype(np.float32)[:, None]
    return x
