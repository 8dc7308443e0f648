"""Seeded synthetic inputs shared by the oracle, the tests and the bench.

This module only draws random numbers and lays them out.  It holds none of
the decode step's arithmetic (no cache update, attention, quantisation or
sampling): every value it returns is an *input*.  Both the CPU oracle and the
HIP path consume the same bits from here.

Recipe (also stated in the design doc):

* every generator is ``numpy.random.Generator(PCG64(SeedSequence([seed, *stream])))``
  so that any part of a large input (one batch row, one cache tensor) can be
  regenerated on its own from ``(seed, stream)``;
* ``U[a, b]`` is ``Generator.uniform`` in float32;
* ``N(0, sigma)`` is ``Generator.standard_normal`` in float32 times sigma;
* bf16 values are the float32 draws rounded to nearest-even in the top 16 bits;
* context lengths are ``clip(rint(exp(mu + sigma * z)), lo, hi)`` with
  ``z ~ N(0, 1)`` (a lognormal length mix);
* page tables come from a Fisher-Yates permutation (``Generator.permutation``)
  of the physical block ids, handed out in order to the rows.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng", "uniform", "normal", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "lognormal_lengths", "permutation", "f16_bits",
]


def rng(seed: int, *stream: int) -> np.random.Generator:
    """Independent generator for ``(seed, *stream)``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def uniform(gen: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return gen.uniform(lo, hi, size=shape).astype(np.float32)


def normal(gen: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the uint16 bit patterns.

    Infinities and quiet NaNs whose top mantissa bit is set (numpy's ``nan``
    and ``-nan``) keep their class; other NaN payloads are not expected.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """Round to IEEE binary16 (nearest-even, numpy's cast) and return uint16 bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def lognormal_lengths(gen: np.random.Generator, n: int, mu: float, sigma: float,
                      lo: int, hi: int) -> np.ndarray:
    z = gen.standard_normal(size=n)
    return np.clip(np.rint(np.exp(mu + sigma * z)), lo, hi).astype(np.int32)


def permutation(gen: np.random.Generator, n: int) -> np.ndarray:
    return gen.permutation(n).astype(np.int32)
