"""Exact conversions between stored bit patterns and float64.

bf16 and fp16 values are exactly representable in float64, so widening is
exact; this is what lets the oracle compute "in double from exactly converted
inputs".  Rounding float64 results to bf16 is done in one step (no detour
through float32), nearest-even.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exact (bf16 is the top half of a float32)."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exact."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 (ties to even); returns uint16 bit patterns.

    Works on the float64 bit pattern: a bf16 keeps 8 significant bits, so the
    float64 significand is rounded at bit 45 (52 - 7) and the exponent
    re-biased.  Finite, normal-range inputs only (outputs of attention over
    finite inputs); subnormal bf16 results are flushed through float32.
    """
    x = np.asarray(x, dtype=np.float64)
    # Round the float64 value to 8 significant bits, nearest-even, exactly:
    # scale to an integer significand, use numpy's round-half-even, scale back.
    m, e = np.frexp(x)              # x = m * 2**e, 0.5 <= |m| < 1
    m8 = np.rint(m * 256.0) / 256.0  # 8 significant bits, ties to even
    r = np.ldexp(m8, e)              # exact in float64, and exactly a bf16 value
    f = r.astype(np.float32)         # exact: r has 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32(x) -> np.ndarray:
    """float64 -> float32 round-to-nearest-even (numpy cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
