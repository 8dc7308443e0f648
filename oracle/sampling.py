"""Greedy and seeded temperature sampling of the final logits.

"Persistent input/output feedback", section "Autoregressive generation":
temperature 0 decodes greedily; a positive temperature samples
``softmax(logits / temperature)``; a seed makes the draw repeatable within the
same implementation; the logits are ``[batch, vocab]`` or
``[batch, sequence, vocab]`` and the final position predicts the next token.

Readings (the pages fix only the distribution; listed in the design doc):

* greedy is the argmax of the logits as given (DOUBLE logits are compared as
  float64 values), ties to the lowest index;
* non-finite values follow ``numpy.argmax``: NaN ranks above every number (the
  first NaN wins) and a row of -inf values gives index 0, so every row gets an
  index inside the vocabulary;
* the temperature ``T`` is a float32 value (the type the library's boundary
  takes);
* a draw is the Gumbel-max choice ``argmax_v (y_v - log(-log u_v))``, which
  has exactly the law ``softmax(x / T)``, with ``y_v = fl32(x_v * invT)``,
  ``invT = fl32(1 / T)`` for FLOAT / FLOAT16 / BFLOAT16 logits and
  ``y_v = fl64(x_v * (1 / T))`` in float64 for DOUBLE logits;
* ``u_v`` is made from output number ``k = b * V + v + 1`` of the SplitMix64
  sequence seeded with ``seed`` (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014): ``u = ((h >> 40) | 1) * 2^-24``,
  an odd multiple of 2^-24, exact in float32 and strictly inside (0, 1).

The oracle evaluates the Gumbel term in float64; a GPU evaluating it in
float32 can only differ on rows whose two best candidates are within a few
float32 ulps, so the draw is compared by agreement rate and near-tie
confirmation, not bit for bit.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64_mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (the finaliser applied to the advanced state)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_outputs(seed: int, k: np.ndarray) -> np.ndarray:
    """Output number ``k`` (1-based) of SplitMix64 started from state ``seed``:
    the state after k increments is ``seed + k * gamma`` (mod 2^64)."""
    k = np.asarray(k, dtype=np.uint64)
    return splitmix64_mix(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * GOLDEN_GAMMA)


def uniforms(seed: int, b: int, V: int) -> np.ndarray:
    """``u[b, v]`` for v in 0..V-1 as float64 (exactly the float32 value)."""
    k = np.uint64(b) * np.uint64(V) + np.arange(V, dtype=np.uint64) + np.uint64(1)
    h = splitmix64_outputs(seed, k)
    return ((h >> np.uint64(40)) | np.uint64(1)).astype(np.float64) * 2.0 ** -24


def last_position(logits: np.ndarray) -> np.ndarray:
    """``[B, V]`` or ``[B, S, V]`` -> ``[B, V]`` (final sequence position)."""
    logits = np.asarray(logits)
    if logits.ndim == 3:
        return logits[:, -1, :]
    if logits.ndim != 2:
        raise ValueError("logits must be [B, V] or [B, S, V]")
    return logits


def _values(logits: np.ndarray) -> np.ndarray:
    """The logits as numbers: float64 arrays (DOUBLE logits) stay float64,
    anything else is taken as float32 values (FLOAT16 / BFLOAT16 widen
    exactly)."""
    x = np.asarray(logits)
    return x if x.dtype == np.float64 else x.astype(np.float32)


def greedy(logits: np.ndarray) -> np.ndarray:
    """Index of the largest logit per row, lowest index on ties.

    ``numpy.argmax`` returns the first (lowest) index among equal maxima, and
    the first NaN when a row holds one.
    """
    x = _values(last_position(logits))
    return np.argmax(x, axis=-1).astype(np.int64)


def temperature32(T: float) -> float:
    """The temperature as the float32 value the boundary receives."""
    return float(np.float32(T))


def inv_temperature(T: float) -> np.float32:
    """``fl32(1 / T)`` for the float32 temperature ``T``."""
    return np.float32(1.0 / temperature32(T))


def gumbel_scores(logits_row: np.ndarray, T: float, seed: int, b: int) -> np.ndarray:
    """Perturbed scores ``y - log(-log u)`` of one row, float64.

    ``y = fl32(x * fl32(1 / T))`` (one float32 multiply, then exact widening)
    for float32 values; ``y = x * (1 / T)`` in float64 for float64 logits.
    """
    x = _values(logits_row)
    with np.errstate(invalid="ignore"):
        if x.dtype == np.float64:
            y = x * (1.0 / temperature32(T))
        else:
            y = (x * inv_temperature(T)).astype(np.float64)
    u = uniforms(seed, b, x.shape[0])
    return y - np.log(-np.log(u))


def sample(logits: np.ndarray, temperature: float, seed: int) -> np.ndarray:
    """Token id per row: greedy when ``temperature == 0``, else a Gumbel-max draw.

    ``logits`` holds the values: float64 for DOUBLE logits, float32 for the
    others (bf16/fp16 inputs widened exactly by the caller).
    """
    if not (temperature >= 0.0):
        raise ValueError("temperature must be >= 0 and not NaN")
    x = _values(last_position(logits))
    if temperature == 0.0:
        return greedy(x)
    out = np.empty(x.shape[0], dtype=np.int64)
    for b in range(x.shape[0]):
        out[b] = int(np.argmax(gumbel_scores(x[b], temperature, seed, b)))
    return out


def top2_gap(scores: np.ndarray) -> float:
    """Difference between the best and second-best score of a row."""
    s = np.sort(np.asarray(scores, dtype=np.float64))
    return float(s[-1] - s[-2])
