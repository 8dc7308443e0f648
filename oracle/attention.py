"""Attention of new queries over the valid cache prefix, in float64.

What is computed -- "Persistent input/output feedback", "Optional heterogeneous
paged KV", sections "Versioned operator schema" and "Kernel implementation":
Q is ``[batch, heads, L, D]``, the query head count is a multiple of the K/V
head count (grouped-query attention), masking is causal by default with an
unbounded left window, only valid visible tokens are read, and the current
K/V take part in the result.  Softmax attention is the plain definition:

    s_j = scale * <q, k_j>,   p_j = exp(s_j - max_i s_i),   o = sum_j p_j v_j / sum_j p_j

The pages use online softmax (one pass, running max and sum) to avoid a
cache-length score matrix; that changes rounding only, so the oracle writes
the definition out directly.

Readings (listed in the design doc): ``scale = 1/sqrt(D)`` unless given; query
head ``h`` reads K/V head ``h // G`` with ``G = Hq / Hkv`` (contiguous
groups); ``valid_len[b]`` counts the token appended in this step.

Left window (same pages, "Versioned operator schema": ``left_window_size``
-1 is unbounded, a non-negative value bounds the preceding tokens; "Kernel
implementation": causal masking and the window decide the visible range): a
query at absolute position ``p`` sees keys ``[max(0, p - W), p]``, i.e. itself
and at most ``W`` preceding tokens.

Split partials and their merge (the long-context split of the same online
softmax): a split over token range R yields ``m = max_{j in R} s_j``,
``l = sum_{j in R} exp(s_j - m)`` and ``o = sum_{j in R} exp(s_j - m) v_j``
(unnormalised); merging rescales each split by ``exp(m_i - m*)``.
"""
from __future__ import annotations

import math

import numpy as np


def _scale(D: int, scale) -> float:
    return 1.0 / math.sqrt(D) if (scale is None or scale <= 0) else float(scale)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query ``q[D]`` over keys ``K[L, D]`` and values ``V[L, D]`` (float64)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = scale * (K @ q)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def visible_begin(pos: int, left_window: int = -1) -> int:
    """First key a query at absolute position ``pos`` sees (the last is ``pos``)."""
    return 0 if left_window < 0 else max(0, pos - left_window)


def decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     valid_len, scale=None, left_window: int = -1) -> np.ndarray:
    """Single-token decode over a contiguous cache.

    ``q`` is ``[B, Hq, Dk]`` (or ``[B, Hq, 1, Dk]``), ``k_cache`` is
    ``[B, Hkv, capacity, Dk]`` and ``v_cache`` ``[B, Hkv, capacity, Dv]``
    (already float64; K and V head sizes may differ: "Contiguous CPU
    Attention feedback"), ``valid_len`` is ``[B]``; the query sits at position
    ``valid_len - 1``.  Returns ``[B, Hq, Dv]`` float64.
    """
    q = np.asarray(q, dtype=np.float64)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    G = Hq // Hkv
    sc = _scale(D, scale)
    out = np.empty((B, Hq, v_cache.shape[-1]), dtype=np.float64)
    for b in range(B):
        L = int(valid_len[b])
        if L < 1:
            raise ValueError("valid_len must be >= 1")
        lo = visible_begin(L - 1, left_window)
        for h in range(Hq):
            kv = h // G
            out[b, h] = attend(q[b, h], k_cache[b, kv, lo:L], v_cache[b, kv, lo:L], sc)
    return out


def split_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, bounds, scale: float):
    """Partials ``(m, l, o)`` of one query for each token range ``[lo, hi)`` in ``bounds``.

    An empty range gives ``m = -inf``, ``l = 0``, ``o = 0``.
    """
    q = np.asarray(q, dtype=np.float64)
    parts = []
    for lo, hi in bounds:
        if hi <= lo:
            parts.append((-math.inf, 0.0, np.zeros(K.shape[1])))
            continue
        s = scale * (np.asarray(K[lo:hi], dtype=np.float64) @ q)
        m = float(s.max())
        p = np.exp(s - m)
        parts.append((m, float(p.sum()), p @ np.asarray(V[lo:hi], dtype=np.float64)))
    return parts


def merge_partials(parts) -> np.ndarray:
    """Log-sum-exp merge: ``m* = max m_i``, ``l* = sum l_i e^(m_i - m*)``,
    ``o = sum o_i e^(m_i - m*) / l*``; empty parts (``l = 0``) contribute nothing."""
    live = [(m, l, o) for (m, l, o) in parts if l > 0]
    if not live:
        raise ValueError("no tokens in any split")
    m_star = max(m for m, _, _ in live)
    l_star = sum(l * math.exp(m - m_star) for m, l, _ in live)
    o = sum(o * math.exp(m - m_star) for m, _, o in live)
    return o / l_star


def chunk_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, p0: int, scale=None,
                    left_window: int = -1) -> np.ndarray:
    """Causal attention of a chunk of C queries of one row.

    ``q`` is ``[Hq, C, D]``; ``K``/``V`` are the row's logical ``[Hkv, p0 + C, D]``
    after the chunk was appended at position ``p0``.  Query ``t`` sits at
    absolute position ``p0 + t`` and attends keys ``[visible_begin(p0 + t), p0 + t]``.
    Returns ``[Hq, C, D]`` float64.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, C, D = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    sc = _scale(D, scale)
    out = np.empty((Hq, C, D), dtype=np.float64)
    for h in range(Hq):
        kv = h // G
        for t in range(C):
            last = p0 + t
            lo = visible_begin(last, left_window)
            out[h, t] = attend(q[h, t], K[kv, lo:last + 1], V[kv, lo:last + 1], sc)
    return out
