"""Stateful (in-place) and stateless (full-prefix) decode loops.

"Custom, quantized, and persistent values", section "Persistent state from
model inputs and outputs": retaining selected outputs as the next call's
inputs is equivalent to the ordinary stateless loop that feeds those outputs
back by hand.  "Persistent input/output feedback", section "Autoregressive
generation": a model without retained state evaluates the full growing prefix.

``stateful_decode`` keeps one capacity-sized cache and appends into it in
place; ``stateless_decode`` rebuilds the K/V prefix by concatenation at every
step and recomputes attention from scratch.  Both return the per-step outputs.
"""
from __future__ import annotations

import numpy as np

from . import attention, cache


def stateful_decode(q_steps, k_steps, v_steps, capacity: int, scale=None):
    """One batch row, ``H`` heads.  ``*_steps`` are ``[T, H, D]`` (q may have Hq heads).

    Returns ``(outputs [T, Hq, D], k_cache, v_cache)``.  Raises
    :class:`cache.CapacityError` at the first step that would overflow; the
    caches are then unchanged by that step.
    """
    T, Hkv, D = k_steps.shape
    k_cache = np.zeros((1, Hkv, capacity, D), dtype=np.float64)
    v_cache = np.zeros((1, Hkv, capacity, D), dtype=np.float64)
    outs = []
    for t in range(T):
        cache.cache_update(k_cache, k_steps[t][None, :, None, :], [t], 1)
        cache.cache_update(v_cache, v_steps[t][None, :, None, :], [t], 1)
        outs.append(attention.decode_attention(q_steps[t][None], k_cache, v_cache, [t + 1], scale)[0])
    return np.stack(outs), k_cache, v_cache


def stateless_decode(q_steps, k_steps, v_steps, scale=None):
    """Same loop, but every step concatenates the retained outputs into fresh arrays."""
    T, Hkv, D = k_steps.shape
    past_k = np.zeros((Hkv, 0, D))
    past_v = np.zeros((Hkv, 0, D))
    outs = []
    for t in range(T):
        present_k = np.concatenate([past_k, k_steps[t][:, None, :]], axis=1)
        present_v = np.concatenate([past_v, v_steps[t][:, None, :]], axis=1)
        L = present_k.shape[1]
        outs.append(attention.decode_attention(q_steps[t][None], present_k[None], present_v[None], [L], scale)[0])
        past_k, past_v = present_k, present_v
    return np.stack(outs)
