"""Byte accounting of the decode step.

"Persistent input/output feedback":

* section "Persistent input/output feedback": ``retained_logical_bytes``
  measures the visible tensor lengths, not the reserved capacity;
* section "Opt-in storage auditing through runtime events": appending one
  FLOAT token with head sizes Dk and Dv copies ``4 * (Dk + Dv)`` bytes, reuse
  within capacity allocates nothing and copies no prefix, and the dense
  fallback for B batches, H KV heads and an L-token prefix copies
  ``4 * B * H * L * (Dk + Dv)`` prefix bytes plus ``4 * B * H * (Dk + Dv)``
  append bytes per token.

"Mutable execution cache", section "Memory planning": an in-place update
counts as zero additional cache bytes; peak memory is workspace plus newly
allocated pages.
"""
from __future__ import annotations


def retained_logical_bytes(valid_len: int, batch: int, heads: int, head_sizes, elem_bytes: int) -> int:
    """Visible bytes of the retained K/V tensors (sum over the tensors in ``head_sizes``)."""
    return sum(int(valid_len) * batch * heads * d * elem_bytes for d in head_sizes)


def append_bytes(new_tokens: int, batch: int, heads: int, head_sizes, elem_bytes: int) -> int:
    """Bytes written by an in-place append of ``new_tokens`` tokens."""
    return sum(int(new_tokens) * batch * heads * d * elem_bytes for d in head_sizes)


def fallback_prefix_bytes(prefix_len: int, batch: int, heads: int, head_sizes, elem_bytes: int) -> int:
    """Prefix bytes a concatenating (non in-place) update copies for one step."""
    return sum(int(prefix_len) * batch * heads * d * elem_bytes for d in head_sizes)


def in_place_extra_cache_bytes() -> int:
    """Additional cache bytes of an in-place update (a second cache is never allocated)."""
    return 0


def decoded_bytes(query_positions, left_window: int, head_sizes, batch: int = 1, heads: int = 1) -> int:
    """FLOAT bytes decoded by windowed attention, counting every visible token
    again for every query ("Persistent input/output feedback", statistics of
    the direct call: decoded FLOAT bytes of visible tokens, repeated reads for
    different queries included).  A query at position ``p`` sees ``[max(0,
    p - W), p]`` for ``W = left_window >= 0`` and ``[0, p]`` for ``W = -1``."""
    visible = 0
    for p in query_positions:
        lo = 0 if left_window < 0 else max(0, int(p) - left_window)
        visible += int(p) - lo + 1
    return visible * batch * heads * sum(int(d) for d in head_sizes) * 4
