"""Pins of stateful == stateless decode and of the byte accounting (CPU only).

Pinned against the pages' printed numbers (the four-token table and the
dense fixture in tests/golden/) and against the stateless full-prefix loop,
which the pages declare equivalent to retained state.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import accounting, cache, stateless

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_steps(T, D, seed=0, Hq=1, Hkv=1):
    g = synth.rng(seed, 1)
    f = lambda *s: synth.uniform(g, s, -1, 1).astype(np.float64)
    return f(T, Hq, D), f(T, Hkv, D), f(T, Hkv, D)


def test_stateful_equals_stateless_on_the_tiny_fixture():
    q, k, v = _tiny_steps(16, 4)
    outs, kc, vc = stateless.stateful_decode(q, k, v, capacity=16)
    ref = stateless.stateless_decode(q, k, v)
    assert np.array_equal(outs, ref)             # same arithmetic, same order: identical
    assert np.array_equal(kc[0, :, :16], np.transpose(k, (1, 0, 2)))


def test_tiny_fixture_overflow_step_fails_and_keeps_the_cache():
    q, k, v = _tiny_steps(17, 4)
    with pytest.raises(cache.CapacityError):
        stateless.stateful_decode(q, k, v, capacity=16)


def test_gqa_stateful_equals_stateless():
    q, k, v = _tiny_steps(9, 8, seed=3, Hq=6, Hkv=2)
    outs, _, _ = stateless.stateful_decode(q, k, v, capacity=12)
    assert np.array_equal(outs, stateless.stateless_decode(q, k, v))


def test_retained_and_append_bytes_reproduce_the_four_token_table():
    table = _golden("feedback_tensor_cache_table.json")
    cols = table["columns"]
    Dk = Dv = 2                                  # 4 * (Dk + Dv) = 16 append bytes per token
    k_cache = np.zeros((1, 1, 4, Dk), np.float32)
    v_cache = np.zeros((1, 1, 4, Dv), np.float32)
    for row in table["rows"]:
        r = dict(zip(cols, row))
        t = r["token"]
        before_k, before_v = k_cache.copy(), v_cache.copy()
        cache.cache_update(k_cache, np.full((1, 1, 1, Dk), t, np.float32), [t - 1], 1)
        cache.cache_update(v_cache, np.full((1, 1, 1, Dv), t, np.float32), [t - 1], 1)
        # bytes that changed are exactly one token row per tensor
        changed = int((k_cache != before_k).sum()) * 4 + int((v_cache != before_v).sum()) * 4
        assert changed == r["kernel_append_copied_bytes"] == accounting.append_bytes(1, 1, 1, [Dk, Dv], 4)
        visible = k_cache[:, :, :t].nbytes + v_cache[:, :, :t].nbytes
        assert visible == r["retained_logical_bytes"] == accounting.retained_logical_bytes(t, 1, 1, [Dk, Dv], 4)
        assert r["kernel_prefix_copied_bytes"] == 0 == accounting.in_place_extra_cache_bytes()


def test_dense_fixture_and_fallback_formula():
    f = _golden("feedback_copy_formulas.json")
    d = f["dense_fixture"]
    assert accounting.append_bytes(d["tokens_per_call"], 1, 1, [d["key_width"], d["value_width"]], 4) == d["append_bytes"]
    # the fallback copies the whole prefix every step: 4 * B * H * L * (Dk + Dv)
    B, H, L, Dk, Dv = 2, 3, 17, 5, 7
    assert accounting.fallback_prefix_bytes(L, B, H, [Dk, Dv], 4) == 4 * B * H * L * (Dk + Dv)
    assert accounting.append_bytes(1, B, H, [Dk, Dv], 4) == 4 * B * H * (Dk + Dv)
