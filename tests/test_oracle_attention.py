"""Pins of the oracle's attention, split merge and chunk attention (CPU only).

Pinned against closed forms (one token, equal keys, two tokens, a dominant
score), symmetries (copies of a query, Hq == Hkv), PyTorch's float64
``scaled_dot_product_attention`` (an independent library implementation of
the same definition), and SciPy's ``logsumexp`` for the merge.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import synth
from oracle import attention


def _rand(seed, *shape):
    return synth.normal(synth.rng(seed), shape).astype(np.float64)


def test_one_token_returns_its_value():
    q, k, v = _rand(1, 8), _rand(2, 1, 8), _rand(3, 1, 8)
    assert np.array_equal(attention.attend(q, k, v, 0.3), v[0])


def test_zero_query_and_equal_keys_give_the_mean_value():
    V = _rand(4, 9, 5)
    assert np.allclose(attention.attend(np.zeros(5), _rand(5, 9, 5), V, 1.0), V.mean(0), atol=1e-15)
    K = np.tile(_rand(6, 1, 5), (9, 1))
    assert np.allclose(attention.attend(_rand(7, 5), K, V, 1.0), V.mean(0), atol=1e-14)


def test_two_tokens_are_a_logistic_mix():
    q, K, V = _rand(8, 4), _rand(9, 2, 4), _rand(10, 2, 4)
    s = 0.7 * (K @ q)
    w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    assert np.allclose(attention.attend(q, K, V, 0.7), w0 * V[0] + (1 - w0) * V[1], rtol=1e-13, atol=1e-15)


def test_dominant_score_selects_its_value():
    K = np.zeros((6, 3))
    K[4] = [100.0, 0, 0]
    V = _rand(11, 6, 3)
    out = attention.attend(np.array([10.0, 0, 0]), K, V, 1.0)
    assert np.allclose(out, V[4], atol=1e-300)


def _sdpa(q, K, V, scale, mask=None):
    """torch float64 SDPA; q [H, Lq, D], K/V [H, Lk, D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale).numpy()


def test_decode_matches_torch_sdpa_with_gqa():
    B, Hq, Hkv, cap, D = 3, 8, 2, 40, 16
    q, kc, vc = _rand(12, B, Hq, D), _rand(13, B, Hkv, cap, D), _rand(14, B, Hkv, cap, D)
    L = [1, 17, 40]
    out = attention.decode_attention(q, kc, vc, L)
    G = Hq // Hkv
    for b in range(B):
        Ke = np.repeat(kc[b, :, :L[b]], G, axis=0)      # head h reads kv head h // G
        Ve = np.repeat(vc[b, :, :L[b]], G, axis=0)
        ref = _sdpa(q[b][:, None, :], Ke, Ve, 1 / math.sqrt(D))[:, 0]
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_copies_of_a_query_in_a_group_agree_and_mha_is_per_head():
    B, Hkv, G, cap, D = 2, 3, 4, 10, 8
    kc, vc = _rand(15, B, Hkv, cap, D), _rand(16, B, Hkv, cap, D)
    q1 = _rand(17, B, Hkv, D)
    q = np.repeat(q1, G, axis=1)
    out = attention.decode_attention(q, kc, vc, [7, 10])
    for h in range(Hkv * G):
        assert np.array_equal(out[:, h], out[:, (h // G) * G])
    mha = attention.decode_attention(q1, kc, vc, [7, 10])
    assert np.array_equal(mha, out[:, ::G])


@pytest.mark.parametrize("cuts", [[], [5], [0, 0, 13], [1, 2, 3, 30], [29, 29]])
def test_split_merge_equals_one_pass(cuts):
    q, K, V = _rand(18, 12), _rand(19, 30, 12), _rand(20, 30, 12)
    edges = [0] + list(cuts) + [30]
    parts = attention.split_partials(q, K, V, list(zip(edges[:-1], edges[1:])), 0.25)
    merged = attention.merge_partials(parts)
    assert np.allclose(merged, attention.attend(q, K, V, 0.25), rtol=1e-13, atol=1e-14)
    # the partials' (m, l) combine to log-sum-exp of all scores (SciPy)
    s = 0.25 * (K @ q)
    live = [(m, l) for m, l, _ in parts if l > 0]
    m_star = max(m for m, _ in live)
    l_star = sum(l * math.exp(m - m_star) for m, l in live)
    assert math.isclose(m_star + math.log(l_star), logsumexp(s), rel_tol=1e-13)


def test_merge_of_nothing_is_an_error():
    with pytest.raises(ValueError):
        attention.merge_partials([(-math.inf, 0.0, np.zeros(3))])


def test_chunk_attention_matches_sdpa_with_an_offset_causal_mask():
    Hq, Hkv, C, p0, D = 4, 2, 7, 5, 8
    q, K, V = _rand(21, Hq, C, D), _rand(22, Hkv, p0 + C, D), _rand(23, Hkv, p0 + C, D)
    out = attention.chunk_attention(q, K, V, p0)
    mask = np.arange(p0 + C)[None, :] <= (p0 + np.arange(C))[:, None]
    ref = _sdpa(q, np.repeat(K, 2, 0), np.repeat(V, 2, 0), 1 / math.sqrt(D), mask)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_chunk_reduces_to_decode():
    Hq, Hkv, C, p0, D = 4, 2, 6, 9, 8
    q, K, V = _rand(24, Hq, C, D), _rand(25, Hkv, p0 + C, D), _rand(26, Hkv, p0 + C, D)
    out = attention.chunk_attention(q, K, V, p0)
    last = attention.decode_attention(q[None, :, -1], K[None], V[None], [p0 + C])[0]
    assert np.array_equal(out[:, -1], last)
    one = attention.chunk_attention(q[:, :1], K[:, :p0 + 1], V[:, :p0 + 1], p0)
    assert np.array_equal(one[:, 0], attention.decode_attention(q[None, :, 0], K[None], V[None], [p0 + 1])[0])


def test_value_head_size_may_differ_from_key_head_size():
    """Dk != Dv: torch float64 scaled_dot_product_attention takes a value width of its own."""
    g = synth.rng(911)
    B, Hq, Hkv, Dk, Dv, cap = 2, 4, 2, 16, 24, 30
    L = np.array([7, 30], np.int32)
    q = synth.normal(g, (B, Hq, Dk)).astype(np.float64)
    k = synth.normal(g, (B, Hkv, cap, Dk)).astype(np.float64)
    v = synth.normal(g, (B, Hkv, cap, Dv)).astype(np.float64)
    got = attention.decode_attention(q, k, v, L)
    assert got.shape == (B, Hq, Dv)
    for b in range(B):
        for h in range(Hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h])[None, None], torch.from_numpy(k[b, h // 2, :L[b]])[None],
                torch.from_numpy(v[b, h // 2, :L[b]])[None])[0, 0].numpy()
            np.testing.assert_allclose(got[b, h], ref, rtol=1e-12, atol=1e-12)
