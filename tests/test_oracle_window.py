"""Pins of the left window ("Persistent input/output feedback", "Versioned
operator schema": left_window_size -1 is unbounded, W >= 0 bounds the
preceding tokens; "Kernel implementation": only visible tokens are read).

* the pages' windowed fixture (six retained tokens, two appended, window 1,
  INT8 keys of width 2 and UINT4 values of width 3): 80 decoded FLOAT bytes
  across the two queries, 7 new payload bytes (tests/golden);
* a torch float64 reference with an explicit banded causal mask;
* W = 0 returns the query's own value row; W >= position or W = -1 equals
  the unwindowed result.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import accounting, affine
from oracle import attention as oattn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "feedback_copy_formulas.json")


def test_windowed_fixture_bytes():
    fx = json.load(open(GOLDEN))["windowed_fixture"]
    n0, new, W = fx["retained_tokens"], fx["new_tokens"], fx["left_window"]
    queries = list(range(n0, n0 + new))
    assert accounting.decoded_bytes(queries, W, (fx["key_width"], fx["value_width"])) == fx["decoded_float_bytes"]
    # the unbounded window would read every retained token again
    assert accounting.decoded_bytes(queries, -1, (2, 3)) == (7 + 8) * 5 * 4
    payload = affine.payload_bytes(new * fx["key_width"], 8) + affine.payload_bytes(new * fx["value_width"], 4)
    assert payload == fx["new_payload_bytes"]


def _torch_banded(q, K, V, positions, W, scale):
    """float64 SDPA with a boolean mask: key j visible to a query at p iff p - W <= j <= p."""
    qt = torch.from_numpy(q)[None]                      # [1, nq, D]
    Kt = torch.from_numpy(K)[None]
    Vt = torch.from_numpy(V)[None]
    j = torch.arange(K.shape[0])[None, :]
    p = torch.tensor(positions)[:, None]
    mask = (j <= p) & ((j >= p - W) if W >= 0 else torch.ones_like(j, dtype=torch.bool))
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask[None], scale=scale)[0].numpy()


@pytest.mark.parametrize("W", [0, 1, 5, 37, 200, -1])
def test_decode_window_matches_banded_reference(W):
    g = synth.rng(901, W + 2)
    B, Hq, Hkv, D, cap = 3, 4, 2, 16, 120
    L = np.array([1, 64, 120], np.int32)
    q = synth.normal(g, (B, Hq, D)).astype(np.float64)
    k = synth.normal(g, (B, Hkv, cap, D)).astype(np.float64)
    v = synth.normal(g, (B, Hkv, cap, D)).astype(np.float64)
    got = oattn.decode_attention(q, k, v, L, left_window=W)
    for b in range(B):
        for h in range(Hq):
            ref = _torch_banded(q[b, h][None], k[b, h // 2, :L[b]], v[b, h // 2, :L[b]], [int(L[b]) - 1], W,
                                1 / np.sqrt(D))[0]
            np.testing.assert_allclose(got[b, h], ref, rtol=1e-12, atol=1e-12)


def test_window_special_cases():
    g = synth.rng(902)
    B, H, D, cap = 2, 2, 8, 50
    L = np.array([50, 9], np.int32)
    q = synth.normal(g, (B, H, D)).astype(np.float64)
    k = synth.normal(g, (B, H, cap, D)).astype(np.float64)
    v = synth.normal(g, (B, H, cap, D)).astype(np.float64)
    own = oattn.decode_attention(q, k, v, L, left_window=0)
    for b in range(B):
        assert np.array_equal(own[b], v[b, :, L[b] - 1])               # only the query's own row
    full = oattn.decode_attention(q, k, v, L)
    assert np.array_equal(oattn.decode_attention(q, k, v, L, left_window=49), full)
    assert np.array_equal(oattn.decode_attention(q, k, v, L, left_window=10 ** 6), full)


@pytest.mark.parametrize("W", [0, 3, 40, -1])
def test_chunk_window_matches_banded_reference(W):
    g = synth.rng(903, W + 2)
    Hq, Hkv, C, p0, D = 4, 2, 24, 30, 16
    q = synth.normal(g, (Hq, C, D)).astype(np.float64)
    K = synth.normal(g, (Hkv, p0 + C, D)).astype(np.float64)
    V = synth.normal(g, (Hkv, p0 + C, D)).astype(np.float64)
    got = oattn.chunk_attention(q, K, V, p0, left_window=W)
    for h in range(Hq):
        ref = _torch_banded(q[h], K[h // 2], V[h // 2], list(range(p0, p0 + C)), W, 1 / np.sqrt(D))
        np.testing.assert_allclose(got[h], ref, rtol=1e-12, atol=1e-12)
