"""The parity bound the chunk-attention tests use (bf16 probabilities in P.V, bf16 output) is checked here
on the CPU: an output computed with those two roundings passes it, and the structural mistakes it is meant
to catch (a key dropped, a key counted twice, a wrong softmax scale) fail it on short rows."""
import numpy as np
import pytest

import synth
from oracle import attention as oattn
from oracle import numeric as onum
from tests.gpu_util import assert_bf16_pv_bound


def _bf16(x):
    return onum.bf16_to_f64(synth.f32_to_bf16_bits(np.asarray(x, np.float32)))


def _rounded_output(q, K, V, scale, keep=None, extra=None):
    """A P.V output with the probabilities rounded to bf16 and the result rounded to bf16; `keep` drops
    keys from the numerator and denominator, `extra` counts one key twice."""
    s = K @ q * scale
    p = np.exp(s - s.max())
    if keep is not None:
        p = p * keep
    num = _bf16(p) @ V
    den = p.sum()
    if extra is not None:
        num = num + _bf16(p[extra]) * V[extra]
        den = den + p[extra]
    return _bf16(num / den)


@pytest.mark.parametrize("n", [3, 17, 64, 100])
def test_two_roundings_stay_inside_the_bound(n):
    g = synth.rng(4242, n)
    D = 128
    for _ in range(20):
        q = _bf16(synth.normal(g, (D,)))
        K = _bf16(synth.normal(g, (n, D)))
        V = _bf16(synth.normal(g, (n, D)))
        scale = 1 / np.sqrt(D)
        ref = oattn.attend(q, K, V, scale)
        assert_bf16_pv_bound(_rounded_output(q, K, V, scale), ref, K @ q * scale, V)


@pytest.mark.parametrize("mistake", ["drop", "twice", "scale"])
def test_structural_mistakes_break_the_bound(mistake):
    """Over 50 short rows (n = 8..40 keys) each mistake must fail the bound on most rows."""
    g = synth.rng(4343, ["drop", "twice", "scale"].index(mistake))
    D, caught, rows = 128, 0, 50
    for _ in range(rows):
        n = int(g.integers(8, 41))
        q = _bf16(synth.normal(g, (D,)))
        K = _bf16(synth.normal(g, (n, D)))
        V = _bf16(synth.normal(g, (n, D)))
        scale = 1 / np.sqrt(D)
        ref = oattn.attend(q, K, V, scale)
        k = int(g.integers(0, n))
        if mistake == "drop":
            keep = np.ones(n)
            keep[k] = 0.0
            got = _rounded_output(q, K, V, scale, keep=keep)
        elif mistake == "twice":
            got = _rounded_output(q, K, V, scale, extra=k)
        else:
            got = _rounded_output(q, K, V, scale * 1.1)
        try:
            assert_bf16_pv_bound(got, ref, K @ q * scale, V)
        except AssertionError:
            caught += 1
    assert caught >= 0.9 * rows, caught
