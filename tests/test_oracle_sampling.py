"""Pins of the oracle's greedy and temperature sampling (CPU only).

SplitMix64 is pinned to its published outputs and to a sequential
implementation; greedy to a brute-force loop with planted ties; the
Gumbel-max draw to the law softmax(x / T) by a chi-square test over seeds,
and to greedy as T -> 0+.  DOUBLE logits: greedy resolves pairs closer than
one float32 ulp, and the float64 draw follows softmax(x / T) too.  Non-finite
logits: a brute-force loop with numpy's argmax order (NaN above every number,
first one wins; an all -inf row gives index 0).
"""
import numpy as np
import pytest
from scipy.stats import chisquare

import synth
from oracle import sampling

MASK = (1 << 64) - 1


def _splitmix_sequential(seed, n):
    """Textbook SplitMix64 next(): advance the state by the golden gamma, then mix."""
    state, out = seed & MASK, []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        out.append(z ^ (z >> 31))
    return out


def test_splitmix64_published_outputs():
    # first outputs of the reference generator started from state 0 and from state 1234567
    assert [int(x) for x in sampling.splitmix64_outputs(0, np.arange(1, 4))] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [int(x) for x in sampling.splitmix64_outputs(1234567, np.arange(1, 6))] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_counter_form_equals_the_sequential_stream():
    seed = 0xDEADBEEF12345678
    assert [int(x) for x in sampling.splitmix64_outputs(seed, np.arange(1, 65))] == _splitmix_sequential(seed, 64)


def test_uniforms_are_odd_multiples_of_2_pow_minus_24_inside_0_1():
    u = sampling.uniforms(7, 3, 5000)
    m = u * 2 ** 24
    assert np.array_equal(m, np.round(m)) and (m.astype(np.int64) % 2 == 1).all()
    assert (u > 0).all() and (u < 1).all()
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    h = np.array(_splitmix_sequential(7, 3 * 5000 + 5000)[3 * 5000:], dtype=np.uint64)
    assert np.array_equal(u, ((h >> np.uint64(40)) | np.uint64(1)).astype(np.float64) / 2 ** 24)


def test_greedy_matches_brute_force_with_ties_to_lowest():
    g = synth.rng(300)
    x = np.round(synth.normal(g, (20, 50)) * 2) / 2          # coarse values: many ties
    for b in range(20):
        best = 0
        for v in range(1, 50):
            if x[b, v] > x[b, best]:
                best = v
        assert sampling.greedy(x)[b] == best
    x3 = np.zeros((2, 3, 4), np.float32)
    x3[:, -1, 2] = 1
    x3[:, 0, 1] = 5                                        # earlier positions are ignored
    assert sampling.greedy(x3).tolist() == [2, 2]


def test_gumbel_draws_follow_softmax_over_temperature():
    x = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 0.9, 1.5], np.float32)
    T = 0.7
    n = 40000
    counts = np.zeros(8)
    for seed in range(n):
        counts[sampling.sample(x[None], T, seed)[0]] += 1
    y = (x * sampling.inv_temperature(T)).astype(np.float64)
    p = np.exp(y - y.max())
    p /= p.sum()
    assert chisquare(counts, p * n).pvalue > 1e-3


def test_draws_are_repeatable_and_rows_use_their_own_counters():
    x = synth.normal(synth.rng(301), (6, 300), 3.0)
    a = sampling.sample(x, 0.7, 5)
    assert np.array_equal(a, sampling.sample(x, 0.7, 5))
    assert not np.array_equal(a, sampling.sample(x, 0.7, 6))
    same = np.tile(x[:1], (6, 1))
    assert len(set(sampling.sample(same, 0.7, 5).tolist())) > 1


def test_small_temperature_is_greedy_when_the_gap_is_large():
    x = synth.normal(synth.rng(302), (10, 1000), 3.0)
    top = np.argmax(x, axis=1)
    x[np.arange(10), top] += 1.0                          # top-2 gap >= 1
    assert np.array_equal(sampling.sample(x, 1e-3, 9), sampling.greedy(x))


@pytest.mark.parametrize("T", [-0.5, float("nan")])
def test_bad_temperature_is_rejected(T):
    with pytest.raises(ValueError):
        sampling.sample(np.zeros((1, 4), np.float32), T, 0)


def _brute_argmax(row):
    """First index of the highest-ranked value, NaN ranking above every number."""
    best = 0
    for v in range(1, len(row)):
        a, b = row[v], row[best]
        if (a != a and b == b) or (a == a and b == b and a > b):
            best = v
    return best


def test_greedy_over_float64_resolves_pairs_below_float32_resolution():
    g = synth.rng(303)
    x = synth.normal(g, (8, 300), 3.0).astype(np.float64)
    for b in range(8):
        top = float(x[b].max()) + 1.0
        i, j = sorted(g.choice(300, size=2, replace=False))
        hi = np.nextafter(top, np.inf)                 # one float64 ulp above: equal in float32
        assert np.float32(hi) == np.float32(top)
        x[b, i], x[b, j] = (top, hi) if b % 2 else (hi, top)
        assert sampling.greedy(x)[b] == (j if b % 2 else i)
        assert sampling.greedy(x)[b] == _brute_argmax(x[b])
    # the float32 view of the same rows ties, so it takes the lower index
    assert np.array_equal(sampling.greedy(x.astype(np.float32)),
                          [_brute_argmax(r) for r in x.astype(np.float32)])


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_non_finite_logits_follow_argmax_order(dtype):
    x = synth.normal(synth.rng(304), (6, 40), 3.0).astype(dtype)
    x[0, :] = -np.inf                                  # all -inf: index 0
    x[1, 7], x[1, 30] = np.nan, np.nan                 # first NaN wins
    x[2, 5], x[2, 9] = np.inf, np.inf                  # +inf ties: lowest index
    x[3, :] = np.nan
    x[4, 3], x[4, 20] = -np.inf, np.nan
    x[5, 11] = -np.nan                                 # a NaN with the sign bit set
    want = [_brute_argmax(r) for r in x]
    assert want == [0, 7, 5, 0, 20, 11]
    assert sampling.greedy(x).tolist() == want
    # a draw keeps the order of its perturbed scores: NaN and +inf rows stay put
    got = sampling.sample(x, 0.7, 3)
    assert got[0] == 0 and got[1] == 7 and got[2] == 5 and got[3] == 0 and got[4] == 20 and got[5] == 11


def test_float64_draws_follow_softmax_over_temperature():
    x = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 0.9, 1.5], np.float64) + 1e-12
    T = 0.7
    n = 40000
    counts = np.zeros(8)
    for seed in range(n):
        counts[sampling.sample(x[None], T, seed)[0]] += 1
    y = x / float(np.float32(T))
    p = np.exp(y - y.max())
    p /= p.sum()
    assert chisquare(counts, p * n).pvalue > 1e-3


def test_float64_small_temperature_is_float64_greedy():
    x = synth.normal(synth.rng(305), (6, 500), 3.0).astype(np.float64)
    top = np.argmax(x, axis=1)
    x[np.arange(6), top] += 1.0
    assert np.array_equal(sampling.sample(x, 1e-3, 4), sampling.greedy(x))
