"""GPU parity of sampling: greedy ids bit-exact against the oracle (ties to the
lowest index, every logits dtype, DOUBLE logits compared as float64 values,
non-finite logits, last position of [B, S, V]); temperature draws repeatable,
in agreement with the oracle up to float32 near-ties, and distributed as
softmax(x / T)."""
import numpy as np
import pytest
import torch
from scipy.stats import chisquare

import place_persistent_kv_amd as pkv
import synth
from oracle import numeric as onum
from oracle import sampling as osamp
from tests.gpu_util import DEV, require_gpu, workspace

pytestmark = pytest.mark.gpu


def _logits_dev(x32, kind):
    if kind == "f32":
        return torch.from_numpy(x32).to(DEV), x32
    if kind == "f64":       # digits below float32's precision; the oracle gets the float64 values
        x64 = x32.astype(np.float64) * (1.0 + 1e-9 * np.sin(np.arange(x32.size)).reshape(x32.shape))
        return torch.from_numpy(x64).to(DEV), x64
    if kind == "bf16":
        bits = synth.f32_to_bf16_bits(x32)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16), onum.bf16_to_f64(bits).astype(np.float32)
    bits = synth.f16_bits(x32)
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.float16), onum.f16_to_f64(bits).astype(np.float32)


def _run(logits, T, seed):
    B = logits.shape[0]
    V = logits.shape[-1]
    ids = torch.full((B,), -1, dtype=torch.int64, device=DEV)
    pkv.sample(logits, T, seed, ids, workspace(pkv.sample_workspace_size(B, V)))
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("kind", ["f32", "bf16", "f16", "f64"])
@pytest.mark.parametrize("B,V", [(5, 1000), (3, 151936), (130, 4097)])
def test_greedy_is_bit_exact(kind, B, V):
    require_gpu()
    g = synth.rng(800, B, V)
    x = synth.normal(g, (B, V), 3.0)
    top = x.max(axis=1, keepdims=True)
    for b in range(B):                                   # planted ties at the maximum
        x[b, g.integers(0, V, size=3)] = top[b, 0]
    dev, xh = _logits_dev(x, kind)
    assert np.array_equal(_run(dev, 0.0, 0), osamp.greedy(xh))


@pytest.mark.parametrize("B,V", [(3, 151936), (40, 9000)])
def test_float64_greedy_resolves_sub_float32_near_ties(B, V):
    """Pairs one float64 ulp apart (equal once rounded to float32) planted inside a thread's run, across
    vector, thread and chunk boundaries (chunks are whole multiples of 1024 logits); the larger one must win."""
    require_gpu()
    g = synth.rng(803, B, V)
    x = synth.normal(g, (B, V), 3.0).astype(np.float64)
    spots = [(0, 1), (1, 2), (1023, 1024), (4095, 4096), (2047, 6000), (8191, 8192), (V - 2, V - 1), (5, V - 1)]
    for b in range(B):
        i, j = spots[b % len(spots)]
        top = float(x[b].max()) + 0.5
        hi = np.nextafter(top, np.inf)
        assert np.float32(hi) == np.float32(top)
        x[b, i], x[b, j] = (top, hi) if (b // len(spots)) % 2 == 0 else (hi, top)
    want = osamp.greedy(x)
    assert not np.array_equal(want, osamp.greedy(x.astype(np.float32)))   # float32 rounding would change ids
    assert np.array_equal(_run(torch.from_numpy(x).to(DEV), 0.0, 0), want)


@pytest.mark.parametrize("kind", ["f32", "bf16", "f16", "f64"])
@pytest.mark.parametrize("T", [0.0, 0.7])
def test_non_finite_logits(kind, T):
    """numpy's argmax order: NaN above every number (first NaN wins), all -inf rows give index 0,
    +inf ties go to the lowest index; every id lies inside the vocabulary."""
    require_gpu()
    B, V = 8, 9000
    x = synth.normal(synth.rng(804), (B, V), 3.0)
    x[0, :] = -np.inf
    x[1, 4097], x[1, 8000] = np.nan, np.nan
    x[2, 3], x[2, 6000] = np.inf, np.inf
    x[3, :] = np.nan
    x[4, 10], x[4, 5000] = -np.inf, np.nan
    x[5, 1] = -np.nan
    x[6, :4096] = -np.inf                              # a whole chunk of -inf before finite values
    dev, xh = _logits_dev(x, kind)
    got = _run(dev, T, 9)
    assert ((got >= 0) & (got < V)).all()
    assert got[:6].tolist() == [0, 4097, 3, 0, 5000, 1]
    if T == 0.0:
        assert np.array_equal(got, osamp.greedy(xh))
    else:
        assert np.array_equal(got[:6], osamp.sample(xh, T, 9)[:6])


def test_greedy_uses_the_last_position():
    require_gpu()
    x = synth.normal(synth.rng(801), (4, 3, 777))
    dev, xh = _logits_dev(x, "f32")
    assert np.array_equal(_run(dev, 0.0, 0), osamp.greedy(xh))


@pytest.mark.parametrize("kind", ["f32", "bf16", "f64"])
def test_temperature_draws_agree_with_the_oracle(kind):
    require_gpu()
    B, V, T = 64, 151936, 0.7
    dev, xh = _logits_dev(synth.normal(synth.rng(802), (B, V), 3.0), kind)
    for seed in (5, 6):
        got = _run(dev, T, seed)
        assert np.array_equal(got, _run(dev, T, seed))               # repeatable
        want = osamp.sample(xh, T, seed)
        for b in np.nonzero(got != want)[0]:
            sc = osamp.gumbel_scores(xh[b], T, seed, b)
            # a disagreement must be a float32 near-tie between the two candidates
            assert abs(sc[got[b]] - sc[want[b]]) <= 1e-5 * max(1.0, abs(sc[want[b]])), b
        assert (got == want).mean() >= 0.99


def test_temperature_draws_follow_softmax():
    require_gpu()
    V, T, rows = 8, 0.7, 40000
    x = np.array([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 0.9, 1.5], np.float32)
    dev = torch.from_numpy(np.tile(x, (rows, 1))).to(DEV)        # independent counters per row
    ids = _run(dev, T, 123)
    counts = np.bincount(ids, minlength=V)
    y = (x * osamp.inv_temperature(T)).astype(np.float64)
    p = np.exp(y - y.max())
    p /= p.sum()
    assert chisquare(counts, p * rows).pvalue > 1e-3
