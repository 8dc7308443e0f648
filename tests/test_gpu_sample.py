"""GPU parity of sampling: greedy ids bit-exact against the oracle (ties to the
lowest index, every logits dtype, last position of [B, S, V]); temperature
draws repeatable, in agreement with the oracle up to float32 near-ties, and
distributed as softmax(x / T)."""
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
    if kind == "f64":       # digits below float32's precision: both sides round each logit to f32 first
        x64 = x32.astype(np.float64) * (1.0 + 1e-9 * np.sin(np.arange(x32.size)).reshape(x32.shape))
        return torch.from_numpy(x64).to(DEV), x64.astype(np.float32)
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
