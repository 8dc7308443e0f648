"""Pins of the oracle's exact widening and bf16 rounding (CPU only).

Pinned against PyTorch's dtype conversions (an independent implementation)
and against hand-worked ties and a case where rounding through float32 first
would give a different bf16.
"""
import numpy as np
import torch

import synth
from oracle import numeric


def test_widening_matches_torch():
    x = synth.normal(synth.rng(400), 5000, 3.0)
    b = torch.from_numpy(x).to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(numeric.bf16_to_f64(bits), b.to(torch.float64).numpy())
    h = x.astype(np.float16)
    assert np.array_equal(numeric.f16_to_f64(h.view(np.uint16)), torch.from_numpy(h).to(torch.float64).numpy())


def test_rounding_float32_values_matches_torch():
    x = synth.normal(synth.rng(401), 5000, 10.0)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(numeric.f64_to_bf16(x.astype(np.float64)), want)


def test_rounding_is_single_step_and_ties_to_even():
    one = 0x3F80
    assert numeric.f64_to_bf16(np.array([1 + 2 ** -8]))[0] == one            # tie -> even (1.0)
    assert numeric.f64_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == one + 2    # tie -> even (1 + 2^-6)
    # just above a tie: direct rounding goes up; rounding through float32 first would land on the tie
    assert numeric.f64_to_bf16(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == one + 1
    assert numeric.f64_to_bf16(np.array([-(1 + 2 ** -8 + 2 ** -40)]))[0] == 0x8000 | (one + 1)
