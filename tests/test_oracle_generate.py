"""Pins of the oracle's generation loop (CPU only): a hand-derived table
example (tests/golden/generate_table_example.json) for EOS, padding, the
early stop and the token limit, and the SplitMix64 counter that the draws of
one generation continue across iterations."""
import json
import os

import numpy as np
import pytest

from oracle import generate as ogen
from oracle import sampling

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "generate_table_example.json")


def _table_fn(table):
    table = np.asarray(table, np.float32)

    def fn(step, inputs):
        inputs = np.asarray(inputs)
        last = inputs[:, -1] if inputs.ndim == 2 else inputs
        return table[last]
    return fn


@pytest.mark.parametrize("case", range(6))
def test_hand_derived_table_example(case):
    g = json.load(open(GOLDEN))
    c = g["cases"][case]
    rows = c.get("rows", [0, 1, 2])
    prompt = np.asarray(c.get("prompt", g["prompt"]), np.int64)[rows if "prompt" not in c else slice(None)]
    eos = c.get("eos", g["eos_token_id"])
    got = ogen.generate(_table_fn(g["table"]), prompt, c["max_new_tokens"], 0.0, 0, eos, c["pad_token_id"])
    assert got.dtype == np.int64
    assert got.tolist() == c["expected"], c["note"]


def test_draws_continue_one_counter():
    """Iteration t, row b, token v draws output number t*B*V + b*V + v + 1 of SplitMix64(seed)."""
    seed, B, V = 0x1234_5678_9ABC_DEF0, 3, 7
    for t in range(4):
        for b in range(B):
            u = sampling.uniforms(ogen.step_seed(seed, t, B, V), b, V)
            k = np.arange(V, dtype=np.uint64) + np.uint64(t * B * V + b * V + 1)
            h = sampling.splitmix64_outputs(seed, k)
            assert np.array_equal(u, ((h >> np.uint64(40)) | np.uint64(1)).astype(np.float64) * 2.0 ** -24)


def test_sampled_generation_is_repeatable_and_seeded():
    g = json.load(open(GOLDEN))
    fn = _table_fn(np.asarray(g["table"], np.float32) * 0.3)
    prompt = np.asarray(g["prompt"], np.int64)
    a = ogen.generate(fn, prompt, 12, 0.8, 7, None, None)
    b = ogen.generate(fn, prompt, 12, 0.8, 7, None, None)
    c = ogen.generate(fn, prompt, 12, 0.8, 8, None, None)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (3, 14) and np.array_equal(a[:, :2], prompt)
    # every new token of a row that emitted EOS is the pad token
    e = ogen.generate(fn, prompt, 12, 0.8, 7, 2, 5)
    for row in e:
        hit = np.nonzero(row[2:] == 2)[0]
        if hit.size:
            assert (row[2 + hit[0] + 1:] == 5).all()


def test_finished_rows_feed_the_pad_token():
    """After a row emits EOS the model sees the pad token for that row."""
    g = json.load(open(GOLDEN))
    seen = []
    base = _table_fn(g["table"])

    def fn(step, inputs):
        seen.append(np.array(inputs, copy=True))
        return base(step, inputs)
    ogen.generate(fn, np.asarray(g["prompt"], np.int64), 5, 0.0, 0, 2, 0)
    # row 2 emits EOS at iteration 1 (its next input is that EOS), then pads; row 0 at iteration 2
    assert seen[2].tolist() == [3, 4, 2] and seen[3].tolist() == [2, 5, 0] and seen[4].tolist() == [0, 4, 0]
