"""The token loop of autoregressive generation.

Test infrastructure: a plain CPU model of the generation loop the library's
driver runs; only the tests, the smoke check and the benchmark's CPU
baseline use it.

"Persistent input/output feedback", section "Autoregressive generation": the
result is an INT64 ``[batch, prompt_length + generated_length]`` array that
includes the prompt; temperature 0 is greedy, a positive temperature samples
``softmax(logits / temperature)``, a seed makes the sampling repeatable;
generation stops at the token limit or once every row has emitted EOS, and a
finished row is padded with ``pad_token_id`` (EOS when not given); the prompt
is evaluated once and every later iteration consumes one new token; the final
logit position predicts the next token.

Readings (listed in the design doc):

* the row that emits EOS keeps that EOS token; every later column of the row
  is the pad token, and the row's input to later iterations is the pad token;
* without an EOS id generation always runs ``max_new_tokens`` iterations;
* the draws of one generation continue one SplitMix64 counter: iteration
  ``t`` samples row ``b``, token ``v`` with output number
  ``t * B * V + b * V + v + 1`` of the sequence seeded with ``seed``, i.e. the
  sampler of ``oracle.sampling`` seeded with ``seed + t * B * V * gamma``
  (mod 2^64).
"""
from __future__ import annotations

import numpy as np

from . import sampling

_MASK64 = (1 << 64) - 1


def step_seed(seed: int, step: int, B: int, V: int) -> int:
    """Seed of iteration ``step``: ``seed + step * B * V * gamma`` mod 2^64."""
    return (int(seed) + int(step) * int(B) * int(V) * int(sampling.GOLDEN_GAMMA)) & _MASK64


def generate(logits_fn, prompt, max_new_tokens: int, temperature: float = 0.0, seed: int = 0,
             eos_token_id=None, pad_token_id=None) -> np.ndarray:
    """Run the token loop.

    ``prompt`` is int64 ``[B, P]``; ``logits_fn(step, inputs)`` returns float
    logits ``[B, V]`` or ``[B, S, V]`` for ``inputs`` (the prompt at step 0,
    then ``[B]`` tokens).  Returns int64 ``[B, P + generated]``.
    """
    prompt = np.asarray(prompt, dtype=np.int64)
    B, P = prompt.shape
    pad = eos_token_id if pad_token_id is None else pad_token_id
    finished = np.zeros(B, dtype=bool)
    columns = [prompt]
    inputs = prompt
    for t in range(int(max_new_tokens)):
        logits = np.asarray(sampling.last_position(logits_fn(t, inputs)), dtype=np.float32)
        V = logits.shape[-1]
        ids = sampling.sample(logits, temperature, step_seed(seed, t, B, V))
        tok = np.where(finished, np.int64(pad if pad is not None else 0), ids) if finished.any() else ids
        if eos_token_id is not None:
            finished = finished | (tok == eos_token_id)
        columns.append(tok[:, None].astype(np.int64))
        inputs = tok
        if eos_token_id is not None and finished.all():
            break
    return np.concatenate(columns, axis=1)
