"""CPU oracle for the persistent-KV decode step -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU statement of what the
decode step computes, written in numpy with float64 arithmetic.  It exists to
check the HIP library; it is not part of the product path.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library and its Python binding never import it, and it
never imports them: the two share no code.  The only module both sides use is
``synth`` (seeded input generators, which holds none of the method's
arithmetic).

Sources (the onnx-light documentation pages):

* "Persistent input/output feedback" (how-to page) -- sections "Contiguous CPU
  Attention feedback", "Opt-in storage auditing through runtime events",
  "Autoregressive generation" and "Optional heterogeneous paged KV";
* "Custom, quantized, and persistent values" (design record) -- sections
  "Struct types and byte-encodable layouts", "One element type, many payload
  lengths", "Quantization examples", "Codebook quantization through a shared
  subtype" and "Persistent state from model inputs and outputs";
* "Mutable execution cache" (design proposal) -- sections "Value model",
  "ShapesContext", "Required alias", "Model example", "Heterogeneous paged
  cache", "Runtime contract", "Existing implementations" and "Memory planning".

Modules:

* ``numeric``   -- exact widening of bf16/fp16 bit patterns, rounding to bf16;
* ``cache``     -- in-place cache update, page pool and paged mapping/gather;
* ``attention`` -- decode attention, split partials and their merge, causal
  chunk attention;
* ``affine``    -- LSB-first code packing, affine decode, INT4 quantise;
* ``sampling``  -- SplitMix64, greedy and Gumbel-max temperature sampling;
* ``accounting``-- retained/append/fallback byte counts;
* ``stateless`` -- stateful (in place) vs stateless (full prefix) decode loops.

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, library routines or brute force (see each test).
"""

from . import numeric, cache, attention, affine, sampling, accounting, stateless  # noqa: F401

__all__ = ["numeric", "cache", "attention", "affine", "sampling", "accounting", "stateless"]
