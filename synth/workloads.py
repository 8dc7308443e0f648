"""The decode workloads, as seeded synthetic input recipes.

Each workload fixes shapes, value distributions and structure (length mix,
page order); tensors are drawn from ``synth.rng(seed, stream...)`` so that
one batch row can be regenerated alone.  Nothing here computes any part of
the decode step.

Workloads (sizes as used by the bench and the full-size parity tests;
the tests also use scaled-down instances of the same recipes):

* ``tiny``     -- 1 row, 1 head, D = 4, float32, capacity 16; Q/K/V ~ U[-1, 1];
                  a 1-token prompt then decode steps appending one K/V row each.
* ``contig``   -- contiguous bf16 cache [8, 8, 4096, 128], 32 query heads;
                  initial valid lengths ~ U{512..4064} (so 32 appends fit);
                  Q/K/V ~ N(0, 1); 32 decode steps of one token.
* ``paged``    -- bf16 pool of 65536 blocks of 16 tokens, 64 rows, 32/8 heads,
                  D = 128, lengths lognormal(mu=8, sigma=1) clipped to
                  [16, 32768], pages handed out in a seeded random order.
* ``paged32k`` -- the same pool with 32 rows of exactly 32768 tokens (the
                  pool is then exactly full).
* ``int4``     -- INT4 pool of 16384 blocks of 16 tokens, 32 rows of 8192
                  tokens, 32/8 heads, D = 128; codes ~ U{0..15}; per 32-element
                  block fp16 scale ~ U[0.01, 0.1] and zero point ~ U{0..15};
                  q ~ N(0, 1) float32.
* ``mixed32k`` -- the paged32k shapes (32 rows x 32768 tokens, a full pool
                  of 65536 pages of 16) appended with the pages' length-threshold
                  format selector: the first 1024 tokens of a row in dense BF16
                  pages, the rest with INT8 keys (scale 0.01, zero point 0) and
                  UINT4 values (scale 0.25, zero point 8); K ~ N(0, 0.3) and
                  V ~ N(0, 0.5) so those scales rarely saturate; q ~ N(0, 1).
* ``qwen``     -- 128 rows, 16/8 heads, D = 128, lengths ~ U{1024..16384},
                  bf16 pages of 16 tokens; a 512-token chunk; logits
                  [128, 151936] ~ N(0, 3) float32 for sampling.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import f16_bits, f32_to_bf16_bits, lognormal_lengths, normal, permutation, rng, uniform

SEEDS = {"tiny": 0, "contig": 1, "paged": 2, "paged32k": 3, "int4": 4, "qwen": 5, "mixed32k": 6}


@dataclass
class PagedSpec:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    maxb: int
    lengths: np.ndarray                     # int32[B] valid tokens per row
    order: np.ndarray = field(repr=False)   # int32[NB] page hand-out order

    def pages(self, b: int) -> int:
        return -(-int(self.lengths[b]) // self.bs)

    # logical content of row b, [Hkv, L_b, D]
    def k_row_bf16(self, b: int, length: int | None = None) -> np.ndarray:
        L = int(self.lengths[b]) if length is None else length
        return f32_to_bf16_bits(normal(rng(self.seed, 2, b), (self.Hkv, L, self.D)))

    def v_row_bf16(self, b: int, length: int | None = None) -> np.ndarray:
        L = int(self.lengths[b]) if length is None else length
        return f32_to_bf16_bits(normal(rng(self.seed, 3, b), (self.Hkv, L, self.D)))

    def q_bf16(self) -> np.ndarray:
        return f32_to_bf16_bits(normal(rng(self.seed, 4), (self.B, self.Hq, self.D)))


def tiny(seed: int = SEEDS["tiny"], steps: int = 17, D: int = 4):
    g = rng(seed, 1)
    f = lambda: uniform(g, (steps, 1, D), -1.0, 1.0)
    q, k, v = f(), f(), f()
    return {"q": q, "k": k, "v": v, "capacity": 16}


def contig(seed: int = SEEDS["contig"], B: int = 8, Hq: int = 32, Hkv: int = 8, D: int = 128,
           cap: int = 4096, steps: int = 32):
    """Initial lengths ~ U{512 .. cap - steps} scaled to the capacity; per-row caches and per-step q/k/v."""
    lo = min(512, cap // 8)
    lengths = rng(seed, 0).integers(lo, cap - steps + 1, size=B).astype(np.int32)
    return {"B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "cap": cap, "steps": steps, "lengths": lengths, "seed": seed}


def contig_cache_row(seed: int, which: int, b: int, Hkv: int, L: int, D: int) -> np.ndarray:
    """Initial K (which=1) or V (which=2) rows of batch row b, bf16 bits [Hkv, L, D]."""
    return f32_to_bf16_bits(normal(rng(seed, which, b), (Hkv, L, D)))


def contig_step(seed: int, step: int, B: int, Hq: int, Hkv: int, D: int):
    """q [B, Hq, D], k/v [B, Hkv, 1, D] of one decode step, bf16 bits."""
    q = f32_to_bf16_bits(normal(rng(seed, 3, step), (B, Hq, D)))
    k = f32_to_bf16_bits(normal(rng(seed, 4, step), (B, Hkv, 1, D)))
    v = f32_to_bf16_bits(normal(rng(seed, 5, step), (B, Hkv, 1, D)))
    return q, k, v


def paged(seed: int = SEEDS["paged"], B: int = 64, Hq: int = 32, Hkv: int = 8, D: int = 128, bs: int = 16,
          NB: int = 65536, max_len: int = 32768) -> PagedSpec:
    lengths = lognormal_lengths(rng(seed, 0), B, 8.0, 1.0, 16, max_len)
    return PagedSpec("paged", seed, B, Hq, Hkv, D, bs, NB, -(-max_len // bs), lengths, permutation(rng(seed, 1), NB))


def paged32k(seed: int = SEEDS["paged32k"], B: int = 32, L: int = 32768, Hq: int = 32, Hkv: int = 8,
             D: int = 128, bs: int = 16, NB: int = 65536) -> PagedSpec:
    lengths = np.full(B, L, dtype=np.int32)
    return PagedSpec("paged32k", seed, B, Hq, Hkv, D, bs, NB, -(-L // bs), lengths, permutation(rng(seed, 1), NB))


@dataclass
class Int4Spec:
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    maxb: int
    lengths: np.ndarray
    order: np.ndarray = field(repr=False)

    def codes_row(self, b: int) -> np.ndarray:
        """uint8 [Hkv, L, D/2]: two U{0..15} codes per byte."""
        L = int(self.lengths[b])
        return rng(self.seed, 2, b).integers(0, 256, size=(self.Hkv, L, self.D // 2), dtype=np.uint8)

    def params_row(self, b: int, stream: int = 3) -> np.ndarray:
        """fp16 bits [Hkv, L, D/32, 2]: scale ~ U[0.01, 0.1], zero point ~ U{0..15}."""
        L = int(self.lengths[b])
        g = rng(self.seed, stream, b)
        shape = (self.Hkv, L, self.D // 32)
        out = np.empty(shape + (2,), dtype=np.uint16)
        out[..., 0] = f16_bits(uniform(g, shape, 0.01, 0.1))
        out[..., 1] = f16_bits(g.integers(0, 16, size=shape).astype(np.float32))
        return out

    def v_codes_row(self, b: int) -> np.ndarray:
        L = int(self.lengths[b])
        return rng(self.seed, 4, b).integers(0, 256, size=(self.Hkv, L, self.D // 2), dtype=np.uint8)

    def v_params_row(self, b: int) -> np.ndarray:
        return self.params_row(b, stream=5)

    def q_f32(self) -> np.ndarray:
        return normal(rng(self.seed, 6), (self.B, self.Hq, self.D))


def int4(seed: int = SEEDS["int4"], B: int = 32, L: int = 8192, Hq: int = 32, Hkv: int = 8, D: int = 128,
         bs: int = 16, NB: int = 16384) -> Int4Spec:
    lengths = np.full(B, L, dtype=np.int32)
    return Int4Spec(seed, B, Hq, Hkv, D, bs, NB, -(-L // bs), lengths, permutation(rng(seed, 1), NB))


@dataclass
class MixedSpec:
    """Shapes, selector and value distributions of a mixed-format pool."""
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    maxb: int
    L: int
    threshold: int                 # tokens kept in the early formats
    early: tuple                   # ((storage, scale, zero_point) of K, of V)
    late: tuple
    k_sigma: float
    v_sigma: float
    order: np.ndarray = field(repr=False)


def mixed32k(seed: int = SEEDS["mixed32k"], B: int = 32, L: int = 32768, Hq: int = 32, Hkv: int = 8,
             D: int = 128, bs: int = 16, NB: int = 65536) -> MixedSpec:
    return MixedSpec(seed, B, Hq, Hkv, D, bs, NB, -(-L // bs), L, 1024, (("BF16", 1.0, 0), ("BF16", 1.0, 0)),
                     (("INT8", 0.01, 0), ("UINT4", 0.25, 8)), 0.3, 0.5, permutation(rng(seed, 1), NB))


def qwen(seed: int = SEEDS["qwen"], B: int = 128, Hq: int = 16, Hkv: int = 8, D: int = 128, bs: int = 16,
         lo: int = 1024, hi: int = 16384, chunk: int = 512, vocab: int = 151936):
    lengths = rng(seed, 0).integers(lo, hi + 1, size=B).astype(np.int32)
    NB = int(sum(-(-(int(x) + chunk) // bs) for x in lengths))
    return {"seed": seed, "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "bs": bs, "lengths": lengths, "chunk": chunk,
            "vocab": vocab, "NB": NB, "maxb": -(-(hi + chunk) // bs), "order": permutation(rng(seed, 1), NB)}


def logits(seed: int, B: int, V: int, sigma: float = 3.0) -> np.ndarray:
    return normal(rng(seed, 9), (B, V), sigma)
