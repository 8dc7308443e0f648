"""Mixed-format paged K/V: per-page storage, append, selected-page conversion, decode.

Test infrastructure: a plain, slow CPU model of what the library's mixed-format
pages compute.  Only the tests, the smoke check and the benchmark's CPU
baseline use it; it shares no code with the library.

What the pages fix:

* "Persistent input/output feedback", "Optional heterogeneous paged KV": each
  append chooses the storage of the pages it creates (a format selector may
  pick K and V formats independently, from the retained length); the choice
  is stored with every new page and earlier pages are never converted by an
  append; new pages may be dense or affine INT8, UINT8, INT4, UINT4, INT2 or
  UINT2; the affine append uses one scalar scale and zero point; quantisation
  rounds ties to even and saturates to the code range; attention reads only
  valid, visible tokens.
* Same page, "Selected-block quantization": converting selected blocks
  decodes each block's dense or affine payload and re-encodes its valid
  prefix in the requested format, K and V independently; rows past the valid
  prefix become the destination's encoding of zero and are not read; a dense
  target ignores scale and zero point; indices and parameters are all checked
  before anything is written.
* "Custom, quantized, and persistent values", "Struct types and byte-encodable
  layouts": codes are packed least-significant bits first (signed codes in
  two's complement); "Quantization examples": a code is worth
  ``(code - zero_point) * scale``.

Readings where the pages leave a step open:

* Page storage: each (page, head) owns a slot of ``block_size * D * 2`` bytes
  (a dense 16-bit page), and the page's rows are packed one after another
  from the start of the slot: row ``t`` starts at byte ``t * D * bits / 8``.
  A pool whose pages are all BF16 is byte for byte a bf16 pool ``[NB, H, bs, D]``.
* Dense storages are BF16 and F16 (the pages' dense BFLOAT16 and FLOAT16
  alternatives); a dense FLOAT page would need a wider slot and is not modelled.
* A page takes the format of the append that writes its first slot; an append
  that continues a partly filled page encodes its rows in that page's stored
  format (partial pages are filled in place, as in the plain paged update).
* A conversion decodes ``(code - zero_point) * scale`` with one float32
  multiply (the pages' scale type is FLOAT) and re-encodes that float32 value
  (affine: float32 divide; dense: nearest-even BF16 / F16).  Bytes of a slot
  past the new format's ``block_size`` rows are left as they were.
* Attention uses the exact decoded values, and the token appended by the step
  is read back as stored (the append runs first): the pages' statistics
  example counts the decoded bytes of the appended tokens as well.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import attention
from .affine import CODE_RANGE, affine_quantize, pack_codes, unpack_codes
from .numeric import bf16_to_f64, f16_to_f64, f64_to_bf16

STORAGES = ("BF16", "F16", "INT8", "UINT8", "INT4", "UINT4", "INT2", "UINT2")
DENSE = ("BF16", "F16")


def bits(storage: str) -> int:
    """Bits per element of a storage."""
    return 16 if storage in DENSE else CODE_RANGE[storage][2]


def row_bytes(storage: str, D: int) -> int:
    """Bytes of one stored row of ``D`` elements (D * bits a multiple of 8)."""
    nbits = int(D) * bits(storage)
    if nbits % 8:
        raise ValueError("a stored row must be a whole number of bytes")
    return nbits // 8


@dataclass(frozen=True)
class Format:
    """Storage of a page's K or V rows: dense BF16 / F16, or affine with a
    float32 ``scale`` and an integer ``zero_point`` in the code range."""
    storage: str
    scale: float = 1.0
    zero_point: int = 0

    def check(self) -> None:
        if self.storage not in STORAGES:
            raise ValueError(f"unknown storage {self.storage!r}")
        if self.storage in DENSE:
            return
        s = np.float32(self.scale)
        if not (np.isfinite(s) and s > 0):
            raise ValueError("affine scale must be positive and finite")
        lo, hi, _ = CODE_RANGE[self.storage]
        if int(self.zero_point) != self.zero_point or not lo <= self.zero_point <= hi:
            raise ValueError(f"zero point must be an integer in [{lo}, {hi}]")

    @property
    def affine(self) -> bool:
        return self.storage not in DENSE


def encode_rows(x32: np.ndarray, fmt: Format) -> np.ndarray:
    """Encode float32 rows ``[..., D]`` as stored bytes ``[..., row_bytes]``."""
    x32 = np.asarray(x32, dtype=np.float32)
    if fmt.storage == "BF16":
        return f64_to_bf16(x32.astype(np.float64)).astype("<u2").view(np.uint8)
    if fmt.storage == "F16":
        return x32.astype("<f2").view(np.uint8)           # nearest-even
    codes = affine_quantize(x32, fmt.scale, fmt.zero_point, fmt.storage)
    return pack_codes(codes, bits(fmt.storage))


def _codes(payload: np.ndarray, fmt: Format, D: int) -> np.ndarray:
    return unpack_codes(payload, bits(fmt.storage), D, signed=fmt.storage.startswith("INT"))


def decode_rows_f32(payload: np.ndarray, fmt: Format, D: int) -> np.ndarray:
    """Stored bytes ``[..., row_bytes]`` -> float32 ``[..., D]``; affine codes
    as one float32 multiply ``(code - zero_point) * scale``."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    if fmt.storage == "BF16":
        return bf16_to_f64(payload.view("<u2")).astype(np.float32)
    if fmt.storage == "F16":
        return payload.view("<f2").astype(np.float32)
    c = (_codes(payload, fmt, D) - int(fmt.zero_point)).astype(np.float32)
    return c * np.float32(fmt.scale)


def decode_rows_exact(payload: np.ndarray, fmt: Format, D: int) -> np.ndarray:
    """Stored bytes -> exact float64 values (an affine product of a code
    difference below 2^9 and a float32 scale is exact in float64)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    if fmt.storage == "BF16":
        return bf16_to_f64(payload.view("<u2"))
    if fmt.storage == "F16":
        return f16_to_f64(payload.view("<u2"))
    c = (_codes(payload, fmt, D) - int(fmt.zero_point)).astype(np.float64)
    return c * float(np.float32(fmt.scale))


class MixedPool:
    """K and V page slots of a fixed pool and the format of every page."""

    def __init__(self, num_blocks: int, heads: int, block_size: int, head_dim: int):
        self.NB, self.H, self.bs, self.D = num_blocks, heads, block_size, head_dim
        slot = block_size * head_dim * 2
        self.data = {"k": np.zeros((num_blocks, heads, slot), np.uint8),
                     "v": np.zeros((num_blocks, heads, slot), np.uint8)}
        self.fmt = {"k": [None] * num_blocks, "v": [None] * num_blocks}

    # -- rows of one page ------------------------------------------------------
    def _rows(self, which: str, page: int, fmt: Format) -> np.ndarray:
        """Rows ``[H, block_size, row_bytes]`` of a page in format ``fmt`` (a view)."""
        rb = row_bytes(fmt.storage, self.D)
        return self.data[which][page, :, :self.bs * rb].reshape(self.H, self.bs, rb)

    def append(self, page_table: np.ndarray, k_bf16: np.ndarray, v_bf16: np.ndarray, position,
               n: int, k_fmt: Format, v_fmt: Format) -> None:
        """Write ``n`` new tokens of every row (bf16 bit patterns ``[B, H, n, D]``)
        at ``position[b]``.  Pages whose first slot this append writes take
        ``k_fmt`` / ``v_fmt``; a partly filled page keeps its own format."""
        k_fmt.check()
        v_fmt.check()
        position = np.asarray(position, dtype=np.int64).reshape(-1)
        B = position.shape[0]
        for b in range(B):
            p0 = int(position[b])
            for j in range(p0 // self.bs, -(-(p0 + n) // self.bs)):
                page = int(page_table[b, j])
                if j * self.bs >= p0:              # the append writes the page's first slot
                    self.fmt["k"][page], self.fmt["v"][page] = k_fmt, v_fmt
                elif self.fmt["k"][page] is None:
                    raise ValueError(f"row {b}: partly filled page {page} has no stored format")
        for which, vals in (("k", k_bf16), ("v", v_bf16)):
            x = bf16_to_f64(vals).astype(np.float32)          # exact
            for b in range(B):
                p0 = int(position[b])
                for j in range(p0 // self.bs, -(-(p0 + n) // self.bs)):
                    page = int(page_table[b, j])
                    fmt = self.fmt[which][page]
                    lo, hi = max(p0, j * self.bs), min(p0 + n, (j + 1) * self.bs)
                    rows = self._rows(which, page, fmt)
                    rows[:, lo - j * self.bs:hi - j * self.bs] = encode_rows(x[b, :, lo - p0:hi - p0], fmt)

    def convert(self, pages, valid_rows, k_fmt: Format | None, v_fmt: Format | None) -> None:
        """Re-encode the first ``valid_rows[i]`` rows of page ``pages[i]`` (K to
        ``k_fmt``, V to ``v_fmt``; ``None`` keeps that tensor); later rows of the
        page become the new format's zero.  Everything is checked first."""
        pages = [int(p) for p in pages]
        valid_rows = [int(v) for v in valid_rows]
        if len(pages) != len(valid_rows):
            raise ValueError("one valid row count per page")
        if len(set(pages)) != len(pages):
            raise ValueError("page ids must be unique")
        for p, nv in zip(pages, valid_rows):
            if not 0 <= p < self.NB:
                raise ValueError(f"page {p} out of range")
            if not 0 <= nv <= self.bs:
                raise ValueError("valid rows must lie in [0, block_size]")
            if self.fmt["k"][p] is None:
                raise ValueError(f"page {p} holds no rows yet")
        for f in (k_fmt, v_fmt):
            if f is not None:
                f.check()
        for which, new in (("k", k_fmt), ("v", v_fmt)):
            if new is None:
                continue
            zero = encode_rows(np.zeros(self.D, np.float32), new)
            for p, nv in zip(pages, valid_rows):
                old = self.fmt[which][p]
                x = decode_rows_f32(self._rows(which, p, old)[:, :nv], old, self.D)
                out = self._rows(which, p, new)
                out[:, :nv] = encode_rows(x, new)
                out[:, nv:] = zero
                self.fmt[which][p] = new

    def gather(self, which: str, page_table_row: np.ndarray, length: int) -> np.ndarray:
        """Exact decoded logical rows ``[H, length, D]`` (float64) of one sequence."""
        out = np.empty((self.H, length, self.D), np.float64)
        for j in range(-(-length // self.bs)):
            page = int(page_table_row[j])
            fmt = self.fmt[which][page]
            n = min(self.bs, length - j * self.bs)
            out[:, j * self.bs:j * self.bs + n] = decode_rows_exact(self._rows(which, page, fmt)[:, :n], fmt, self.D)
        return out


def decode_attention(pool: MixedPool, q: np.ndarray, page_table: np.ndarray, lengths, scale=None,
                     left_window: int = -1) -> np.ndarray:
    """Single-token decode over mixed pages: the plain decode attention on the
    exactly decoded K/V of every row.  ``q`` is ``[B, Hq, D]`` float64."""
    lengths = [int(L) for L in lengths]
    B, cap = len(lengths), max(lengths)
    K = np.zeros((B, pool.H, cap, pool.D))
    V = np.zeros((B, pool.H, cap, pool.D))
    for b, L in enumerate(lengths):
        K[b, :, :L] = pool.gather("k", page_table[b], L)
        V[b, :, :L] = pool.gather("v", page_table[b], L)
    return attention.decode_attention(q, K, V, lengths, scale, left_window)


def appended_payload_bytes(page_storages_k, page_storages_v, position: int, n: int, block_size: int,
                           Dk: int, Dv: int, heads: int = 1) -> int:
    """Payload bytes an append of ``n`` tokens at ``position`` writes for one
    row: every new K and V row in its page's storage (metadata excluded).
    ``page_storages_*[j]`` is the storage of logical block ``j``."""
    total = 0
    for p in range(position, position + n):
        j = p // block_size
        total += row_bytes(page_storages_k[j], Dk) + row_bytes(page_storages_v[j], Dv)
    return total * heads


def decoded_float_bytes(page_storages_k, page_storages_v, length: int, block_size: int, Dk: int,
                        Dv: int, left_window: int = -1, heads: int = 1) -> int:
    """FLOAT bytes one decode query at ``length - 1`` decodes: 4 bytes per
    element of every visible K or V row held in an affine page."""
    lo = attention.visible_begin(length - 1, left_window)
    total = 0
    for t in range(lo, length):
        j = t // block_size
        total += (4 * Dk if page_storages_k[j] not in DENSE else 0)
        total += (4 * Dv if page_storages_v[j] not in DENSE else 0)
    return total * heads


def length_threshold_formats(retained: int, threshold: int, early: tuple, late: tuple) -> tuple:
    """The pages' selector example: one (K, V) format pair while fewer than
    ``threshold`` tokens are retained, another afterwards."""
    return early if retained < threshold else late
