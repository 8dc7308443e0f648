"""Sub-byte code packing, affine decode and affine quantisation.

Packing -- "Custom, quantized, and persistent values", section "Struct types
and byte-encodable layouts" (the closed affine branch): codes are row-major;
4-bit types put two codes in a byte and 2-bit types four, least-significant
bits first, unused final high bits zero; ``n`` codes take exactly
``ceil(n * bit_width / 8)`` bytes.  The same page's codebook example (section
"Codebook quantization through a shared subtype") shows the order on bytes:
``0xE4`` holds the 2-bit indices 0, 1, 2, 3.

Decode -- same page, section "Quantization examples": the value of a code is
``(code - zero_point) * scale``.

Quantise -- "Persistent input/output feedback", "Optional heterogeneous paged
KV": rounding is to nearest with ties to even and the result saturates to the
code range; for unsaturated inputs the reconstruction is within half a scale
of the source.  The division ``x / scale`` follows the QuantizeLinear
contract the affine branch refers to, done in float32 (the pages' FLOAT scale
type) so the rounding decision is reproducible; the result is an integer
code, decided in the same precision on both sides.

The INT4 KV format of the decode step (a reading, listed in the design doc): each
token row of ``D`` values is split into ``D/32`` blocks of 32 elements along
the head dimension; block ``i`` has an fp16 ``scale`` and an fp16
``zero_point`` that holds an integer 0..15; codes are UINT4 (0..15), packed
two per byte, even element in the low nibble.
"""
from __future__ import annotations

import numpy as np

from .numeric import f16_to_f64

CODE_RANGE = {  # storage type -> (min code, max code, bit width)
    "INT8": (-128, 127, 8), "UINT8": (0, 255, 8),
    "INT4": (-8, 7, 4), "UINT4": (0, 15, 4),
    "INT2": (-2, 1, 2), "UINT2": (0, 3, 2),
}


def payload_bytes(n: int, bit_width: int) -> int:
    """Bytes of a packed code payload of ``n`` codes: ceil(n * bit_width / 8)."""
    return -(-int(n) * int(bit_width) // 8)


def pack_codes(codes, bit_width: int) -> np.ndarray:
    """Pack unsigned code fields (masked to ``bit_width`` bits) LSB first.

    ``codes`` is ``[..., n]``; returns ``[..., ceil(n * bit_width / 8)]`` uint8.
    Code ``i`` goes to byte ``i // (8 / bit_width)`` at bit ``bit_width * (i % (8 / bit_width))``.
    """
    codes = np.asarray(codes, dtype=np.int64)
    n = codes.shape[-1]
    per = 8 // bit_width
    mask = (1 << bit_width) - 1
    out = np.zeros(codes.shape[:-1] + (payload_bytes(n, bit_width),), dtype=np.int64)
    for i in range(n):
        out[..., i // per] |= (codes[..., i] & mask) << (bit_width * (i % per))
    return out.astype(np.uint8)


def unpack_codes(payload, bit_width: int, n: int, signed: bool = False) -> np.ndarray:
    """Inverse of :func:`pack_codes` on ``[..., bytes]``; ``signed`` sign-extends two's complement."""
    payload = np.asarray(payload, dtype=np.uint8).astype(np.int64)
    per = 8 // bit_width
    mask = (1 << bit_width) - 1
    out = np.empty(payload.shape[:-1] + (n,), dtype=np.int64)
    for i in range(n):
        out[..., i] = (payload[..., i // per] >> (bit_width * (i % per))) & mask
    if signed:
        out = np.where(out >= 1 << (bit_width - 1), out - (1 << bit_width), out)
    return out


def affine_decode(codes, scale, zero_point) -> np.ndarray:
    """``(code - zero_point) * scale`` in float64."""
    codes = np.asarray(codes, dtype=np.float64)
    return (codes - np.asarray(zero_point, dtype=np.float64)) * np.asarray(scale, dtype=np.float64)


def affine_quantize(x, scale, zero_point, storage: str) -> np.ndarray:
    """``clamp(round_half_even(x / scale) + zero_point, lo, hi)`` with a float32 divide."""
    lo, hi, _ = CODE_RANGE[storage]
    q = np.rint(np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float64)
    return np.clip(q + float(zero_point), lo, hi).astype(np.int64)


# ---------------------------------------------------------------------------
# INT4 KV rows: codes [..., D/2] uint8, params [..., D/32, 2] fp16 (scale, zp)
# ---------------------------------------------------------------------------

INT4_BLOCK = 32


def int4_dequant_rows(codes: np.ndarray, params_bits: np.ndarray) -> np.ndarray:
    """Decode INT4 token rows to float64.

    ``codes`` is ``[..., D/2]`` uint8 and ``params_bits`` ``[..., D/32, 2]``
    uint16 fp16 patterns ``(scale, zero_point)``.  Element ``d`` is the nibble
    ``d % 2`` of byte ``d // 2`` (low nibble first) and uses block ``d // 32``.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    D = codes.shape[-1] * 2
    c = unpack_codes(codes, 4, D)                       # [..., D]
    par = f16_to_f64(params_bits)                       # [..., D/32, 2]
    out = np.empty(c.shape, dtype=np.float64)
    for blk in range(D // INT4_BLOCK):
        sl = slice(blk * INT4_BLOCK, (blk + 1) * INT4_BLOCK)
        out[..., sl] = affine_decode(c[..., sl], par[..., blk, 0:1], par[..., blk, 1:2])
    return out


def int4_quantize_rows(x: np.ndarray, scale_bits: int, zero_point_bits: int):
    """Quantise float32 rows ``[..., D]`` with one fp16 scale and fp16 integer zero point.

    Returns ``(codes [..., D/2] uint8, params [..., D/32, 2] uint16)`` where
    every block's param slot holds the same ``(scale, zero_point)`` pair (the
    append uses scalar parameters per call).
    """
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    s = np.float32(f16_to_f64(np.uint16(scale_bits)))
    z = float(f16_to_f64(np.uint16(zero_point_bits)))
    codes = pack_codes(affine_quantize(x, s, z, "UINT4"), 4)
    params = np.empty(x.shape[:-1] + (D // INT4_BLOCK, 2), dtype=np.uint16)
    params[..., 0] = scale_bits
    params[..., 1] = zero_point_bits
    return codes, params
