"""Pins of the oracle's code packing, affine decode and INT4 quantisation (CPU only).

Pinned against the worked examples the pages print (tests/golden/*.json):
payload sizes, the LSB-first order shown on the 0xE4 byte, the
``(code - zero_point) * scale`` decode of the fixed-parameter INT4 type, the
half-scale reconstruction bound, and the four-step accuracy table.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import synth
from oracle import affine, attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_payload_sizes_of_the_worked_examples():
    g = _golden("affine_examples.json")
    fixed = g["linear_int4_fixed"]
    assert affine.payload_bytes(fixed["codes"], 4) == fixed["payload_bytes"]
    # with per-value parameters: codes + FLOAT scale + INT64 zero point
    assert affine.payload_bytes(128, 4) + 4 + 8 == g["linear_int4_with_parameters"]["payload_bytes"]
    blk = g["int4_block"]
    record = affine.payload_bytes(blk["codes_per_record"], 4) + blk["scale_bytes"]
    assert affine.payload_bytes(blk["codes_per_record"], 4) == blk["code_bytes"]
    assert record == blk["record_bytes"]
    for ex in blk["examples"]:
        records = ex["logical_elements"] // blk["codes_per_record"]
        assert records == ex["records"] and records * record == ex["payload_bytes"]
    cb = g["codebook2_block_32"]
    assert affine.payload_bytes(32, 2) + 4 == cb["record_bytes"]
    assert 128 * cb["record_bytes"] == cb["payload_bytes_128_records"]
    w = _golden("feedback_copy_formulas.json")["windowed_fixture"]
    got = (affine.payload_bytes(w["new_tokens"] * w["key_width"], 8)
           + affine.payload_bytes(w["new_tokens"] * w["value_width"], 4))
    assert got == w["new_payload_bytes"]


def test_lsb_first_order_on_the_codebook_record():
    cb = _golden("affine_examples.json")["codebook2_block_32"]
    raw = bytes.fromhex(cb["raw_hex"])
    idx = affine.unpack_codes(np.frombuffer(raw[:8], np.uint8), 2, 32)
    assert list(idx[:4]) == cb["first_byte_indices"]
    assert list(idx) == cb["first_byte_indices"] * 8
    scale = struct.unpack("<f", raw[8:12])[0]
    assert scale == cb["scale"]
    decoded = scale * np.asarray(cb["codebook"])[idx]
    assert list(decoded[:4]) == cb["decoded_first_four"]
    assert affine.pack_codes(idx, 2).tobytes() == raw[:8]


def test_four_bit_packing_puts_the_even_element_low():
    assert affine.pack_codes([1, 2, 15], 4).tolist() == [0x21, 0x0F]   # unused high bits zero
    assert affine.unpack_codes(np.array([0x21, 0x0F], np.uint8), 4, 3).tolist() == [1, 2, 15]
    assert affine.unpack_codes(np.array([0xF8], np.uint8), 4, 2, signed=True).tolist() == [-8, -1]


def test_fixed_parameter_int4_decode():
    fixed = _golden("affine_examples.json")["linear_int4_fixed"]
    codes = np.arange(-8, 8)
    got = affine.affine_decode(codes, fixed["scale"], fixed["zero_point"])
    assert got.tolist() == [(c + 2) * 0.25 for c in range(-8, 8)]


def test_quantize_rounds_half_to_even_and_saturates():
    s = 0.25
    x = np.array([2.5, 3.5, -2.5, 0.125, 1.5, 100.0, -100.0], np.float32)
    got = affine.affine_quantize(x * s, s, 8, "UINT4")
    assert got.tolist() == [8 + 2, 8 + 4, 8 - 2, 8 + 0, 8 + 2, 15, 0]


@pytest.mark.parametrize("storage,scale,zp", [("UINT4", 0.25, 8), ("INT4", 0.25, 0),
                                               ("UINT8", 0.01, 128), ("INT8", 0.01, 0)])
def test_reconstruction_within_half_a_scale(storage, scale, zp):
    lo, hi, _ = affine.CODE_RANGE[storage]
    x = synth.uniform(synth.rng(200), 4000, (lo - zp) * scale, (hi - zp) * scale)
    c = affine.affine_quantize(x, scale, zp, storage)
    err = np.abs(affine.affine_decode(c, np.float32(scale), zp) - x.astype(np.float64))
    assert err.max() <= scale / 2 * (1 + 1e-6)


def test_int4_rows_round_trip_and_layout():
    g = synth.rng(201)
    x = synth.uniform(g, (3, 5, 64), -0.7, 0.7)
    s_bits = int(synth.f16_bits(np.float32(0.1)))
    z_bits = int(synth.f16_bits(np.float32(8.0)))
    codes, params = affine.int4_quantize_rows(x, s_bits, z_bits)
    assert codes.shape == (3, 5, 32) and params.shape == (3, 5, 2, 2)
    back = affine.int4_dequant_rows(codes, params)
    s = float(np.uint16(s_bits).view(np.float16))
    assert np.abs(back - x).max() <= s / 2 * (1 + 1e-6)
    # element 0 lives in the low nibble of byte 0, element 1 in the high nibble
    c0 = affine.affine_quantize(x[0, 0, :2], np.float32(s), 8.0, "UINT4")
    assert codes[0, 0, 0] == c0[0] | (c0[1] << 4)


def _accuracy_fixture(storage, scale, zp, D, pattern):
    """Four-step fixture: components +/-(0.173 * step); history quantised, current token exact."""
    comp = _golden("quant_accuracy_table.json")["component_per_step"]
    sign = np.array([pattern(d) for d in range(D)], np.float64)
    hist_k, hist_v, exact_k, exact_v = [], [], [], []
    worst = 0.0
    for step in range(1, 5):
        q = k = v = (comp * step * sign).astype(np.float32)
        Kq = np.array(hist_k + [k], np.float64)
        Vq = np.array(hist_v + [v], np.float64)
        Kx = np.array(exact_k + [k], np.float64)
        Vx = np.array(exact_v + [v], np.float64)
        sc = 1 / math.sqrt(D)
        err = np.abs(attention.attend(q, Kq, Vq, sc) - attention.attend(q, Kx, Vx, sc)).max()
        worst = max(worst, err)
        dq = lambda a: affine.affine_decode(affine.affine_quantize(a, scale, zp, storage), np.float32(scale), zp)
        hist_k.append(dq(k))
        hist_v.append(dq(v))
        exact_k.append(k)
        exact_v.append(v)
    return worst


@pytest.mark.parametrize("D", [2, 4, 8, 32])
@pytest.mark.parametrize("pattern", [lambda d: (-1) ** d, lambda d: (-1) ** (d // 2), lambda d: 1])
def test_four_step_accuracy_table(D, pattern):
    for row in _golden("quant_accuracy_table.json")["rows"]:
        worst = _accuracy_fixture(row["storage"], row["scale"], row["zero_point"], D, pattern)
        assert worst <= row["tolerance"], (row, worst)
