"""Pins of the mixed-format page oracle (CPU only).

Pinned against: the hand-derived worked example of the pages' block
conversion (tests/golden/mixed_convert_example.json), the plain paged oracle
(an all-BF16 mixed pool is a bf16 pool byte for byte), exact round trips of
representable values, the half-scale reconstruction bound, the pages'
four-step accuracy table and the pages' windowed statistics fixture.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import affine, attention, cache, mixed

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F = mixed.Format


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _one_page_pool(g, k_vals, v_vals, fmt_k=F("BF16"), fmt_v=F("BF16")):
    bs, D = g["block_size"], g["head_dim"]
    pool = mixed.MixedPool(8, 1, bs, D)
    table = np.array([[3]], np.int32)                      # the example's block 3
    n = len(k_vals)
    pool.append(table, _bf16(k_vals)[None, None], _bf16(v_vals)[None, None], [0], n, fmt_k, fmt_v)
    return pool


def test_worked_conversion_example():
    g = _golden("mixed_convert_example.json")
    pool = _one_page_pool(g, g["k_values"], g["v_values"])
    nv = g["valid_rows"]
    ki, vu = g["k_int2"], g["v_uint4"]
    pool.convert([3], [nv], F("INT2", ki["scale"], ki["zero_point"]), F("UINT4", vu["scale"], vu["zero_point"]))
    k_rows = pool.data["k"][3, 0, :4].tolist()
    assert k_rows == [int(h, 16) for h in ki["row_bytes_hex"]]
    v_rows = pool.data["v"][3, 0, :8].tobytes().hex()
    assert v_rows == "".join(vu["row_bytes_hex"])
    # bytes past the new rows keep the earlier dense payload
    first = _bf16(g["k_values"][0]).astype("<u2").view(np.uint8)
    assert pool.data["k"][3, 0, 4:8].tolist() == first[4:8].tolist()
    # then dense: FLOAT16 keys, BFLOAT16 values; scale and zero point are ignored
    pool.convert([3], [nv], F("F16", 1.0, 0), F("BF16", 1.0, 0))
    k16 = pool.data["k"][3, 0].view("<u2").reshape(4, 4)
    v16 = pool.data["v"][3, 0].view("<u2").reshape(4, 4)
    assert k16.tolist() == [[int(h, 16) for h in r] for r in g["k_f16_bits"]]
    assert v16.tolist() == [[int(h, 16) for h in r] for r in g["v_bf16_bits"]]
    # the stored codes decode to the values the example lists
    dec = mixed.decode_rows_exact(np.array([[0x49], [0x27]], np.uint8), F("INT2", 0.25, 0), 4)
    assert dec.tolist() == [[c * 0.25 for c in r] for r in ki["codes"][:2]]


def test_all_bf16_pool_is_a_plain_paged_pool():
    g = synth.rng(300)
    NB, H, bs, D, B, n0, n1 = 24, 2, 4, 8, 3, 6, 5
    order = synth.permutation(synth.rng(301), NB)
    maxb = 4
    table = order[:B * maxb].reshape(B, maxb).astype(np.int32)
    plain = np.zeros((NB, H, bs, D), np.uint16)
    pool = mixed.MixedPool(NB, H, bs, D)
    pos = np.array([0, 0, 0])
    for n in (n0, n1):
        k = _bf16(synth.normal(g, (B, H, n, D)))
        v = _bf16(synth.normal(g, (B, H, n, D)))
        pool.append(table, k, v, pos, n, F("BF16"), F("BF16"))
        cache.paged_cache_update(plain, table, k, pos, n, bs)
        pos = pos + n
    assert pool.data["k"].tobytes() == plain.tobytes()


@pytest.mark.parametrize("storage", ["INT8", "UINT8", "INT4", "UINT4", "INT2", "UINT2"])
def test_representable_values_round_trip(storage):
    lo, hi, nb = affine.CODE_RANGE[storage]
    zp = (lo + hi + 1) // 2
    s = 0.125
    codes = np.arange(lo, hi + 1)
    D = len(codes) * 2 if len(codes) * nb % 8 else len(codes)
    codes = np.resize(codes, D)
    x = ((codes - zp) * s).astype(np.float32)
    enc = mixed.encode_rows(x, F(storage, s, zp))
    assert enc.tolist() == affine.pack_codes(codes, nb).tolist()
    assert mixed.decode_rows_f32(enc, F(storage, s, zp), D).tolist() == x.tolist()


def test_signed_codes_are_twos_complement_lsb_first():
    assert mixed.encode_rows(np.array([-1, 0, 7, -8], np.float32), F("INT4", 1.0, 0)).tolist() == [0x0F, 0x87]
    assert mixed.encode_rows(np.array([-2, -1, 0, 1], np.float32), F("INT2", 1.0, 0)).tolist() == [0x4E]
    assert mixed.encode_rows(np.array([-128, 127], np.float32), F("INT8", 1.0, 0)).tolist() == [0x80, 0x7F]


@pytest.mark.parametrize("storage,scale,zp", [("INT8", 0.01, 0), ("UINT8", 0.01, 128), ("INT4", 0.25, 0),
                                               ("UINT4", 0.25, 8), ("INT2", 0.5, -1), ("UINT2", 0.5, 2)])
def test_reconstruction_within_half_a_scale(storage, scale, zp):
    lo, hi, _ = affine.CODE_RANGE[storage]
    x = synth.uniform(synth.rng(302), (50, 16), (lo - zp) * scale, (hi - zp) * scale)
    fmt = F(storage, scale, zp)
    back = mixed.decode_rows_exact(mixed.encode_rows(x, fmt), fmt, 16)
    assert np.abs(back - x.astype(np.float64)).max() <= scale / 2 * (1 + 1e-6)
    # beyond the range: saturation to the end codes
    far = np.full(16, (hi - zp + 5) * scale, np.float32)
    assert mixed.decode_rows_exact(mixed.encode_rows(far, fmt), fmt, 16).max() == (hi - zp) * float(np.float32(scale))


def test_unused_rows_become_the_zero_of_the_new_format():
    pool = mixed.MixedPool(4, 1, 4, 8)
    table = np.array([[1]], np.int32)
    vals = _bf16(synth.normal(synth.rng(303), (1, 1, 4, 8)))
    pool.append(table, vals, vals, [0], 4, F("BF16"), F("BF16"))
    pool.convert([1], [2], F("UINT4", 0.5, 8), F("INT8", 0.5, -3))
    assert pool.data["k"][1, 0, 8:16].tolist() == [0x88] * 8          # rows 2, 3: code 8
    assert pool.data["v"][1, 0, 16:32].tolist() == [0xFD] * 16        # rows 2, 3: code -3
    pool.convert([1], [1], F("BF16"), None)
    assert pool.data["k"][1, 0, 16:64].tolist() == [0] * 48           # rows 1..3: +0.0
    assert pool.fmt["v"][1] == F("INT8", 0.5, -3)                     # V kept


def test_append_into_a_partial_page_keeps_its_format():
    pool = mixed.MixedPool(4, 1, 4, 8)
    table = np.array([[2, 0]], np.int32)
    g = synth.rng(304)
    a = _bf16(synth.uniform(g, (1, 1, 3, 8), -1, 1))
    pool.append(table, a, a, [0], 3, F("INT8", 0.01, 0), F("INT8", 0.01, 0))
    b = _bf16(synth.uniform(g, (1, 1, 2, 8), -1, 1))
    pool.append(table, b, b, [3], 2, F("UINT4", 0.25, 8), F("BF16"))
    assert pool.fmt["k"][2] == F("INT8", 0.01, 0) and pool.fmt["k"][0] == F("UINT4", 0.25, 8)
    assert pool.fmt["v"][0] == F("BF16")
    x = mixed.bf16_to_f64(b[0, 0]).astype(np.float32)
    assert pool.data["k"][2, 0, 24:32].tolist() == mixed.encode_rows(x[0], F("INT8", 0.01, 0)).tolist()
    assert pool.data["k"][0, 0, 0:4].tolist() == mixed.encode_rows(x[1], F("UINT4", 0.25, 8)).tolist()
    # one row into page 0 (its second slot): the page keeps UINT4 / BF16
    c = _bf16(synth.uniform(g, (1, 1, 1, 8), -1, 1))
    pool.append(table, c, c, [5], 1, F("INT2", 0.5, 0), F("INT2", 0.5, 0))
    assert pool.fmt["k"][0] == F("UINT4", 0.25, 8) and pool.fmt["v"][0] == F("BF16")
    xc = mixed.bf16_to_f64(c[0, 0, 0]).astype(np.float32)
    assert pool.data["k"][0, 0, 4:8].tolist() == mixed.encode_rows(xc, F("UINT4", 0.25, 8)).tolist()


def test_conversion_checks_everything_first():
    pool = mixed.MixedPool(4, 1, 4, 8)
    table = np.array([[1]], np.int32)
    vals = _bf16(np.ones((1, 1, 2, 8)))
    pool.append(table, vals, vals, [0], 2, F("BF16"), F("BF16"))
    before = pool.data["k"].copy()
    bad = [(([1, 1], [2, 2]), F("INT8", 1, 0)), (([5], [2]), F("INT8", 1, 0)), (([1], [5]), F("INT8", 1, 0)),
           (([0], [1]), F("INT8", 1, 0)), (([1], [2]), F("INT8", 0.0, 0)), (([1], [2]), F("INT8", math.inf, 0)),
           (([1], [2]), F("UINT4", 1.0, 16)), (([1], [2]), F("INT2", 1.0, -3)), (([1], [2]), F("FP8", 1.0, 0))]
    for (pages, valid), fmt in bad:
        with pytest.raises(ValueError):
            pool.convert(pages, valid, fmt, F("BF16"))
    assert np.array_equal(pool.data["k"], before) and pool.fmt["k"][1] == F("BF16")


def test_attention_on_lossless_pages_is_plain_attention():
    g = synth.rng(305)
    H, Hq, bs, D, L = 2, 4, 4, 8, 11
    s = 0.125
    codes = np.rint(synth.uniform(g, (1, H, L, D), -7.4, 7.4))
    x = (codes * s).astype(np.float32)                 # exact in bf16 and in every 4-bit+ format with z = 0
    kb = _bf16(x)
    vb = _bf16(x[..., ::-1].copy())
    table = np.array([[5, 1, 3]], np.int32)
    pool = mixed.MixedPool(8, H, bs, D)
    pool.append(table, kb[..., :4, :], vb[..., :4, :], [0], 4, F("INT4", s, 0), F("INT8", s, 0))
    pool.append(table, kb[..., 4:8, :], vb[..., 4:8, :], [4], 4, F("F16"), F("INT4", s, 0))
    pool.append(table, kb[..., 8:, :], vb[..., 8:, :], [8], 3, F("INT8", s, 0), F("BF16"))
    q = synth.normal(g, (1, Hq, D)).astype(np.float64)
    got = mixed.decode_attention(pool, q, table, [L])
    want = attention.decode_attention(q, x.astype(np.float64), x[..., ::-1].astype(np.float64), [L])
    assert np.abs(got - want).max() < 1e-12
    win = mixed.decode_attention(pool, q, table, [L], left_window=5)
    want_w = attention.decode_attention(q, x.astype(np.float64), x[..., ::-1].astype(np.float64), [L], left_window=5)
    assert np.abs(win - want_w).max() < 1e-12


@pytest.mark.parametrize("D", [2, 4, 8, 32])
def test_four_step_accuracy_table_through_pages(D):
    """The pages' four-step fixture with each of its storages on the pages:
    components +/-(0.173 * step), K/V appended with the storage, attention of
    the mixed pool against unquantised dense attention."""
    table_ = _golden("quant_accuracy_table.json")
    comp = table_["component_per_step"]
    sign = np.array([(-1) ** d for d in range(D)], np.float64)
    for row in table_["rows"]:
        fmt = F(row["storage"], row["scale"], row["zero_point"])
        pool = mixed.MixedPool(4, 1, 4, D)
        pt = np.array([[0]], np.int32)
        exact_k, worst = [], 0.0
        for step in range(1, 5):
            x = np.float32(comp * step) * sign.astype(np.float32)
            xb = _bf16(x)
            pool.append(pt, xb[None, None, None], xb[None, None, None], [step - 1], 1, fmt, fmt)
            exact_k.append(mixed.bf16_to_f64(xb))
            q = mixed.bf16_to_f64(xb)[None, None]
            got = mixed.decode_attention(pool, q, pt, [step])
            E = np.array(exact_k)[None, None]
            want = attention.decode_attention(q, E, E, [step])
            worst = max(worst, np.abs(got - want).max())
        assert worst <= row["tolerance"], (row, worst)


def test_windowed_statistics_fixture():
    w = _golden("feedback_copy_formulas.json")["windowed_fixture"]
    assert w["key_storage"] == "INT8" and w["value_storage"] == "UINT4"
    L0, n, W = w["retained_tokens"], w["new_tokens"], w["left_window"]
    k_st = [w["key_storage"]] * 4
    v_st = [w["value_storage"]] * 4
    # queries at L0 and L0 + 1, every visible row in affine pages
    dec = sum(mixed.decoded_float_bytes(k_st, v_st, L0 + i + 1, 4, w["key_width"], w["value_width"], W)
              for i in range(w["queries"]))
    assert dec == w["decoded_float_bytes"]
    # dense pages decode nothing
    assert mixed.decoded_float_bytes(["BF16"] * 4, ["F16"] * 4, 8, 4, 2, 3, W) == 0
    # payload of the append: the new rows in their storages (4-bit V rows of an even width)
    assert mixed.appended_payload_bytes(k_st, v_st, L0, n, 4, 2, 4) == n * (2 + 2)


def test_length_threshold_selector():
    early, late = (F("BF16"), F("BF16")), (F("INT8", 0.01, 0), F("UINT4", 0.25, 8))
    assert mixed.length_threshold_formats(1023, 1024, early, late) == early
    assert mixed.length_threshold_formats(1024, 1024, early, late) == late
