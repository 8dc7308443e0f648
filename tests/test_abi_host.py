"""The C ABI on the host (no GPU): exported symbols and every validation error.

Validation runs before any HIP call, so these calls fail on the CPU with the
documented status and never touch the (fake) device addresses they are given.
Page-pool bookkeeping is host-only and is compared bit for bit with the
oracle's pool on the same hand-out order.
"""
import os
import re

import numpy as np
import pytest

import place_persistent_kv_amd as pkv
import synth
from oracle import cache as ocache

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pkv.h")
FAKE = 0x7F0000000000          # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if getattr(pkv._lib, n, None) is None]
    assert not missing, missing
    assert set(names) <= set(pkv._SIG), "binding signature table lags the header"
    assert pkv.abi_version() == pkv.ABI_VERSION == 10


def R(ptr, dtype, shape):
    return pkv.Raw(ptr, dtype, shape)


def status_of(fn, *a, **k):
    with pytest.raises(pkv.PkvError) as e:
        fn(*a, **k)
    return e.value.status


# --------------------------------------------------------------------------- bindings
def test_bindings_are_exclusive():
    b1 = pkv.bind_writable(R(FAKE, pkv.U8, [4096]))
    try:
        assert status_of(pkv.bind_writable, R(FAKE + 4095, pkv.U8, [10])) == pkv.E_BUSY
        b2 = pkv.bind_writable(R(FAKE + 4096, pkv.U8, [10]))      # adjacent: fine
        b2.close()
    finally:
        b1.close()
    b3 = pkv.bind_writable(R(FAKE, pkv.U8, [4096]))              # released range can be bound again
    b3.close()
    assert status_of(pkv.bind_writable, R(0, pkv.U8, [10])) == pkv.E_ARG


# --------------------------------------------------------------------------- contiguous update
CACHE = R(FAKE, pkv.BF16, [2, 3, 16, 8])
CACHE_BYTES = 2 * 3 * 16 * 8 * 2
VALS = R(FAKE + 0x100000, pkv.BF16, [2, 3, 4, 8])


@pytest.mark.parametrize("pos", [[13, 0], [0, -1], [0, 17]])
def test_cache_update_capacity_error(pos):
    with pkv.bind_writable(CACHE):
        assert status_of(pkv.cache_update, CACHE, VALS, pos, 4) == pkv.E_CAPACITY


def test_cache_update_requires_a_writable_binding():
    assert status_of(pkv.cache_update, CACHE, VALS, [0, 12], 4) == pkv.E_READONLY
    with pkv.bind_writable(R(FAKE, pkv.U8, [CACHE_BYTES - 2])):   # binding one element short
        assert status_of(pkv.cache_update, CACHE, VALS, [0, 12], 4) == pkv.E_READONLY


def test_cache_update_rejects_values_inside_the_cache():
    with pkv.bind_writable(CACHE):
        inside = R(FAKE + 64, pkv.BF16, [2, 3, 4, 8])
        assert status_of(pkv.cache_update, CACHE, inside, [0, 0], 4) == pkv.E_ALIAS


def test_cache_update_shape_and_dtype_errors():
    with pkv.bind_writable(CACHE):
        assert status_of(pkv.cache_update, CACHE, R(VALS.ptr, pkv.F32, [2, 3, 4, 8]), [0, 0], 4) == pkv.E_DTYPE
        assert status_of(pkv.cache_update, CACHE, R(VALS.ptr, pkv.BF16, [2, 3, 4, 4]), [0, 0], 4) == pkv.E_LAYOUT
        assert status_of(pkv.cache_update, CACHE, VALS, [0, 0], 3) == pkv.E_LAYOUT
        assert status_of(pkv.cache_update, CACHE, VALS, [0, 0], -1) == pkv.E_ARG


def test_paired_contiguous_update_checks_both_tensors():
    """pkv_cache_update_kv: every check of the K update and of the V update, plus K/V agreement."""
    vcache = R(FAKE + 0x40000, pkv.BF16, [2, 3, 16, 8])
    vvals = R(FAKE + 0x140000, pkv.BF16, [2, 3, 4, 8])
    f = pkv.cache_update_kv
    with pkv.bind_writable(CACHE):
        assert status_of(f, CACHE, vcache, VALS, vvals, [0, 0], 4) == pkv.E_READONLY   # V cache not writable
    with pkv.bind_writable(CACHE), pkv.bind_writable(vcache):
        assert status_of(f, CACHE, vcache, VALS, vvals, [13, 0], 4) == pkv.E_CAPACITY
        assert status_of(f, CACHE, vcache, VALS, vvals, [0, 0], -1) == pkv.E_ARG
        assert status_of(f, CACHE, vcache, VALS, R(vvals.ptr, pkv.F16, vvals.shape), [0, 0], 4) == pkv.E_DTYPE
        assert status_of(f, CACHE, vcache, VALS, R(vvals.ptr, pkv.BF16, [2, 3, 4, 4]), [0, 0], 4) == pkv.E_LAYOUT
        assert status_of(f, CACHE, vcache, VALS, R(CACHE.ptr + 64, pkv.BF16, vvals.shape), [0, 0], 4) \
            == pkv.E_ALIAS                                                               # V values inside the K cache
        assert status_of(f, CACHE, CACHE, VALS, vvals, [0, 0], 4) == pkv.E_ALIAS         # one cache for K and V
    other = R(FAKE + 0x80000, pkv.BF16, [2, 3, 20, 8])
    with pkv.bind_writable(CACHE), pkv.bind_writable(other):
        assert status_of(f, CACHE, other, VALS, vvals, [0, 0], 4) == pkv.E_LAYOUT       # capacities differ


def test_decode_step_checks_the_append_and_the_attention():
    """pkv_decode_step: the append's checks, the attention's, and no overlap of what the launch writes (the
    caches, out, the workspace) with what it reads."""
    kc = R(FAKE + 0x100000, pkv.BF16, [2, 2, 64, 128])
    vc = R(FAKE + 0x900000, pkv.BF16, [2, 2, 64, 128])
    kv = R(FAKE + 0x1100000, pkv.BF16, [2, 2, 1, 128])
    vv = R(FAKE + 0x1200000, pkv.BF16, [2, 2, 1, 128])
    q = R(FAKE + 0x1300000, pkv.BF16, [2, 8, 128])
    out = R(FAKE + 0x1400000, pkv.F32, [2, 8, 128])
    f = pkv.decode_step
    assert status_of(f, kc, vc, kv, vv, [3, 4], 1, q, out) == pkv.E_READONLY
    with pkv.bind_writable(kc), pkv.bind_writable(vc):
        assert status_of(f, kc, vc, kv, vv, [3, 64], 1, q, out) == pkv.E_CAPACITY
        assert status_of(f, kc, vc, kv, vv, [3, 4], -1, q, out) == pkv.E_ARG
        assert status_of(f, kc, vc, kv, R(vv.ptr, pkv.F16, vv.shape), [3, 4], 1, q, out) == pkv.E_DTYPE
        assert status_of(f, kc, vc, kv, vv, [3, 4], 1, R(q.ptr, pkv.BF16, [2, 6, 128]), out) == pkv.E_LAYOUT
        assert status_of(f, kc, vc, kv, vv, [3, 4], 1, R(kc.ptr, pkv.BF16, q.shape), out) == pkv.E_ALIAS
        assert status_of(f, kc, vc, kv, vv, [3, 4], 1, q, R(vc.ptr, pkv.F32, out.shape)) == pkv.E_ALIAS
        assert status_of(f, kc, vc, kv, vv, [3, 4], 1, q, R(kv.ptr, pkv.F32, out.shape)) == pkv.E_ALIAS
        none_k, none_v = R(kv.ptr, pkv.BF16, [2, 2, 0, 128]), R(vv.ptr, pkv.BF16, [2, 2, 0, 128])
        assert status_of(f, kc, vc, none_k, none_v, [0, 4], 0, q, out) == pkv.E_CAPACITY   # valid_len 0
        assert status_of(f, kc, vc, kv, vv, [3, 4], 1, q, out, left_window=-2) == pkv.E_ARG
    long_k = R(FAKE + 0x2000000, pkv.BF16, [2, 2, 2048, 128])
    long_v = R(FAKE + 0x3000000, pkv.BF16, [2, 2, 2048, 128])
    with pkv.bind_writable(long_k), pkv.bind_writable(long_v):
        args = (long_k, long_v, kv, vv, [1500, 2000], 1, q, out)
        assert status_of(f, *args, num_splits=4) == pkv.E_NOMEM
        need = pkv.decode_workspace_size(2, 8, 2, 128, 2048, 4)
        assert status_of(f, *args, workspace=R(kv.ptr, pkv.U8, [need]), num_splits=4) == pkv.E_ALIAS


# --------------------------------------------------------------------------- pool
def test_pool_matches_the_oracle_pool():
    g = synth.rng(500)
    NB, bs, S, maxb = 64, 4, 6, 12
    order = synth.permutation(g, NB)
    lib = pkv.Pool(NB, bs, S, maxb, order)
    ref = ocache.PagePool(NB, bs, S, maxb, order)
    lens = np.zeros(S, np.int64)
    for it in range(12):
        seqs = sorted(g.choice(S, size=int(g.integers(1, S + 1)), replace=False).tolist())
        new = [int(lens[s] + g.integers(0, 9)) for s in seqs]
        need = sum(max(0, ocache.pages_for(n, bs) - ref.held[s]) for s, n in zip(seqs, new))
        if any(ocache.pages_for(n, bs) > maxb for n in new):
            assert status_of(lib.reserve, seqs, new) == pkv.E_PAGE
        elif need > len(ref.free):
            assert status_of(lib.reserve, seqs, new) == pkv.E_NOMEM
        else:
            lib.reserve(seqs, new)
            for s, n in zip(seqs, new):
                ref.reserve(s, n)
                lens[s] = max(lens[s], n)
        if it % 5 == 4:
            lib.release(seqs[0])
            ref.release(seqs[0])
            lens[seqs[0]] = 0
        assert np.array_equal(lib.table(), ref.table)
        assert lib.free_count() == len(ref.free)
        for s in range(S):
            assert lib.query(s)[0] == ref.held[s]


def test_pool_errors_change_nothing():
    lib = pkv.Pool(7, 4, 2, 4)
    lib.reserve([0], [9])                     # 3 pages, 4 left
    table, free = lib.table(), lib.free_count()
    assert status_of(lib.reserve, [0, 1], [12, 17]) == pkv.E_PAGE     # 5 pages > max 4
    assert status_of(lib.reserve, [1, 1], [1, 1]) == pkv.E_PAGE       # listed twice
    assert status_of(lib.reserve, [1], [4 * 6]) == pkv.E_PAGE
    assert status_of(lib.reserve, [0, 1], [16, 16]) == pkv.E_NOMEM    # needs 1 + 4 > 4 free
    assert status_of(lib.reserve, [2], [1]) == pkv.E_PAGE             # sequence out of range
    assert np.array_equal(lib.table(), table) and lib.free_count() == free
    assert status_of(pkv.Pool, 4, 4, 1, 1, [0, 1, 1, 3]) == pkv.E_ARG


# --------------------------------------------------------------------------- paged update
def test_paged_update_needs_reserved_pages_and_capacity():
    pool = pkv.Pool(16, 4, 2, 4)
    pool.reserve([0, 1], [5, 4])              # row 0: 2 pages, row 1: 1 page
    kv = R(FAKE, pkv.BF16, [16, 2, 4, 8])
    vals = R(FAKE + 0x100000, pkv.BF16, [2, 2, 1, 8])
    table = R(FAKE + 0x200000, pkv.I32, [2, 4])
    with pkv.bind_writable(kv):
        assert status_of(pkv.paged_cache_update, pool, kv, table, vals, [7, 4], 1) == pkv.E_PAGE   # row 1 page 1
        assert status_of(pkv.paged_cache_update, pool, kv, table, vals, [16, 0], 1) == pkv.E_CAPACITY
        assert status_of(pkv.paged_cache_update, None, kv, table, vals, [0, 0], 1) == pkv.E_ARG
        bad = R(FAKE, pkv.BF16, [16, 2, 8, 8])
    assert status_of(pkv.paged_cache_update, pool, kv, table, vals, [0, 0], 1) == pkv.E_READONLY
    with pkv.bind_writable(bad):
        assert status_of(pkv.paged_cache_update, pool, bad, table, vals, [0, 0], 1) == pkv.E_LAYOUT


def test_paired_kv_update_checks_both_tensors_before_any_write():
    """pkv_paged_cache_update_kv: every check of the K update and of the V update, plus K/V agreement."""
    pool = pkv.Pool(16, 4, 2, 4)
    pool.reserve([0, 1], [5, 4])
    kp = R(FAKE, pkv.BF16, [16, 2, 4, 8])
    vp = R(FAKE + 0x40000, pkv.BF16, [16, 2, 4, 8])
    kv = R(FAKE + 0x100000, pkv.BF16, [2, 2, 1, 8])
    vv = R(FAKE + 0x140000, pkv.BF16, [2, 2, 1, 8])
    table = R(FAKE + 0x200000, pkv.I32, [2, 4])
    f = pkv.paged_cache_update_kv
    with pkv.bind_writable(kp):
        assert status_of(f, pool, kp, vp, table, kv, vv, [0, 0], 1) == pkv.E_READONLY   # V pool not writable
    with pkv.bind_writable(kp), pkv.bind_writable(vp):
        assert status_of(f, pool, kp, vp, table, kv, vv, [7, 4], 1) == pkv.E_PAGE       # row 1, page 1
        assert status_of(f, pool, kp, vp, table, kv, vv, [16, 0], 1) == pkv.E_CAPACITY
        assert status_of(f, None, kp, vp, table, kv, vv, [0, 0], 1) == pkv.E_ARG
        assert status_of(f, pool, kp, vp, None, kv, vv, [0, 0], 1) == pkv.E_ARG          # page table required
        assert status_of(f, pool, kp, vp, table, kv, R(vv.ptr, pkv.F16, vv.shape), [0, 0], 1) == pkv.E_DTYPE
        assert status_of(f, pool, kp, vp, table, kv, R(vv.ptr, pkv.BF16, [2, 2, 2, 8]), [0, 0], 1) \
            == pkv.E_LAYOUT                                                              # V values of another length
        assert status_of(f, pool, kp, vp, table, kv, R(kp.ptr + 64, pkv.BF16, vv.shape), [0, 0], 1) \
            == pkv.E_ALIAS                                                               # V values inside the K pool
        assert status_of(f, pool, kp, kp, table, kv, vv, [0, 0], 1) == pkv.E_ALIAS       # one pool for K and V
    big = R(FAKE + 0x400000, pkv.BF16, [16, 2, 4, 16])
    with pkv.bind_writable(kp), pkv.bind_writable(big):
        assert status_of(f, pool, kp, big, table, kv, R(vv.ptr, pkv.BF16, [2, 2, 1, 16]), [0, 0], 1) \
            == pkv.E_LAYOUT                                                              # pools of two head sizes


def test_int4_update_parameter_checks():
    pool = pkv.Pool(16, 4, 2, 4)
    pool.reserve([0, 1], [4, 4])
    codes = R(FAKE, pkv.U8, [16, 2, 4, 32])
    params = R(FAKE + 0x100000, pkv.F16, [16, 2, 4, 2, 2])
    vals = R(FAKE + 0x200000, pkv.F32, [2, 2, 1, 64])
    table = R(FAKE + 0x300000, pkv.I32, [2, 4])
    one = int(synth.f16_bits(np.float32(1.0)))
    with pkv.bind_writable(codes), pkv.bind_writable(params):
        for s_bits, z_bits in [(int(synth.f16_bits(np.float32(-0.5))), 0), (0, 0), (0x7C00, 0), (0x7E00, 0),
                               (one, int(synth.f16_bits(np.float32(0.5)))),
                               (one, int(synth.f16_bits(np.float32(16.0)))),
                               (one, int(synth.f16_bits(np.float32(-1.0))))]:
            assert status_of(pkv.paged_cache_update_int4, pool, codes, params, table, vals, s_bits, z_bits,
                             [0, 0], 1) == pkv.E_ARG
        odd = R(FAKE + 0x200000, pkv.F32, [2, 2, 1, 48])
        assert status_of(pkv.paged_cache_update_int4, pool, R(FAKE, pkv.U8, [16, 2, 4, 24]), params, table,
                         odd, one, 0, [0, 0], 1) == pkv.E_LAYOUT
        assert status_of(pkv.paged_cache_update_int4, pool, codes, params, table,
                         R(vals.ptr, pkv.U8, [2, 2, 1, 64]), one, 0, [0, 0], 1) == pkv.E_DTYPE


# --------------------------------------------------------------------------- decode
Q = R(FAKE, pkv.BF16, [2, 8, 1, 128])
OUT = R(FAKE + 0x10000, pkv.BF16, [2, 8, 1, 128])
KC = R(FAKE + 0x100000, pkv.BF16, [2, 2, 64, 128])
VC = R(FAKE + 0x200000, pkv.BF16, [2, 2, 64, 128])


@pytest.mark.parametrize("L", [[0, 5], [65, 5], [-3, 1]])
def test_decode_valid_len_range(L):
    assert status_of(pkv.decode_attention, Q, KC, VC, L, OUT) == pkv.E_CAPACITY


def test_decode_shape_and_dtype_errors():
    assert status_of(pkv.decode_attention, R(FAKE, pkv.BF16, [2, 6, 1, 128]), R(KC.ptr, pkv.BF16, [2, 4, 64, 128]),
                     R(VC.ptr, pkv.BF16, [2, 4, 64, 128]), [1, 1], R(OUT.ptr, pkv.BF16, [2, 6, 1, 128])) == pkv.E_LAYOUT
    assert status_of(pkv.decode_attention, Q, R(KC.ptr, pkv.F32, KC.shape), VC, [1, 1], OUT) == pkv.E_DTYPE
    assert status_of(pkv.decode_attention, Q, KC, VC, [1, 1], R(OUT.ptr, pkv.F16, OUT.shape)) == pkv.E_DTYPE
    assert status_of(pkv.decode_attention, Q, KC, VC, [1, 1], R(OUT.ptr, pkv.BF16, [2, 8, 1, 64])) == pkv.E_LAYOUT
    assert status_of(pkv.decode_attention, Q, KC, VC, [1, 1], R(Q.ptr, pkv.BF16, Q.shape)) == pkv.E_ALIAS


def test_left_window_must_be_minus_one_or_more():
    assert status_of(pkv.decode_attention, Q, KC, VC, [1, 1], OUT, left_window=-2) == pkv.E_ARG
    table = R(FAKE + 0x2000000, pkv.I32, [2, 8])
    kp = R(FAKE + 0x100000, pkv.BF16, [32, 2, 16, 128])
    vp = R(FAKE + 0x900000, pkv.BF16, [32, 2, 16, 128])
    assert status_of(pkv.paged_decode_attention, Q, kp, vp, table, 8, 16, [4, 4], OUT, left_window=-5) == pkv.E_ARG
    qc = R(FAKE + 0x3000000, pkv.BF16, [2, 4, 8, 128])
    oc = R(FAKE + 0x3400000, pkv.BF16, [2, 4, 8, 128])
    assert status_of(pkv.chunk_attention, qc, kp, vp, table, 8, 16, [0, 0], oc, left_window=-2) == pkv.E_ARG


def test_decode_workspace_is_checked():
    # 64 tokens with 8 splits of 64-token minimum -> 1 split: no workspace needed on the fast path;
    # force splits on a longer cache instead
    kc = R(FAKE + 0x100000, pkv.BF16, [2, 2, 1024, 128])
    vc = R(FAKE + 0x900000, pkv.BF16, [2, 2, 1024, 128])
    assert status_of(pkv.decode_attention, Q, kc, vc, [1000, 900], OUT, num_splits=4) == pkv.E_NOMEM
    need = pkv.decode_workspace_size(2, 8, 2, 128, 1024, 4)
    small = R(FAKE + 0x2000000, pkv.U8, [need - 256])
    assert status_of(pkv.decode_attention, Q, kc, vc, [1000, 900], OUT, workspace=small, num_splits=4) == pkv.E_NOMEM
    inside = R(kc.ptr, pkv.U8, [need])
    assert status_of(pkv.decode_attention, Q, kc, vc, [1000, 900], OUT, workspace=inside, num_splits=4) == pkv.E_ALIAS


def test_workspace_bound_covers_any_lengths():
    for B, Hq, D, L, S in [(32, 32, 128, 32768, 0), (8, 32, 128, 4096, 0), (1, 1, 4, 16, 0), (3, 8, 64, 5000, 7)]:
        n = pkv.decode_workspace_size(B, Hq, Hq // 4 or 1, D, L, S)
        assert n >= B * Hq * D * 4 and n % 256 == 0
    assert pkv.decode_workspace_size(0, 8, 2, 128, 16, 0) == 0


def test_paged_decode_checks_reserved_pages():
    pool = pkv.Pool(32, 16, 2, 8)
    pool.reserve([0, 1], [40, 16])
    kp = R(FAKE + 0x100000, pkv.BF16, [32, 2, 16, 128])
    vp = R(FAKE + 0x900000, pkv.BF16, [32, 2, 16, 128])
    table = R(FAKE + 0x2000000, pkv.I32, [2, 8])
    assert status_of(pkv.paged_decode_attention, Q, kp, vp, table, 8, 16, [40, 17], OUT, pool=pool) == pkv.E_PAGE
    assert status_of(pkv.paged_decode_attention, Q, kp, vp, table, 8, 32, [40, 16], OUT, pool=pool) == pkv.E_LAYOUT
    assert status_of(pkv.paged_decode_attention, Q, kp, vp, table, 8, 16, [129, 16], OUT) == pkv.E_CAPACITY


# --------------------------------------------------------------------------- INT4 decode and chunk attention
def _int4_pools(bs=16, NB=32, Hkv=2, offset=0):
    kc = R(FAKE + 0x100000 + offset, pkv.U8, [NB, Hkv, bs, 64])
    vc = R(FAKE + 0x900000 + offset, pkv.U8, [NB, Hkv, bs, 64])
    kp = R(FAKE + 0x1100000 + offset, pkv.F16, [NB, Hkv, bs, 4, 2])
    vp = R(FAKE + 0x1900000 + offset, pkv.F16, [NB, Hkv, bs, 4, 2])
    return kc, kp, vc, vp


def test_int4_decode_layout_checks():
    q = R(FAKE + 0x3000000, pkv.F32, [2, 8, 1, 128])
    out = R(FAKE + 0x3100000, pkv.F32, [2, 8, 1, 128])
    table = R(FAKE + 0x2000000, pkv.I32, [2, 8])
    kc, kp, vc, vp = _int4_pools()
    f = pkv.paged_decode_attention_int4
    # block size must match the pool and be a power of two >= 16
    assert status_of(f, q, kc, kp, vc, vp, table, 8, 32, [16, 16], out) == pkv.E_LAYOUT
    kc8, kp8, vc8, vp8 = _int4_pools(bs=8)
    assert status_of(f, q, kc8, kp8, vc8, vp8, table, 8, 8, [16, 16], out) == pkv.E_LAYOUT
    # every pool 16-byte aligned
    bad = R(kp.ptr + 4, pkv.F16, kp.shape)
    assert status_of(f, q, kc, bad, vc, vp, table, 8, 16, [16, 16], out) == pkv.E_LAYOUT
    # q and out f32; Hq / Hkv in {1, 2, 4, 8}
    assert status_of(f, R(q.ptr, pkv.BF16, q.shape), kc, kp, vc, vp, table, 8, 16, [16, 16], out) == pkv.E_DTYPE
    q6 = R(q.ptr, pkv.F32, [2, 6, 1, 128])
    assert status_of(f, q6, kc, kp, vc, vp, table, 8, 16, [16, 16], R(out.ptr, pkv.F32, q6.shape)) == pkv.E_LAYOUT
    # lengths within max_blocks * block_size
    assert status_of(f, q, kc, kp, vc, vp, table, 8, 16, [129, 16], out) == pkv.E_CAPACITY


def test_chunk_attention_checks():
    q = R(FAKE + 0x3000000, pkv.BF16, [2, 4, 32, 128])
    out = R(FAKE + 0x3400000, pkv.BF16, [2, 4, 32, 128])
    kp = R(FAKE + 0x100000, pkv.BF16, [32, 2, 16, 128])
    vp = R(FAKE + 0x900000, pkv.BF16, [32, 2, 16, 128])
    table = R(FAKE + 0x2000000, pkv.I32, [2, 8])
    f = pkv.chunk_attention
    # p0 + C must fit the table's capacity, p0 >= 0
    assert status_of(f, q, kp, vp, table, 8, 16, [97, 0], out) == pkv.E_CAPACITY
    assert status_of(f, q, kp, vp, table, 8, 16, [-1, 0], out) == pkv.E_CAPACITY
    # block size: equal to the pool's, a power of two, at least 4
    kp2 = R(kp.ptr, pkv.BF16, [32, 2, 2, 128])
    vp2 = R(vp.ptr, pkv.BF16, [32, 2, 2, 128])
    assert status_of(f, q, kp2, vp2, table, 8, 2, [0, 0], out) == pkv.E_LAYOUT
    kp12 = R(kp.ptr, pkv.BF16, [32, 2, 12, 128])
    vp12 = R(vp.ptr, pkv.BF16, [32, 2, 12, 128])
    assert status_of(f, q, kp12, vp12, table, 8, 12, [0, 0], out) == pkv.E_LAYOUT
    assert status_of(f, q, kp, vp, table, 8, 32, [0, 0], out) == pkv.E_LAYOUT
    # with a pool handle, every row needs ceil((p0 + C) / bs) reserved pages
    pool = pkv.Pool(32, 16, 2, 8)
    pool.reserve([0, 1], [48, 64])
    assert status_of(f, q, kp, vp, table, 8, 16, [16, 40], out, pool=pool) == pkv.E_PAGE   # row 1: 72 tokens
    # head size 128 and bf16 only
    assert status_of(f, R(q.ptr, pkv.F32, q.shape), kp, vp, table, 8, 16, [0, 0], R(out.ptr, pkv.F32, out.shape)) \
        == pkv.E_DTYPE
    # the pools, q and out are read and written in 16-byte pieces
    for bad in ({"kp": R(kp.ptr + 8, pkv.BF16, kp.shape)}, {"vp": R(vp.ptr + 2, pkv.BF16, vp.shape)},
                {"q": R(q.ptr + 4, pkv.BF16, q.shape)}, {"out": R(out.ptr + 8, pkv.BF16, out.shape)}):
        args = {**dict(q=q, kp=kp, vp=vp, out=out), **bad}
        assert status_of(f, args["q"], args["kp"], args["vp"], table, 8, 16, [0, 0], args["out"]) == pkv.E_LAYOUT
        assert "16-byte" in pkv.last_error()


def test_chunk_split_workspace_is_checked():
    q = R(FAKE + 0x3000000, pkv.BF16, [2, 4, 32, 128])
    out = R(FAKE + 0x3400000, pkv.BF16, [2, 4, 32, 128])
    kp = R(FAKE + 0x100000, pkv.BF16, [32, 2, 16, 128])
    vp = R(FAKE + 0x900000, pkv.BF16, [32, 2, 16, 128])
    table = R(FAKE + 0x2000000, pkv.I32, [2, 8])
    f = pkv.chunk_attention
    need = pkv.chunk_workspace_size(2, 4, 2, 32, 4)
    for S in (-1, 65):
        assert status_of(f, q, kp, vp, table, 8, 16, [40, 0], out, workspace=R(FAKE + 0x4000000, pkv.U8, [need]),
                         num_splits=S) == pkv.E_ARG
    assert status_of(f, q, kp, vp, table, 8, 16, [40, 0], out, num_splits=4) == pkv.E_NOMEM
    small = R(FAKE + 0x4000000, pkv.U8, [need - 256])
    assert status_of(f, q, kp, vp, table, 8, 16, [40, 0], out, workspace=small, num_splits=4) == pkv.E_NOMEM
    skew = R(FAKE + 0x4000000 + 128, pkv.U8, [need])
    assert status_of(f, q, kp, vp, table, 8, 16, [40, 0], out, workspace=skew, num_splits=4) == pkv.E_ARG
    for inside in (out.ptr, kp.ptr, q.ptr):
        ws = R(inside, pkv.U8, [need])
        assert status_of(f, q, kp, vp, table, 8, 16, [40, 0], out, workspace=ws, num_splits=4) == pkv.E_ALIAS


def test_chunk_workspace_size():
    up = lambda x: -(-x // 256) * 256
    for B, Hq, Hkv, C, S in [(2, 4, 2, 32, 4), (1, 16, 8, 512, 8), (3, 8, 8, 7, 64), (300, 2, 1, 5, 2)]:
        rows = min(B, 256)
        assert pkv.chunk_workspace_size(B, Hq, Hkv, C, S) == up(rows * Hq * C * S * 128 * 4) + \
            up(rows * Hq * C * S * 2 * 4)
    assert pkv.chunk_workspace_size(2, 4, 2, 32, 1) == 0                  # no split, no workspace
    assert pkv.chunk_workspace_size(128, 16, 8, 512, 0) == 0              # a launch that fills the device
    assert pkv.chunk_workspace_size(1, 16, 8, 512, 0) > 0                 # one row leaves CUs idle
    for bad in [(0, 4, 2, 32, 2), (2, 6, 4, 32, 2), (2, 4, 2, 0, 2), (2, 4, 2, 32, 65), (2, 32, 2, 32, 2)]:
        assert pkv.chunk_workspace_size(*bad) == 0


# --------------------------------------------------------------------------- sampling
@pytest.mark.parametrize("T", [-1.0, float("nan"), float("-inf")])
def test_sample_rejects_bad_temperature(T):
    logits = R(FAKE, pkv.F32, [4, 1000])
    ids = R(FAKE + 0x100000, pkv.I64, [4])
    ws = R(FAKE + 0x200000, pkv.U8, [pkv.sample_workspace_size(4, 1000)])
    assert status_of(pkv.sample, logits, T, 0, ids, ws) == pkv.E_ARG


def test_sample_shape_errors():
    ids = R(FAKE + 0x100000, pkv.I64, [4])
    ws = R(FAKE + 0x200000, pkv.U8, [pkv.sample_workspace_size(4, 1000)])
    assert status_of(pkv.sample, R(FAKE, pkv.I32, [4, 1000]), 0.0, 0, ids, ws) == pkv.E_DTYPE
    assert status_of(pkv.sample, R(FAKE, pkv.F32, [4000]), 0.0, 0, ids, ws) == pkv.E_LAYOUT
    assert status_of(pkv.sample, R(FAKE, pkv.F32, [4, 1000]), 0.0, 0, ids, None) == pkv.E_NOMEM


def test_one_hip_runtime_in_the_process():
    """libpkv must run on torch's HIP runtime: a second runtime would not share torch's streams."""
    maps = open("/proc/self/maps").read()
    libs = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln and "/" in ln}
    assert len(libs) == 1, libs


# --------------------------------------------------------------------------- mixed-format pages
MNB, MH, MBS, MD = 8, 2, 16, 128
MK = R(FAKE, pkv.BF16, [MNB, MH, MBS, MD])
MV = R(FAKE + 0x200000, pkv.BF16, [MNB, MH, MBS, MD])
MDESC = R(FAKE + 0x400000, pkv.U8, [MNB, 16])
MTABLE = FAKE + 0x500000
MVALS_K = R(FAKE + 0x600000, pkv.BF16, [1, MH, 4, MD])
MVALS_V = R(FAKE + 0x700000, pkv.BF16, [1, MH, 4, MD])
BF = pkv.page_format("BF16")


def _mixed_bindings():
    return [pkv.bind_writable(MK), pkv.bind_writable(MV), pkv.bind_writable(MDESC)]


@pytest.mark.parametrize("fmt", [pkv.page_format(9), pkv.page_format("INT8", 0.0, 0),
                                 pkv.page_format("INT8", float("inf"), 0), pkv.page_format("INT8", float("nan"), 0),
                                 pkv.page_format("UINT4", 0.5, 16), pkv.page_format("INT2", 0.5, -3),
                                 pkv.page_format("UINT8", 0.5, -1), pkv.page_format("INT8", 0.5, 128)])
def test_mixed_formats_are_checked(fmt):
    pool = pkv.Pool(MNB, MBS, 2, 4)
    pool.reserve([0], [4])
    bs = _mixed_bindings()
    try:
        assert status_of(pkv.mixed_cache_update, pool, MK, MV, MDESC, MTABLE, MVALS_K, MVALS_V, [0], 4,
                         fmt, BF) == pkv.E_ARG
        assert status_of(pkv.mixed_cache_update, pool, MK, MV, MDESC, MTABLE, MVALS_K, MVALS_V, [0], 4,
                         BF, fmt) == pkv.E_ARG
        assert status_of(pkv.mixed_convert_pages, MK, MV, MDESC, [1], [4], fmt, None) == pkv.E_ARG
    finally:
        for b in bs:
            b.close()


def test_mixed_update_errors():
    pool = pkv.Pool(MNB, MBS, 2, 4)
    pool.reserve([0], [4])
    i8 = pkv.page_format("INT8", 0.01, 0)
    # no binding: read-only
    assert status_of(pkv.mixed_cache_update, pool, MK, MV, MDESC, MTABLE, MVALS_K, MVALS_V, [0], 4, i8, i8) \
        == pkv.E_READONLY
    bs = _mixed_bindings()
    try:
        ok = (MK, MV, MDESC, MTABLE, MVALS_K, MVALS_V)
        assert status_of(pkv.mixed_cache_update, pool, *ok, [14], 4, i8, i8) == pkv.E_PAGE    # past the page held
        assert status_of(pkv.mixed_cache_update, pool, *ok, [-1], 4, i8, i8) == pkv.E_CAPACITY
        f32v = R(MVALS_K.ptr, pkv.F32, [1, MH, 4, MD])
        assert status_of(pkv.mixed_cache_update, pool, MK, MV, MDESC, MTABLE, f32v, MVALS_V, [0], 4, i8, i8) \
            == pkv.E_DTYPE
        bad_desc = R(MDESC.ptr, pkv.U8, [MNB, 8])
        assert status_of(pkv.mixed_cache_update, pool, MK, MV, bad_desc, MTABLE, MVALS_K, MVALS_V, [0], 4, i8, i8) \
            == pkv.E_LAYOUT
        inside = R(FAKE + 64, pkv.BF16, [1, MH, 4, MD])
        assert status_of(pkv.mixed_cache_update, pool, MK, MV, MDESC, MTABLE, inside, MVALS_V, [0], 4, i8, i8) \
            == pkv.E_ALIAS
        odd = R(MVALS_K.ptr + 2, pkv.BF16, [1, MH, 4, MD])
        assert status_of(pkv.mixed_cache_update, pool, MK, MV, MDESC, MTABLE, odd, MVALS_V, [0], 4, i8, i8) \
            == pkv.E_LAYOUT
    finally:
        for b in bs:
            b.close()


def test_mixed_conversion_errors():
    bs = _mixed_bindings()
    i4 = pkv.page_format("INT4", 0.25, 0)
    try:
        assert status_of(pkv.mixed_convert_pages, MK, MV, MDESC, [1, 1], [4, 4], i4, None) == pkv.E_ARG
        assert status_of(pkv.mixed_convert_pages, MK, MV, MDESC, [MNB], [4], i4, None) == pkv.E_PAGE
        assert status_of(pkv.mixed_convert_pages, MK, MV, MDESC, [-1], [4], None, i4) == pkv.E_PAGE
        assert status_of(pkv.mixed_convert_pages, MK, MV, MDESC, [1], [MBS + 1], i4, i4) == pkv.E_ARG
        big_k = R(FAKE, pkv.BF16, [2, 1, 1024, 64])
        big_v = R(FAKE + 0x200000, pkv.BF16, [2, 1, 1024, 64])
        big_d = R(FAKE + 0x400000, pkv.U8, [2, 16])
        assert status_of(pkv.mixed_convert_pages, big_k, big_v, big_d, [0], [4], i4, None) == pkv.E_LAYOUT
    finally:
        for b in bs:
            b.close()
    # converting needs writable pools; nothing to convert needs nothing
    assert status_of(pkv.mixed_convert_pages, MK, MV, MDESC, [1], [4], i4, None) == pkv.E_READONLY
    pkv.mixed_convert_pages(MK, MV, MDESC, [1], [4], None, None)


def test_mixed_decode_errors():
    q = R(FAKE + 0x800000, pkv.BF16, [1, 4, MD])
    out = R(FAKE + 0x900000, pkv.BF16, [1, 4, MD])
    ws = FAKE + 0xA00000

    def call(q=q, k=MK, v=MV, d=MDESC, out=out, bs=MBS, lens=(20,), win=-1):
        return status_of(pkv.paged_decode_attention_mixed, q, k, v, d, MTABLE, 4, bs, list(lens), out,
                         R(ws, pkv.U8, [1 << 20]), left_window=win)
    assert call(q=R(q.ptr, pkv.F32, [1, 4, MD]), out=R(out.ptr, pkv.F32, [1, 4, MD])) == pkv.E_DTYPE
    assert call(q=R(q.ptr, pkv.BF16, [1, 6, MD]), out=R(out.ptr, pkv.BF16, [1, 6, MD])) == pkv.E_LAYOUT   # G = 3
    k64 = R(FAKE, pkv.BF16, [MNB, MH, MBS, 64])
    v64 = R(FAKE + 0x200000, pkv.BF16, [MNB, MH, MBS, 64])
    assert call(q=R(q.ptr, pkv.BF16, [1, 4, 64]), out=R(out.ptr, pkv.BF16, [1, 4, 64]), k=k64, v=v64) \
        == pkv.E_LAYOUT
    k8 = R(FAKE, pkv.BF16, [MNB, MH, 8, MD])
    v8 = R(FAKE + 0x200000, pkv.BF16, [MNB, MH, 8, MD])
    assert call(k=k8, v=v8, bs=8) == pkv.E_LAYOUT                                                  # block < 16
    assert call(d=R(MDESC.ptr, pkv.U8, [MNB - 1, 16])) == pkv.E_LAYOUT
    assert call(lens=(0,)) == pkv.E_CAPACITY
    assert call(lens=(65,)) == pkv.E_CAPACITY
    assert call(win=-2) == pkv.E_ARG


def test_length_threshold_selector():
    early = (pkv.page_format("BF16"), pkv.page_format("BF16"))
    late = (pkv.page_format("INT8", 0.01, 0), pkv.page_format("UINT4", 0.25, 8))
    sel = pkv.LengthThresholdSelector(1024, early, late)
    assert sel(0) is early and sel(1023) is early and sel(1024) is late


# --------------------------------------------------------------------------- generation loop
def test_generate_step_seed_matches_the_oracle():
    from oracle import generate as ogen
    for seed, t, B, V in [(0, 0, 1, 1), (7, 3, 128, 151936), (2 ** 64 - 1, 1000, 32, 50000)]:
        assert pkv.generate_step_seed(seed, t, B, V) == ogen.step_seed(seed, t, B, V)


def test_generate_finish_errors():
    tok = R(FAKE, pkv.I64, [4, 10])
    ids, fin, nxt, unf = FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, FAKE + 0x4000
    with pytest.raises(pkv.PkvError) as e:
        pkv._check(pkv._lib.pkv_generate_finish(ids, fin, tok.ptr, 10, 10, 4, 2, 2, nxt, unf, None), "x")
    assert e.value.status == pkv.E_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv._check(pkv._lib.pkv_generate_finish(ids, fin, tok.ptr, 10, -1, 4, 2, 2, nxt, unf, None), "x")
    assert e.value.status == pkv.E_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv._check(pkv._lib.pkv_generate_finish(None, fin, tok.ptr, 10, 0, 4, 2, 2, nxt, unf, None), "x")
    assert e.value.status == pkv.E_ARG
    with pytest.raises(pkv.PkvError) as e:      # next_ids inside tokens
        pkv._check(pkv._lib.pkv_generate_finish(ids, fin, tok.ptr, 10, 0, 4, 2, 2, tok.ptr + 8, unf, None), "x")
    assert e.value.status == pkv.E_ALIAS


def test_noalloc_decode_validates_before_any_hip_call():
    """The static-scratch variant fails its checks on the host, the scratch size limit included."""
    B, Hq, Hkv, D, bs, NB, maxb = 12, 64, 8, 128, 16, 4096, 300
    q = R(FAKE, pkv.BF16, [B, Hq, D])
    kp = R(FAKE + (1 << 30), pkv.BF16, [NB, Hkv, bs, D])
    vp = R(FAKE + (2 << 30), pkv.BF16, [NB, Hkv, bs, D])
    out = R(FAKE + (3 << 30), pkv.F32, [B, Hq, D])
    table = FAKE + (4 << 30)
    lens = [4096] * B
    # partials of 64 splits per row exceed the 16 MiB scratch
    assert pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, 64) > pkv.NOALLOC_SCRATCH_BYTES
    assert status_of(pkv.paged_decode_attention_noalloc, q, kp, vp, table, maxb, bs, lens, out,
                     num_splits=64) == pkv.E_NOMEM
    assert "static scratch" in pkv.last_error()
    assert status_of(pkv.paged_decode_attention_noalloc, q, kp, vp, table, maxb, bs, [0] * B, out) == pkv.E_CAPACITY
    assert status_of(pkv.paged_decode_attention_noalloc, q, kp, vp, table, maxb, 8, lens, out) == pkv.E_LAYOUT
    assert status_of(pkv.paged_decode_attention_noalloc, R(FAKE, pkv.F16, [B, Hq, D]), kp, vp, table, maxb, bs,
                     lens, out) == pkv.E_DTYPE


# --------------------------------------------------------------------------- device-driven step
def test_device_step_entry_points_validate_host_arguments():
    """Shapes, dtypes, bounds, bindings and aliasing of the *_dev calls are checked on the host."""
    B, H, cap, D = 2, 2, 64, 128
    kc = R(FAKE, pkv.BF16, [B, H, cap, D])
    vc = R(FAKE + (1 << 24), pkv.BF16, [B, H, cap, D])
    kv = R(FAKE + (2 << 24), pkv.BF16, [B, H, 1, D])
    vv = R(FAKE + (3 << 24), pkv.BF16, [B, H, 1, D])
    pos, st = FAKE + (4 << 24), FAKE + (5 << 24)
    f = pkv.cache_update_kv_dev
    with pkv.bind_writable(kc), pkv.bind_writable(vc):
        assert status_of(f, kc, vc, kv, vv, pos, 1, None) == pkv.E_ARG                    # status required
        assert status_of(f, kc, vc, kv, vv, None, 1, st) == pkv.E_ARG                     # position required
        assert status_of(f, kc, vc, R(kv.ptr, pkv.BF16, [B, H, 65, D]), R(vv.ptr, pkv.BF16, [B, H, 65, D]),
                         pos, 65, st) == pkv.E_ARG                                        # at most 64 tokens
        assert status_of(f, kc, vc, kv, R(vv.ptr, pkv.F16, vv.shape), pos, 1, st) == pkv.E_DTYPE
        assert status_of(f, kc, R(vc.ptr, pkv.BF16, [B, H, cap - 1, D]), kv, vv, pos, 1, st) == pkv.E_LAYOUT
        assert status_of(f, kc, vc, R(kv.ptr + 2, pkv.BF16, kv.shape), vv, pos, 1, st) == pkv.E_LAYOUT
        assert status_of(f, kc, vc, kv, vv, kc.ptr + 64, 1, st) == pkv.E_ALIAS            # position inside the cache
        assert status_of(f, kc, vc, R(kc.ptr, pkv.BF16, kv.shape), vv, pos, 1, st) == pkv.E_ALIAS
    assert status_of(f, kc, vc, kv, vv, pos, 1, st) == pkv.E_READONLY                     # no writable binding
    # paged: a pool handle matching the pools
    kp = R(FAKE, pkv.BF16, [32, H, 16, D])
    vp = R(FAKE + (1 << 24), pkv.BF16, [32, H, 16, D])
    with pkv.bind_writable(kp), pkv.bind_writable(vp):
        pool = pkv.Pool(32, 16, B, 4)
        assert status_of(pkv.paged_cache_update_kv_dev, None, kp, vp, FAKE + (6 << 24), kv, vv, pos, 1, st) \
            == pkv.E_ARG
        assert status_of(pkv.paged_cache_update_kv_dev, pkv.Pool(16, 16, B, 4), kp, vp, FAKE + (6 << 24), kv, vv,
                         pos, 1, st) == pkv.E_LAYOUT
    # attention: max_len within the capacity, status required
    q = R(FAKE + (7 << 24), pkv.BF16, [B, 4, D])
    out = R(FAKE + (8 << 24), pkv.BF16, [B, 4, D])
    ws = R(FAKE + (9 << 24), pkv.U8, [1 << 20])
    g = pkv.decode_attention_dev
    assert status_of(g, q, kc, vc, pos, cap + 1, out, st, ws) == pkv.E_CAPACITY
    assert status_of(g, q, kc, vc, pos, 0, out, st, ws) == pkv.E_CAPACITY
    assert status_of(g, q, kc, vc, pos, cap, out, None, ws) == pkv.E_ARG
    assert status_of(g, q, kc, vc, None, cap, out, st, ws) == pkv.E_ARG
    assert status_of(g, q, kc, vc, pos, cap, out, out.ptr, ws) == pkv.E_ALIAS
    assert status_of(pkv.paged_decode_attention_dev, q, kp, vp, FAKE + (6 << 24), 4, 16, pos, 65, out, st, ws) \
        == pkv.E_CAPACITY
    assert status_of(pkv.advance, None, 1, n=1) == pkv.E_ARG
    assert status_of(pkv.sample_dev, R(FAKE, pkv.F32, [2, 100]), 0.5, 0, FAKE + 512,
                     FAKE + (1 << 24), R(FAKE + 256, pkv.U8, [1 << 16])) == pkv.E_ALIAS


def test_empty_batches_of_the_new_calls_do_nothing():
    """B = 0 through the fused step, its device-position form and the split chunk attention: every check passes
    and nothing is launched (this runs without a GPU)."""
    kc = R(FAKE + 0x100000, pkv.BF16, [0, 2, 64, 128])
    vc = R(FAKE + 0x900000, pkv.BF16, [0, 2, 64, 128])
    kv = R(FAKE + 0x1100000, pkv.BF16, [0, 2, 1, 128])
    vv = R(FAKE + 0x1200000, pkv.BF16, [0, 2, 1, 128])
    q = R(FAKE + 0x1300000, pkv.BF16, [0, 8, 128])
    out = R(FAKE + 0x1400000, pkv.F32, [0, 8, 128])
    pkv.decode_step(kc, vc, kv, vv, [], 1, q, out)
    pkv.decode_step_dev(kc, vc, kv, vv, FAKE + 0x1500000, 1, q, 64, out, FAKE + 0x1600000)
    qc = R(FAKE + 0x3000000, pkv.BF16, [0, 4, 32, 128])
    oc = R(FAKE + 0x3400000, pkv.BF16, [0, 4, 32, 128])
    kp = R(FAKE + 0x100000, pkv.BF16, [32, 2, 16, 128])
    vp = R(FAKE + 0x900000, pkv.BF16, [32, 2, 16, 128])
    table = R(FAKE + 0x2000000, pkv.I32, [1, 8])
    pkv.chunk_attention(qc, kp, vp, table, 8, 16, [], oc, num_splits=4)
    assert pkv.chunk_workspace_size(0, 4, 2, 32, 4) == 0
