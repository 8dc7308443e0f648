"""GPU parity of the in-place cache updates, the device page table and the
paged gather: bit-exact against the oracle, pointer identity, untouched
sentinels, and errors that leave every byte unchanged."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import affine as oaffine
from oracle import cache as ocache
from tests.gpu_util import DEV, bits_host, bytes_host, require_gpu, sentinel_dev

pytestmark = pytest.mark.gpu

DTYPES = {"f32": (torch.float32, np.float32), "bf16": (torch.bfloat16, np.uint16),
          "f16": (torch.float16, np.uint16), "u8": (torch.uint8, np.uint8)}


def _values(g, shape, kind):
    if kind == "f32":
        return synth.uniform(g, shape, -1, 1)
    if kind == "bf16":
        return synth.f32_to_bf16_bits(synth.normal(g, shape))
    if kind == "f16":
        return synth.f16_bits(synth.normal(g, shape))
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def _dev(arr, kind):
    tdt, _ = DTYPES[kind]
    if kind in ("bf16", "f16"):
        return torch.from_numpy(arr.view(np.int16)).to(DEV).view(tdt)
    return torch.from_numpy(arr).to(DEV)


@pytest.mark.parametrize("kind,D,n", [("f32", 4, 1), ("bf16", 128, 1), ("bf16", 128, 5), ("f16", 6, 3),
                                      ("u8", 7, 2), ("f32", 64, 33)])
def test_contiguous_update_is_bit_exact_in_place(kind, D, n):
    require_gpu()
    g = synth.rng(600, D, n)
    B, H, cap = 3, 4, 61
    cache = sentinel_dev((B, H, cap, D), DTYPES[kind][0])
    host = bytes_host(cache).view(DTYPES[kind][1]).reshape(B, H, cap, D).copy()
    with pkv.bind_writable(cache):
        for step in range(3):
            pos = g.integers(0, cap - n + 1, size=B).astype(np.int32)
            vals = _values(g, (B, H, n, D), kind)
            out = pkv.cache_update(cache, _dev(vals, kind), pos, n)
            assert out == cache.data_ptr()
            assert ocache.cache_update(host, vals, pos, n) is host
            assert np.array_equal(bytes_host(cache), host.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("kind,D,n", [("bf16", 128, 1), ("f32", 4, 3), ("f16", 6, 2), ("u8", 7, 5)])
def test_paired_contiguous_update_equals_two_single_updates(kind, D, n):
    """pkv_cache_update_kv writes both caches exactly as the oracle's K update and V update would (every
    byte, sentinels included; row sizes that force the 16-, 4- and 1-byte copy widths); a failing call
    writes neither cache."""
    require_gpu()
    g = synth.rng(612, D, n)
    B, H, cap = 3, 2, 37
    kc, vc = sentinel_dev((B, H, cap, D), DTYPES[kind][0]), sentinel_dev((B, H, cap, D), DTYPES[kind][0])
    kh = bytes_host(kc).view(DTYPES[kind][1]).reshape(B, H, cap, D).copy()
    vh = kh.copy()
    with pkv.bind_writable(kc), pkv.bind_writable(vc):
        for step in range(3):
            pos = g.integers(0, cap - n + 1, size=B).astype(np.int32)
            kvals, vvals = _values(g, (B, H, n, D), kind), _values(g, (B, H, n, D), kind)
            pkv.cache_update_kv(kc, vc, _dev(kvals, kind), _dev(vvals, kind), pos, n)
            ocache.cache_update(kh, kvals, pos, n)
            ocache.cache_update(vh, vvals, pos, n)
            assert same_bytes(kc, kh) and same_bytes(vc, vh)
        vals = _dev(_values(g, (B, H, n, D), kind), kind)
        with pytest.raises(pkv.PkvError) as e:
            pkv.cache_update_kv(kc, vc, vals, vals, [0, cap - n + 1, 0], n)
        assert e.value.status == pkv.E_CAPACITY
        assert same_bytes(kc, kh) and same_bytes(vc, vh)


def test_overflow_and_readonly_leave_the_cache_untouched():
    require_gpu()
    cache = sentinel_dev((1, 1, 16, 4), torch.float32)
    vals = torch.ones((1, 1, 1, 4), device=DEV)
    with pkv.bind_writable(cache):
        for t in range(16):
            pkv.cache_update(cache, vals * t, [t], 1)
        before = bytes_host(cache)
        with pytest.raises(pkv.PkvError) as e:
            pkv.cache_update(cache, vals, [16], 1)
        assert e.value.status == pkv.E_CAPACITY
    with pytest.raises(pkv.PkvError) as e:
        pkv.cache_update(cache, vals, [0], 1)              # binding released: read-only now
    assert e.value.status == pkv.E_READONLY
    assert np.array_equal(bytes_host(cache), before)


def _paged_setup(g, NB, H, bs, D, S, maxb, kind="bf16"):
    order = synth.permutation(g, NB)
    lib_pool = pkv.Pool(NB, bs, S, maxb, order)
    ref_pool = ocache.PagePool(NB, bs, S, maxb, order)
    table = torch.full((S, maxb), -1, dtype=torch.int32, device=DEV)
    kv = sentinel_dev((NB, H, bs, D), DTYPES[kind][0])
    host = bytes_host(kv).view(DTYPES[kind][1]).reshape(NB, H, bs, D).copy()
    return lib_pool, ref_pool, table, kv, host


@pytest.mark.parametrize("bs,D", [(16, 128), (4, 8), (32, 64)])
def test_paged_update_and_gather_are_bit_exact(bs, D):
    require_gpu()
    g = synth.rng(601, bs, D)
    B, H, maxb = 4, 3, 12
    NB = B * maxb + 5
    lib_pool, ref_pool, table, kv, host = _paged_setup(g, NB, H, bs, D, B, maxb)
    lengths = np.zeros(B, np.int32)
    with pkv.bind_writable(kv):
        for n in [1, bs + 3, 1, 2 * bs - 1, 1]:
            if (lengths + n > maxb * bs).any():
                break
            vals = _values(g, (B, H, n, D), "bf16")
            new = (lengths + n).tolist()
            lib_pool.reserve(range(B), new, table)
            for b in range(B):
                ref_pool.reserve(b, new[b])
            assert np.array_equal(table.cpu().numpy(), ref_pool.table)          # device page table
            assert pkv.paged_cache_update(lib_pool, kv, table, _dev(vals, "bf16"), lengths, n) == kv.data_ptr()
            ocache.paged_cache_update(host, ref_pool.table, vals, lengths, n, bs, held_pages=ref_pool.held)
            lengths += n
            assert np.array_equal(bits_host(kv), host)                         # every byte of the pool
    for b in range(B):
        out = torch.empty((H, int(lengths[b]), D), dtype=torch.bfloat16, device=DEV)
        pkv.paged_gather(kv, table, maxb, b, int(lengths[b]), out)
        assert np.array_equal(bits_host(out), ocache.paged_gather(host, ref_pool.table[b], int(lengths[b]), bs))


@pytest.mark.parametrize("bs,D,kind", [(16, 128, "bf16"), (4, 8, "f32"), (32, 6, "f16")])
def test_paired_kv_update_equals_two_single_updates(bs, D, kind):
    """pkv_paged_cache_update_kv writes both pools exactly as the oracle's K update and V update would
    (every byte of both pools, sentinels included), across page boundaries and for rows whose byte size
    forces the narrower copy widths; a failing call writes neither pool."""
    require_gpu()
    g = synth.rng(611, bs, D)
    B, H, maxb = 3, 2, 10
    NB = B * maxb + 3
    lib_pool, ref_pool, table, kp, khost = _paged_setup(g, NB, H, bs, D, B, maxb, kind)
    vp = sentinel_dev((NB, H, bs, D), DTYPES[kind][0])
    vhost = bytes_host(vp).view(DTYPES[kind][1]).reshape(NB, H, bs, D).copy()
    lengths = np.zeros(B, np.int32)
    with pkv.bind_writable(kp), pkv.bind_writable(vp):
        for n in [1, bs + 3, 2 * bs - 1, 1]:
            kvals, vvals = _values(g, (B, H, n, D), kind), _values(g, (B, H, n, D), kind)
            new = (lengths + n).tolist()
            lib_pool.reserve(range(B), new, table)
            for b in range(B):
                ref_pool.reserve(b, new[b])
            pkv.paged_cache_update_kv(lib_pool, kp, vp, table, _dev(kvals, kind), _dev(vvals, kind), lengths, n)
            ocache.paged_cache_update(khost, ref_pool.table, kvals, lengths, n, bs, held_pages=ref_pool.held)
            ocache.paged_cache_update(vhost, ref_pool.table, vvals, lengths, n, bs, held_pages=ref_pool.held)
            lengths += n
            assert same_bytes(kp, khost) and same_bytes(vp, vhost)
        # past the reserved pages: rejected before any write, both pools unchanged
        vals = _dev(_values(g, (B, H, bs, D), kind), kind)
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_cache_update_kv(lib_pool, kp, vp, table, vals, vals, lengths, bs)
        assert e.value.status == pkv.E_PAGE
        assert same_bytes(kp, khost) and same_bytes(vp, vhost)


def same_bytes(dev, host):
    return np.array_equal(bytes_host(dev), np.ascontiguousarray(host).view(np.uint8).reshape(-1))


def test_paged_update_past_reserved_pages_fails_without_writing():
    require_gpu()
    g = synth.rng(602)
    lib_pool, ref_pool, table, kv, host = _paged_setup(g, 8, 1, 4, 8, 1, 4)
    lib_pool.reserve([0], [4], table)
    vals = _dev(_values(g, (1, 1, 2, 8), "bf16"), "bf16")
    with pkv.bind_writable(kv):
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_cache_update(lib_pool, kv, table, vals, [3], 2)
        assert e.value.status == pkv.E_PAGE
    assert np.array_equal(bits_host(kv), host)


def test_release_resets_the_device_row():
    require_gpu()
    pool = pkv.Pool(16, 4, 2, 4, synth.permutation(synth.rng(603), 16))
    table = torch.full((2, 4), -1, dtype=torch.int32, device=DEV)
    pool.reserve([0, 1], [9, 16], table)
    pool.release(0, table)
    t = table.cpu().numpy()
    assert (t[0] == -1).all() and np.array_equal(t, pool.table())
    assert pool.free_count() == 16 - 4


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_int4_append_is_bit_exact(src):
    require_gpu()
    g = synth.rng(604, 0 if src == "f32" else 1)
    B, H, D, bs, maxb = 3, 2, 128, 16, 4
    NB = B * maxb
    order = synth.permutation(g, NB)
    lib_pool = pkv.Pool(NB, bs, B, maxb, order)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    codes = sentinel_dev((NB, H, bs, D // 2), torch.uint8)
    params = sentinel_dev((NB, H, bs, D // 32, 2), torch.float16)
    host_c = bytes_host(codes).reshape(NB, H, bs, D // 2).copy()
    host_p = bits_host(params).reshape(NB, H, bs, D // 32, 2).copy()
    s_bits = int(synth.f16_bits(np.float32(0.0625)))
    z_bits = int(synth.f16_bits(np.float32(8.0)))
    s = float(np.uint16(s_bits).view(np.float16))
    lengths = np.array([0, 5, 17], np.int32)
    lib_pool.reserve(range(B), lengths.tolist(), table)
    for b in range(B):
        ref_pool.reserve(b, int(lengths[b]))
    with pkv.bind_writable(codes), pkv.bind_writable(params):
        for n in [1, 7, 20]:
            x = synth.uniform(g, (B, H, n, D), -0.7, 0.7)
            x[..., :16] = (np.round(x[..., :16] / s) + 0.5) * s            # exact ties: half to even
            x[..., 16:20] = np.array([9.0, -9.0, 0.5 * s, -0.5 * s], np.float32)  # saturation
            if src == "bf16":
                xb = synth.f32_to_bf16_bits(x)
                x = synth.bf16_bits_to_f32(xb)
                dev = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
            else:
                dev = torch.from_numpy(x).to(DEV)
            new = (lengths + n).tolist()
            lib_pool.reserve(range(B), new, table)
            for b in range(B):
                ref_pool.reserve(b, new[b])
            pkv.paged_cache_update_int4(lib_pool, codes, params, table, dev, s_bits, z_bits, lengths, n)
            c_rows, p_rows = oaffine.int4_quantize_rows(x, s_bits, z_bits)
            ocache.paged_cache_update(host_c, ref_pool.table, c_rows, lengths, n, bs, ref_pool.held)
            ocache.paged_cache_update(host_p.reshape(NB, H, bs, -1), ref_pool.table, p_rows.reshape(B, H, n, -1),
                                      lengths, n, bs, ref_pool.held)
            lengths += n
            assert np.array_equal(bytes_host(codes).reshape(host_c.shape), host_c)
            assert np.array_equal(bits_host(params), host_p)
