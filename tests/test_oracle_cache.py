"""Pins of the oracle's in-place update, page pool and paged mapping (CPU only).

Each check ties the oracle to something other than its own code: the pages'
contract (alias identity, capacity error with no write, in-place pages,
all-or-nothing page allocation), sentinel bytes, pool invariants, and the
equality of two independently written layouts (contiguous vs paged).
"""
import numpy as np
import pytest

import synth
from oracle import cache

SENTINEL = np.uint8(0xA5)


def _sentinel_cache(shape, dtype):
    c = np.empty(shape, dtype=dtype)
    c.view(np.uint8)[...] = SENTINEL
    return c


def test_update_writes_only_the_range_and_returns_the_same_storage():
    g = synth.rng(100, 0)
    B, H, cap, D, n = 3, 2, 11, 5, 3
    c = _sentinel_cache((B, H, cap, D), np.float32)
    before = c.copy()
    vals = synth.uniform(g, (B, H, n, D), -1, 1)
    pos = np.array([0, 4, 8])
    out = cache.cache_update(c, vals, pos, n)
    assert out is c                                    # the result aliases the input
    for b in range(B):
        inside = np.zeros(cap, bool)
        inside[pos[b]:pos[b] + n] = True
        assert np.array_equal(c[b][:, inside], vals[b])            # new rows are the values
        assert c[b][:, ~inside].tobytes() == before[b][:, ~inside].tobytes()   # the rest untouched


@pytest.mark.parametrize("pos,n", [([9, 0, 0], 3), ([-1, 0, 0], 1), ([0, 0, 12], 0)])
def test_overflow_is_an_error_and_writes_nothing(pos, n):
    c = _sentinel_cache((3, 2, 11, 5), np.float32)
    before = c.tobytes()
    with pytest.raises(cache.CapacityError):
        cache.cache_update(c, np.zeros((3, 2, n, 5), np.float32), pos, n)
    assert c.tobytes() == before


def test_zero_length_update_at_capacity_is_allowed():
    c = _sentinel_cache((1, 1, 4, 2), np.float32)
    before = c.tobytes()
    assert cache.cache_update(c, np.zeros((1, 1, 0, 2), np.float32), [4], 0) is c
    assert c.tobytes() == before


def test_tiny_fixture_fills_capacity_then_the_next_step_fails():
    """1-token prompt + 15 appends fill capacity 16; the next append overflows."""
    g = synth.rng(0, 1)
    c = _sentinel_cache((1, 1, 16, 4), np.float32)
    for t in range(16):
        cache.cache_update(c, synth.uniform(g, (1, 1, 1, 4), -1, 1), [t], 1)
    snapshot = c.tobytes()
    with pytest.raises(cache.CapacityError):
        cache.cache_update(c, np.ones((1, 1, 1, 4), np.float32), [16], 1)
    assert c.tobytes() == snapshot


def test_pool_reserve_takes_only_missing_pages_all_or_nothing():
    order = synth.permutation(synth.rng(101), 10)
    pool = cache.PagePool(10, 4, 3, 8, order)
    assert pool.reserve(0, 5) == list(order[:2])       # ceil(5/4) = 2 pages
    assert pool.reserve(0, 8) == []                    # still 2 pages: nothing new
    assert pool.reserve(0, 9) == [order[2]]            # one missing page
    assert pool.reserve(1, 1) == [order[3]]
    free_before, table_before = list(pool.free), pool.table.copy()
    with pytest.raises(cache.PoolExhausted):
        pool.reserve(2, 4 * 7)                         # needs 7 > 6 free
    assert pool.free == free_before and np.array_equal(pool.table, table_before)
    with pytest.raises(cache.PageError):
        pool.reserve(2, 4 * 8 + 1)                     # more than max_blocks_per_seq
    held = pool.table[pool.table >= 0]
    assert len(set(held.tolist())) == held.size        # no physical id handed out twice
    assert pool.used() + len(pool.free) == 10
    pool.release(0)
    assert pool.used() + len(pool.free) == 10 and pool.held[0] == 0
    assert sorted(pool.free + pool.table[pool.table >= 0].tolist()) == list(range(10))


def test_paged_layout_matches_the_contiguous_layout():
    """Two independently written layouts hold the same logical rows after the same appends."""
    g = synth.rng(102)
    B, H, D, bs, cap = 3, 2, 6, 4, 23
    NB = B * cache.pages_for(cap, bs) + 3
    pool_arr = _sentinel_cache((NB, H, bs, D), np.float32)
    pp = cache.PagePool(NB, bs, B, cache.pages_for(cap, bs), synth.permutation(g, NB))
    contig = _sentinel_cache((B, H, cap, D), np.float32)
    lengths = np.zeros(B, np.int64)
    for n in [1, 5, 3, 1, 7, 2]:
        if (lengths + n > cap).any():
            break
        vals = synth.uniform(g, (B, H, n, D), -1, 1)
        for b in range(B):
            pp.reserve(b, int(lengths[b] + n))
        cache.cache_update(contig, vals, lengths, n)
        cache.paged_cache_update(pool_arr, pp.table, vals, lengths, n, bs, held_pages=pp.held)
        lengths += n
    for b in range(B):
        got = cache.paged_gather(pool_arr, pp.table[b], int(lengths[b]), bs)
        assert got.tobytes() == contig[b, :, :lengths[b]].tobytes()
    # pages nobody reserved keep their sentinel bytes
    held = set(pp.table[pp.table >= 0].tolist())
    for phys in range(NB):
        if phys not in held:
            assert (pool_arr[phys].view(np.uint8) == SENTINEL).all()


def test_partial_page_is_filled_in_place():
    pool_arr = _sentinel_cache((4, 1, 4, 2), np.float32)
    pp = cache.PagePool(4, 4, 1, 4, [2, 0, 3, 1])
    pp.reserve(0, 3)
    cache.paged_cache_update(pool_arr, pp.table, np.ones((1, 1, 3, 2), np.float32), [0], 3, 4, pp.held)
    before = pool_arr.copy()
    pp.reserve(0, 4)                                   # still one page: nothing allocated
    assert pp.held[0] == 1
    cache.paged_cache_update(pool_arr, pp.table, np.full((1, 1, 1, 2), 2, np.float32), [3], 1, 4, pp.held)
    assert np.array_equal(pool_arr[2, 0, 3], [2, 2])   # slot 3 of physical page 2
    mask = np.ones(pool_arr.shape, bool)
    mask[2, 0, 3] = False
    assert pool_arr[mask].tobytes() == before[mask].tobytes()


def test_paged_update_past_reserved_pages_is_an_error_with_no_write():
    pool_arr = _sentinel_cache((4, 1, 4, 2), np.float32)
    pp = cache.PagePool(4, 4, 1, 4)
    pp.reserve(0, 4)
    before = pool_arr.tobytes()
    with pytest.raises(cache.PageError):
        cache.paged_cache_update(pool_arr, pp.table, np.ones((1, 1, 2, 2), np.float32), [3], 2, 4, pp.held)
    assert pool_arr.tobytes() == before
