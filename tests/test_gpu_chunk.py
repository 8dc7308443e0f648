"""GPU parity of the chunked in-place append + causal chunk attention (MFMA)
against the float64 oracle, and its reduction to single-token decode."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import numeric as onum
from tests.gpu_util import (DEV, assert_bf16_pv_bound, bf16_dev, bits_host, rel_err_rows, require_gpu,
                            workspace)

pytestmark = pytest.mark.gpu


BF16_NAN = 0x7FC0
def _assert_chunk_bound(got, ref, qh, K, V, p0, left_window=-1):
    """The bf16 P.V bound (`assert_bf16_pv_bound`) for every query of a chunk: query t at p0 + t sees keys
    [p0 + t - W, p0 + t] (all earlier ones without a window)."""
    Hq, C, D = got.shape
    G = Hq // K.shape[0]
    pos = p0 + np.arange(C)
    keys = np.arange(K.shape[1])
    vis = keys[None, :] <= pos[:, None]
    if left_window >= 0:
        vis &= keys[None, :] >= (pos - left_window)[:, None]
    for h in range(Hq):
        s = np.where(vis, qh[h] @ K[h // G].T / np.sqrt(D), -np.inf)
        assert_bf16_pv_bound(got[h], ref[h], s, np.broadcast_to(V[h // G], (C,) + V[h // G].shape))


def _chunk(d, q, out, maxb, bs, p0, W=-1, S=1):
    """Chunk attention on `d`'s pools; S != 1 splits every workgroup's key range (0: library choice)."""
    B, Hq, C, _ = out.shape
    Hkv = d["kd"].shape[1]
    ws = None if S == 1 else workspace(pkv.chunk_workspace_size(B, Hq, Hkv, C, S))
    pkv.chunk_attention(q, d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"], left_window=W,
                        workspace=ws, num_splits=S)


def _setup(seed, B, Hq, Hkv, D, bs, p0, C, maxb, fill=0):
    """Prefix of p0[b] tokens already in the pages; returns device state and the host mirror.  Slots no
    append writes (past a row's length, and unreserved pages) hold the bf16 bits `fill`."""
    g = synth.rng(seed)
    NB = int(sum(-(-(int(x) + C) // bs) for x in p0)) + 2
    order = synth.permutation(g, NB)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    lib_pool = pkv.Pool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    kp = np.full((NB, Hkv, bs, D), fill, np.uint16)
    vp = np.full_like(kp, fill)
    for b in range(B):
        ref_pool.reserve(b, int(p0[b]) + C)
        L = int(p0[b])
        if L:
            kr = synth.f32_to_bf16_bits(synth.normal(synth.rng(seed, 1, b), (1, Hkv, L, D)))
            vr = synth.f32_to_bf16_bits(synth.normal(synth.rng(seed, 2, b), (1, Hkv, L, D)))
            ocache.paged_cache_update(kp, ref_pool.table[b:b + 1], kr, [0], L, bs)
            ocache.paged_cache_update(vp, ref_pool.table[b:b + 1], vr, [0], L, bs)
    lib_pool.reserve(range(B), (np.asarray(p0) + C).tolist(), table)
    assert np.array_equal(table.cpu().numpy(), ref_pool.table)
    new_k = synth.f32_to_bf16_bits(synth.normal(synth.rng(seed, 3), (B, Hkv, C, D)))
    new_v = synth.f32_to_bf16_bits(synth.normal(synth.rng(seed, 4), (B, Hkv, C, D)))
    q = synth.f32_to_bf16_bits(synth.normal(synth.rng(seed, 5), (B, Hq, C, D)))
    return dict(kp=kp, vp=vp, kd=bf16_dev(kp), vd=bf16_dev(vp), table=table, lib_pool=lib_pool,
                ref_pool=ref_pool, new_k=new_k, new_v=new_v, q=q)


@pytest.mark.parametrize("G,C,bs", [(2, 100, 16), (1, 64, 16), (4, 7, 16), (8, 130, 32), (2, 1, 16), (2, 300, 8),
                                    (2, 100, 4)])
def test_chunk_append_and_causal_attention_match_oracle(G, C, bs):
    require_gpu()
    B, Hkv, D = 3, 2, 128
    Hq = Hkv * G
    p0 = np.array([0, 37, 200], np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(900 + G + C, B, Hq, Hkv, D, bs, p0, C, maxb)
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update(d["lib_pool"], d["kd"], d["table"], bf16_dev(d["new_k"]), p0, C)
        pkv.paged_cache_update(d["lib_pool"], d["vd"], d["table"], bf16_dev(d["new_v"]), p0, C)
    ocache.paged_cache_update(d["kp"], d["ref_pool"].table, d["new_k"], p0, C, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp"], d["ref_pool"].table, d["new_v"], p0, C, bs, d["ref_pool"].held)
    assert np.array_equal(bits_host(d["kd"]), d["kp"]) and np.array_equal(bits_host(d["vd"]), d["vp"])
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    pkv.chunk_attention(bf16_dev(d["q"]), d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"])
    got = onum.bf16_to_f64(bits_host(out))
    qh = onum.bf16_to_f64(d["q"])
    for b in range(B):
        L = int(p0[b]) + C
        K = onum.bf16_to_f64(ocache.paged_gather(d["kp"], d["ref_pool"].table[b], L, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(d["vp"], d["ref_pool"].table[b], L, bs))
        ref = oattn.chunk_attention(qh[b], K, V, int(p0[b]))
        _assert_chunk_bound(got[b], ref, qh[b], K, V, int(p0[b]))


@pytest.mark.parametrize("W,G,C", [(0, 2, 100), (5, 2, 100), (63, 4, 40), (64, 1, 300), (150, 2, 300),
                                   (1000, 8, 64)])
def test_chunk_left_window_matches_oracle(W, G, C):
    """A left window W: query t sees keys [p0 + t - W, p0 + t]; tiles before every window are skipped."""
    require_gpu()
    B, Hkv, D, bs = 3, 2, 128, 16
    Hq = Hkv * G
    p0 = np.array([0, 37, 400], np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(950 + W + C, B, Hq, Hkv, D, bs, p0, C, maxb)
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update(d["lib_pool"], d["kd"], d["table"], bf16_dev(d["new_k"]), p0, C)
        pkv.paged_cache_update(d["lib_pool"], d["vd"], d["table"], bf16_dev(d["new_v"]), p0, C)
    ocache.paged_cache_update(d["kp"], d["ref_pool"].table, d["new_k"], p0, C, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp"], d["ref_pool"].table, d["new_v"], p0, C, bs, d["ref_pool"].held)
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    pkv.chunk_attention(bf16_dev(d["q"]), d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"],
                        left_window=W)
    got = onum.bf16_to_f64(bits_host(out))
    qh = onum.bf16_to_f64(d["q"])
    for b in range(B):
        L = int(p0[b]) + C
        K = onum.bf16_to_f64(ocache.paged_gather(d["kp"], d["ref_pool"].table[b], L, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(d["vp"], d["ref_pool"].table[b], L, bs))
        ref = oattn.chunk_attention(qh[b], K, V, int(p0[b]), left_window=W)
        _assert_chunk_bound(got[b], ref, qh[b], K, V, int(p0[b]), W)


@pytest.mark.parametrize("S,G,C,bs,W", [(2, 2, 100, 16, -1), (3, 1, 64, 16, -1), (5, 4, 130, 32, -1),
                                       (64, 2, 100, 16, -1), (3, 2, 300, 8, 150), (4, 8, 64, 16, 1000),
                                       (7, 2, 1, 16, -1), (2, 2, 90, 4, 63), (0, 2, 256, 16, -1)])
def test_split_over_keys_matches_oracle(S, G, C, bs, W):
    """The key range of every workgroup cut into S parts whose partials the log-sum-exp merge combines
    (S = 0: the library's choice, which splits this small batch).  Parts hold whole tiles, a part may hold
    none (S = 64 against rows of two tiles), and a query may see no key of a part (the diagonal tiles and
    the window's first tiles)."""
    require_gpu()
    B, Hkv, D = 3, 2, 128
    Hq = Hkv * G
    p0 = np.array([0, 37, 1200], np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(1040 + S + G + C, B, Hq, Hkv, D, bs, p0, C, maxb)
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update_kv(d["lib_pool"], d["kd"], d["vd"], d["table"], bf16_dev(d["new_k"]),
                                  bf16_dev(d["new_v"]), p0, C)
    ocache.paged_cache_update(d["kp"], d["ref_pool"].table, d["new_k"], p0, C, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp"], d["ref_pool"].table, d["new_v"], p0, C, bs, d["ref_pool"].held)
    if S == 0:
        assert pkv.chunk_workspace_size(B, Hq, Hkv, C, 0) > 0
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    _chunk(d, bf16_dev(d["q"]), out, maxb, bs, p0, W, S)
    got = onum.bf16_to_f64(bits_host(out))
    qh = onum.bf16_to_f64(d["q"])
    for b in range(B):
        L = int(p0[b]) + C
        K = onum.bf16_to_f64(ocache.paged_gather(d["kp"], d["ref_pool"].table[b], L, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(d["vp"], d["ref_pool"].table[b], L, bs))
        ref = oattn.chunk_attention(qh[b], K, V, int(p0[b]), left_window=W)
        _assert_chunk_bound(got[b], ref, qh[b], K, V, int(p0[b]), W)


def test_split_workspace_errors():
    require_gpu()
    B, Hkv, G, D, bs, C = 1, 2, 2, 128, 16, 64
    Hq = Hkv * G
    p0 = np.array([500], np.int32)
    maxb = -(-(int(p0[0]) + C) // bs) + 1
    d = _setup(1060, B, Hq, Hkv, D, bs, p0, C, maxb)
    q = bf16_dev(d["q"])
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    need = pkv.chunk_workspace_size(B, Hq, Hkv, C, 4)
    ws = workspace(need + 512)
    cases = [(None, 4, pkv.E_NOMEM), (ws[:need - 256], 4, pkv.E_NOMEM), (ws[128:need + 128], 4, pkv.E_ARG),
             (ws, 65, pkv.E_ARG), (ws, -1, pkv.E_ARG)]
    for w, S, status in cases:
        with pytest.raises(pkv.PkvError) as e:
            pkv.chunk_attention(q, d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"],
                                workspace=w, num_splits=S)
        assert e.value.status == status, (S, status)
    big = workspace(need + out.numel() * 2)       # the workspace may not overlap the output
    inner = big[:out.numel() * 2].view(torch.bfloat16).view(out.shape)
    with pytest.raises(pkv.PkvError) as e:
        pkv.chunk_attention(q, d["kd"], d["vd"], d["table"], maxb, bs, p0, inner, pool=d["lib_pool"],
                            workspace=big, num_splits=4)
    assert e.value.status == pkv.E_ALIAS


@pytest.mark.parametrize("rise", [10.0, 14.0])
def test_running_max_rise_in_a_later_tile(rise):
    """One prefix key in a later, unmasked tile outscores the rest by about `rise` log2 units (the typical
    maximum of the other keys is about 3.6).  At 10 the rise above the running max stays mostly inside the
    lazy margin of 8, so probabilities up to about 2^8 are accumulated under the old max; at 14 it passes
    the margin and the max moves, rescaling the output.  Both must match the oracle."""
    require_gpu()
    B, Hkv, D, bs, G, C, d0 = 2, 2, 128, 16, 2, 64, 7
    Hq = Hkv * G
    p0 = np.array([300, 700], np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(1010 + int(rise), B, Hq, Hkv, D, bs, p0, C, maxb)
    d["q"][..., d0] = synth.f32_to_bf16_bits(np.float32(4.0))
    d["new_k"][..., d0] = 0
    table = d["ref_pool"].table
    lift = synth.f32_to_bf16_bits(np.float32(rise * np.sqrt(D) / (4.0 * np.log2(np.e))))
    for b, p in ((0, 150), (1, 400)):
        for pos in range(int(p0[b])):
            d["kp"][int(table[b, pos // bs]), :, pos % bs, d0] = 0
        d["kp"][int(table[b, p // bs]), :, p % bs, d0] = lift
    d["kd"] = bf16_dev(d["kp"])
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update(d["lib_pool"], d["kd"], d["table"], bf16_dev(d["new_k"]), p0, C)
        pkv.paged_cache_update(d["lib_pool"], d["vd"], d["table"], bf16_dev(d["new_v"]), p0, C)
    ocache.paged_cache_update(d["kp"], table, d["new_k"], p0, C, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp"], table, d["new_v"], p0, C, bs, d["ref_pool"].held)
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    pkv.chunk_attention(bf16_dev(d["q"]), d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"])
    got = onum.bf16_to_f64(bits_host(out))
    qh = onum.bf16_to_f64(d["q"])
    for b in range(B):
        L = int(p0[b]) + C
        K = onum.bf16_to_f64(ocache.paged_gather(d["kp"], table[b], L, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(d["vp"], table[b], L, bs))
        ref = oattn.chunk_attention(qh[b], K, V, int(p0[b]))
        _assert_chunk_bound(got[b], ref, qh[b], K, V, int(p0[b]))


def test_last_chunk_query_equals_decode():
    require_gpu()
    B, Hkv, G, D, bs, C = 2, 2, 2, 128, 16, 48
    Hq = Hkv * G
    p0 = np.array([10, 333], np.int32)
    maxb = 30
    d = _setup(950, B, Hq, Hkv, D, bs, p0, C, maxb)
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update(d["lib_pool"], d["kd"], d["table"], bf16_dev(d["new_k"]), p0, C)
        pkv.paged_cache_update(d["lib_pool"], d["vd"], d["table"], bf16_dev(d["new_v"]), p0, C)
    q = bf16_dev(d["q"])
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    pkv.chunk_attention(q, d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"])
    dec = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    lens = (p0 + C).tolist()
    pkv.paged_decode_attention(q[:, :, -1, :].contiguous(), d["kd"], d["vd"], d["table"], maxb, bs, lens, dec,
                               workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs)), pool=d["lib_pool"])
    torch.cuda.synchronize()
    last = onum.bf16_to_f64(bits_host(out[:, :, -1, :].contiguous()))
    assert rel_err_rows(last, dec.double().cpu().numpy()) <= 2e-2


def test_chunk_capacity_and_page_errors():
    require_gpu()
    B, Hkv, D, bs, C = 1, 1, 128, 16, 20
    d = _setup(960, B, 2, Hkv, D, bs, np.array([5], np.int32), C, 2)
    out = torch.empty((B, 2, C, D), dtype=torch.bfloat16, device=DEV)
    q = bf16_dev(d["q"])
    with pytest.raises(pkv.PkvError) as e:
        pkv.chunk_attention(q, d["kd"], d["vd"], d["table"], 2, bs, [13], out, pool=d["lib_pool"])
    assert e.value.status == pkv.E_CAPACITY
    small = pkv.Pool(d["lib_pool"].num_blocks, bs, 1, 2)
    small.reserve([0], [16])
    with pytest.raises(pkv.PkvError) as e:
        pkv.chunk_attention(q, d["kd"], d["vd"], d["table"], 2, bs, [5], out, pool=small)
    assert e.value.status == pkv.E_PAGE


@pytest.mark.parametrize("W,G,C,bs,S", [(-1, 2, 300, 16, 1), (-1, 4, 130, 32, 1), (-1, 1, 64, 16, 1),
                                        (37, 2, 300, 16, 1), (200, 8, 100, 16, 1), (-1, 2, 300, 16, 3),
                                        (37, 2, 300, 16, 2)])
def test_planted_key_marks_the_causal_and_window_edges(W, G, C, bs, S):
    """Every query carries 4.0 in one dimension and one key per (row, kv head) carries 128.0 there and 0
    elsewhere, so it outscores every other key by e^40.  A query that sees that key must return its V row
    exactly; a query that must not see it (the key lies after the query, or before its window) must return
    bit for bit what it returned before the key was planted.  Keys sit at tile, page and diagonal edges."""
    require_gpu()
    B, Hkv, D, d0 = 3, 2, 128, 5
    Hq = Hkv * G
    p0 = np.array([0, 37, 200], np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(970 + G + C + max(W, 0), B, Hq, Hkv, D, bs, p0, C, maxb)
    d["q"][..., d0] = synth.f32_to_bf16_bits(np.float32(4.0))
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update(d["lib_pool"], d["kd"], d["table"], bf16_dev(d["new_k"]), p0, C)
        pkv.paged_cache_update(d["lib_pool"], d["vd"], d["table"], bf16_dev(d["new_v"]), p0, C)
    q = bf16_dev(d["q"])
    base = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    _chunk(d, q, base, maxb, bs, p0, W, S)
    base_h = bits_host(base)
    table = d["ref_pool"].table
    probe = np.zeros(D, np.float32)
    probe[d0] = 128.0
    picks = {}
    for b in range(B):
        L = int(p0[b]) + C
        cands = sorted({x for x in (0, 15, 16, 63, 64, int(p0[b]), int(p0[b]) + 1, int(p0[b]) + 31, int(p0[b]) + 32,
                                    int(p0[b]) + 63, int(p0[b]) + 64, int(p0[b]) + C // 2, L - 1) if 0 <= x < L})
        for kvh in range(Hkv):
            p = cands[(b * Hkv + kvh) * 5 % len(cands)]
            picks[(b, kvh)] = p
            d["kd"][int(table[b, p // bs]), kvh, p % bs] = bf16_dev(synth.f32_to_bf16_bits(probe))
    out = torch.empty_like(base)
    _chunk(d, q, out, maxb, bs, p0, W, S)
    got = bits_host(out)
    vh = bits_host(d["vd"])
    seen = unseen = 0
    for (b, kvh), p in picks.items():
        vrow = vh[int(table[b, p // bs]), kvh, p % bs]
        for t in range(C):
            pos = int(p0[b]) + t
            lo = oattn.visible_begin(pos, W)
            for h in range(kvh * G, (kvh + 1) * G):
                if lo <= p <= pos:
                    assert np.array_equal(got[b, h, t], vrow), (b, h, t, p)
                    seen += 1
                else:
                    assert np.array_equal(got[b, h, t], base_h[b, h, t]), (b, h, t, p)
                    unseen += 1
    assert seen and unseen


@pytest.mark.parametrize("G,C,bs,W,S", [(2, 100, 16, -1, 1), (4, 70, 32, -1, 1), (2, 300, 8, -1, 1),
                                        (1, 5, 16, -1, 1), (2, 129, 64, -1, 1), (2, 100, 16, 40, 1),
                                        (4, 90, 4, -1, 1), (2, 100, 16, -1, 3), (4, 90, 4, -1, 2)])
def test_unwritten_slots_are_never_used(G, C, bs, W, S):
    """Every slot no append writes holds a bf16 NaN: the rows past each row's length in its last page, and
    the pages no row holds.  Lengths end inside a page and inside a 64-key tile.  The outputs must be finite
    and match the oracle, which only sees the written rows (a NaN key past the last one is masked; a NaN
    value row times a zero probability would still poison the products, so it must never be read as is)."""
    require_gpu()
    B, Hkv, D = 3, 2, 128
    Hq = Hkv * G
    p0 = np.array([3, 41, 190], np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(990 + G + C + bs, B, Hq, Hkv, D, bs, p0, C, maxb, fill=BF16_NAN)
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update(d["lib_pool"], d["kd"], d["table"], bf16_dev(d["new_k"]), p0, C)
        pkv.paged_cache_update(d["lib_pool"], d["vd"], d["table"], bf16_dev(d["new_v"]), p0, C)
    ocache.paged_cache_update(d["kp"], d["ref_pool"].table, d["new_k"], p0, C, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp"], d["ref_pool"].table, d["new_v"], p0, C, bs, d["ref_pool"].held)
    assert np.array_equal(bits_host(d["kd"]), d["kp"]) and np.array_equal(bits_host(d["vd"]), d["vp"])
    assert any((int(x) + C) % bs for x in p0)                     # some row ends inside a page
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    _chunk(d, bf16_dev(d["q"]), out, maxb, bs, p0, W, S)
    got = onum.bf16_to_f64(bits_host(out))
    assert np.isfinite(got).all()
    qh = onum.bf16_to_f64(d["q"])
    for b in range(B):
        L = int(p0[b]) + C
        K = onum.bf16_to_f64(ocache.paged_gather(d["kp"], d["ref_pool"].table[b], L, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(d["vp"], d["ref_pool"].table[b], L, bs))
        assert np.isfinite(K).all() and np.isfinite(V).all()
        ref = oattn.chunk_attention(qh[b], K, V, int(p0[b]), left_window=W)
        _assert_chunk_bound(got[b], ref, qh[b], K, V, int(p0[b]), W)
