"""Parity at the workloads' full sizes, in the launch configuration the bench
uses (library split choice, full pools), on sampled rows the oracle computes
one by one.

Large K/V pools are drawn on the device with a seeded torch generator; the
pages of the sampled rows are read back as oracle inputs before any library
kernel touches them.  The page tables are checked bit for bit against the
oracle's pool on the same hand-out order."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import affine as oaffine
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import numeric as onum
from oracle import sampling as osamp
from synth import workloads
from tests.gpu_util import (DEV, assert_bf16_pv_bound, bf16_dev, bits_host, bytes_host, rel_err_rows, require_gpu,
                            workspace)

pytestmark = pytest.mark.gpu


def _randn_bf16(shape, gen):
    return torch.randn(shape, generator=gen, device=DEV, dtype=torch.bfloat16)


def _pages_host(pool_dev, ids):
    idx = torch.from_numpy(np.asarray(ids, np.int64)).to(DEV)
    return bits_host(pool_dev.index_select(0, idx).contiguous())


F32_TOL = 1e-5          # float32 outputs: the fp32 bar (bf16 inputs are exact, accumulation is float32)


def _bf16_round(x: torch.Tensor) -> np.ndarray:
    return bits_host(x.to(torch.bfloat16))


def _split_edges(L, left_window, tps):
    """Token positions next to the edges the kernel cuts a row at (splits of tps tokens from the window's
    64-aligned base, each split's four wave quarters, 16-token pages): the places an off-by-one would hit.
    Only chooses where probes go; the expected output does not depend on it."""
    lo = oattn.visible_begin(L - 1, left_window)
    base = lo // 64 * 64
    edges = {lo, lo + 1, L - 2, L - 1, base + 15, base + 16}
    for cut in range(base, L, tps):
        for q in range(4):
            e = cut + q * (tps // 4)
            edges.update({e - 1, e, e + 15, e + 16})
    return sorted(e for e in edges if lo <= e < L)


def _auto_tps(L, Hkv):
    """Tokens per split of the library's automatic plan (about 1024 workgroups, at least 384 tokens, 64-token
    quanta); used only to aim probes at split edges."""
    t = -(-int(np.sum(L)) * Hkv // 1024)
    return max(384, -(-t // 64) * 64)


def _plant_probes(spec, kd, nk, qh, table_host, probe_rows, left_window, tps):
    """Give one key per (probe row, kv head) a score far above every other key of the row (the query heads of
    the group all see it), at a position next to a page, split or window edge; with a left window, a key with an
    even larger score just before the window.  The attention output of those heads must then be that token's
    V row.  Returns {(b, kvh): (position, outside position or None)}."""
    G = spec.Hq // spec.Hkv
    q32 = onum.bf16_to_f64(qh)
    planted, k = {}, 0
    for b in probe_rows:
        L = int(spec.lengths[b])
        edges = _split_edges(L, left_window, tps)
        for kvh in range(spec.Hkv):
            pos = edges[(k * 7) % len(edges)]
            k += 1
            dirn = q32[b, kvh * G:(kvh + 1) * G].sum(axis=0)
            lo = oattn.visible_begin(L - 1, left_window)
            out_pos = lo - 1 if lo > 0 else None
            for p, mult in ((pos, 16.0), (out_pos, 32.0)):
                if p is None:
                    continue
                row = synth.f32_to_bf16_bits((dirn * mult).astype(np.float32))
                if p == L - 1:                                   # the token this step appends
                    nk[b, kvh, 0] = bf16_dev(row)
                else:
                    kd[int(table_host[b, p // spec.bs]), kvh, p % spec.bs] = bf16_dev(row)
            planted[(b, kvh)] = (pos, out_pos)
    return planted


def _paged_decode_case(spec, seed, check_rows, probe_rows, left_window=-1):
    """Append one token per row at position L-1 and attend over L tokens (or the last left_window + 1) in the
    bench's launch configuration.  f32 output: the checked rows against the oracle at the fp32 bar, the probe
    rows equal to their planted token's V row.  bf16 output (what the bench times): the f32 result rounded."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    B, Hq, Hkv, D, bs, NB, maxb = spec.B, spec.Hq, spec.Hkv, spec.D, spec.bs, spec.NB, spec.maxb
    L = spec.lengths.astype(np.int32)
    kd, vd = _randn_bf16((NB, Hkv, bs, D), gen), _randn_bf16((NB, Hkv, bs, D), gen)
    q = _randn_bf16((B, Hq, D), gen)
    nk, nv = _randn_bf16((B, Hkv, 1, D), gen), _randn_bf16((B, Hkv, 1, D), gen)
    lib_pool = pkv.Pool(NB, bs, B, maxb, spec.order)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, spec.order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), L.tolist(), table)
    for b in range(B):
        ref_pool.reserve(b, int(L[b]))
    assert np.array_equal(table.cpu().numpy(), ref_pool.table)
    pt = ref_pool.table
    qh = bits_host(q)
    planted = _plant_probes(spec, kd, nk, qh, pt, probe_rows, left_window, _auto_tps(L, Hkv))
    host = {}
    for b in check_rows:
        ids = ref_pool.table[b, :spec.pages(b)]
        host[b] = (ids, _pages_host(kd, ids), _pages_host(vd, ids))
    nkh, nvh = bits_host(nk), bits_host(nv)

    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, int(L.max())))
    pos = (L - 1).tolist()
    with pkv.bind_writable(kd), pkv.bind_writable(vd):
        pkv.paged_cache_update(lib_pool, kd, table, nk, pos, 1)
        pkv.paged_cache_update(lib_pool, vd, table, nv, pos, 1)
    out32 = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    pkv.paged_decode_attention(q, kd, vd, table, maxb, bs, L.tolist(), out32, ws, pool=lib_pool,
                               left_window=left_window)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    pkv.paged_decode_attention(q, kd, vd, table, maxb, bs, L.tolist(), out, ws, pool=lib_pool,
                               left_window=left_window)
    assert np.array_equal(bits_host(out), _bf16_round(out32))       # one rounding of the same float32 result
    torch.cuda.synchronize()
    got = out32.double().cpu().numpy()
    G = Hq // Hkv
    worst = 0.0
    for b in check_rows:
        ids, kp, vp = host[b]
        local = np.arange(len(ids), dtype=np.int32)[None]          # the row's pages, renumbered 0..n-1
        ocache.paged_cache_update(kp, local, nkh[b:b + 1], [int(L[b]) - 1], 1, bs)
        ocache.paged_cache_update(vp, local, nvh[b:b + 1], [int(L[b]) - 1], 1, bs)
        assert np.array_equal(_pages_host(kd, ids), kp) and np.array_equal(_pages_host(vd, ids), vp)
        K = onum.bf16_to_f64(ocache.paged_gather(kp, local[0], int(L[b]), bs))
        V = onum.bf16_to_f64(ocache.paged_gather(vp, local[0], int(L[b]), bs))
        qb = onum.bf16_to_f64(qh[b])
        lo = oattn.visible_begin(int(L[b]) - 1, left_window)
        ref = np.stack([oattn.attend(qb[h], K[h // G][lo:], V[h // G][lo:], 1 / np.sqrt(D)) for h in range(Hq)])
        err = rel_err_rows(got[b], ref)
        worst = max(worst, err)
        assert err <= F32_TOL, (b, err)
    for (b, kvh), (p, _outside) in planted.items():
        if p == int(L[b]) - 1:
            want = onum.bf16_to_f64(nvh[b, kvh, 0])
        else:
            want = onum.bf16_to_f64(bits_host(vd[int(pt[b, p // bs]), kvh, p % bs]))
        for h in range(kvh * G, (kvh + 1) * G):
            assert rel_err_rows(got[b, h], want) <= F32_TOL, (b, kvh, h, p)
    print(f"paged decode {spec.name} window {left_window}: {len(check_rows)} rows vs oracle, worst {worst:.2e}; "
          f"{len(planted)} probes exact")
    return got


def _rows_by_rule(L, bs, tps, want=8):
    """Shortest, longest and median rows, plus rows ending on a page edge, one past it, one short of it, and
    next to a split edge, up to `want` distinct rows."""
    order = np.argsort(L, kind="stable")
    picks = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    rules = [lambda x: x % bs == 0, lambda x: x % bs == 1, lambda x: x % bs == bs - 1,
             lambda x: x % tps in (0, 1, tps - 1), lambda x: x % 64 == 0]
    for rule in rules:
        for b in order:
            if rule(int(L[b])) and int(b) not in picks:
                picks.append(int(b))
                break
    for b in order[::max(1, len(order) // want)]:
        if len(picks) >= want:
            break
        if int(b) not in picks:
            picks.append(int(b))
    return sorted(picks[:max(want, len(picks))])


def test_paged32k_full_size_step():
    """The headline workload exactly as bench.py runs it: 32 x 32768 tokens, a full 65536-page pool."""
    require_gpu()
    spec = workloads.paged32k()
    check = [0, 4, 9, 13, 18, 22, 27, 31]
    _paged_decode_case(spec, 3, check, [b for b in range(spec.B) if b not in check])


def test_paged32k_window_full_size():
    """The windowed bench row: the same pool and rows, left window 4095 (the last 4096 tokens); probes also put
    a larger score just before the window, which must not be seen."""
    require_gpu()
    spec = workloads.paged32k()
    check = [0, 7, 15, 16, 23, 31, 3, 28]
    _paged_decode_case(spec, 3, sorted(check), [b for b in range(spec.B) if b not in check], left_window=4095)


def test_paged_lognormal_full_size():
    require_gpu()
    spec = workloads.paged()
    check = _rows_by_rule(spec.lengths, spec.bs, _auto_tps(spec.lengths, spec.Hkv))
    probes = [b for b in range(spec.B) if b not in check][::2]
    _paged_decode_case(spec, 2, check, probes)


def test_contiguous_full_size_32_steps():
    """8 x 8 x 4096 x 128 bf16 caches, initial lengths U{512..4064}, 32 appends + attention each step; the same
    steps through the fused step (`decode_step`) give the same output bits and cache bytes."""
    require_gpu()
    w = workloads.contig()
    B, Hq, Hkv, D, cap, S, seed = w["B"], w["Hq"], w["Hkv"], w["D"], w["cap"], w["steps"], w["seed"]
    L0 = w["lengths"]
    kh = np.zeros((B, Hkv, cap, D), np.uint16)
    vh = np.zeros_like(kh)
    for b in range(B):
        kh[b, :, :L0[b]] = workloads.contig_cache_row(seed, 1, b, Hkv, int(L0[b]), D)
        vh[b, :, :L0[b]] = workloads.contig_cache_row(seed, 2, b, Hkv, int(L0[b]), D)
    kc, vc = bf16_dev(kh), bf16_dev(vh)
    kf, vf = bf16_dev(kh), bf16_dev(vh)              # the same run through the fused step
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device=DEV)
    outf = torch.empty_like(out)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap))
    lengths = L0.copy()
    G = Hq // Hkv
    with pkv.bind_writable(kc), pkv.bind_writable(vc), pkv.bind_writable(kf), pkv.bind_writable(vf):
        for step in range(S):
            qs, ks, vs = workloads.contig_step(seed, step, B, Hq, Hkv, D)
            assert pkv.cache_update(kc, bf16_dev(ks), lengths, 1) == kc.data_ptr()
            assert pkv.cache_update(vc, bf16_dev(vs), lengths, 1) == vc.data_ptr()
            pkv.decode_step(kf, vf, bf16_dev(ks), bf16_dev(vs), lengths, 1, bf16_dev(qs).reshape(B, Hq, 1, D), outf,
                            ws)
            ocache.cache_update(kh, ks, lengths, 1)
            ocache.cache_update(vh, vs, lengths, 1)
            lengths = lengths + 1
            pkv.decode_attention(bf16_dev(qs).reshape(B, Hq, 1, D), kc, vc, lengths, out, ws)
            assert torch.equal(out.view(torch.int16), outf.view(torch.int16)), step
            if step in (0, 17, S - 1):
                out32 = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=DEV)
                pkv.decode_attention(bf16_dev(qs).reshape(B, Hq, 1, D), kc, vc, lengths, out32, ws)
                assert np.array_equal(bits_host(out), _bf16_round(out32)), step
                torch.cuda.synchronize()
                got = out32.double().cpu().numpy()[:, :, 0]
                qd = onum.bf16_to_f64(qs)
                for b in range(B):
                    K = onum.bf16_to_f64(kh[b, :, :lengths[b]])
                    V = onum.bf16_to_f64(vh[b, :, :lengths[b]])
                    ref = np.stack([oattn.attend(qd[b, h], K[h // G], V[h // G], 1 / np.sqrt(D)) for h in range(Hq)])
                    assert rel_err_rows(got[b], ref) <= F32_TOL, (step, b)
    assert np.array_equal(bits_host(kc), kh) and np.array_equal(bits_host(vc), vh)   # every cache byte
    assert np.array_equal(bits_host(kf), kh) and np.array_equal(bits_host(vf), vh)


def test_int4_full_size():
    require_gpu()
    spec = workloads.int4()
    B, Hq, Hkv, D, bs, NB, maxb = spec.B, spec.Hq, spec.Hkv, spec.D, spec.bs, spec.NB, spec.maxb
    ref_pool = ocache.PagePool(NB, bs, B, maxb, spec.order)
    lib_pool = pkv.Pool(NB, bs, B, maxb, spec.order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), spec.lengths.tolist(), table)
    kc = np.zeros((NB, Hkv, bs, D // 2), np.uint8)
    vc = np.zeros_like(kc)
    kp = np.zeros((NB, Hkv, bs, D // 32, 2), np.uint16)
    vp = np.zeros_like(kp)
    check = [0, 4, 9, 13, 17, 22, 27, 31]
    logical = {}
    for b in range(B):
        ref_pool.reserve(b, int(spec.lengths[b]))
        L = int(spec.lengths[b])
        rows = (spec.codes_row(b), spec.params_row(b), spec.v_codes_row(b), spec.v_params_row(b))
        for dst, src in zip((kc, kp.reshape(NB, Hkv, bs, -1), vc, vp.reshape(NB, Hkv, bs, -1)),
                            (rows[0], rows[1].reshape(Hkv, L, -1), rows[2], rows[3].reshape(Hkv, L, -1))):
            ocache.paged_cache_update(dst, ref_pool.table[b:b + 1], src[None], [0], L, bs)
        if b in check:
            logical[b] = (oaffine.int4_dequant_rows(rows[0], rows[1]), oaffine.int4_dequant_rows(rows[2], rows[3]))
    assert np.array_equal(table.cpu().numpy(), ref_pool.table)
    dev16 = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.float16)
    q = spec.q_f32()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, int(spec.lengths.max())))
    pkv.paged_decode_attention_int4(torch.from_numpy(q).to(DEV), torch.from_numpy(kc).to(DEV), dev16(kp),
                                    torch.from_numpy(vc).to(DEV), dev16(vp), table, maxb, bs,
                                    spec.lengths.tolist(), out, ws, pool=lib_pool)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    G = Hq // Hkv
    for b in check:
        K, V = logical[b]
        ref = np.stack([oattn.attend(q[b, h].astype(np.float64), K[h // G], V[h // G], 1 / np.sqrt(D))
                        for h in range(Hq)])
        assert rel_err_rows(got[b], ref) <= 1e-3, b


def test_qwen_shaped_layer_decode_chunk_and_sampling():
    """One of the 28 layers at full size: decode append + attention, a 512-token chunk append +
    causal chunk attention (sampled queries), and greedy / T=0.7 sampling of [128, 151936] logits."""
    require_gpu()
    w = workloads.qwen()
    B, Hq, Hkv, D, bs, C, maxb = w["B"], w["Hq"], w["Hkv"], w["D"], w["bs"], w["chunk"], w["maxb"]
    L = w["lengths"].astype(np.int32)
    NB = w["NB"]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    kd, vd = _randn_bf16((NB, Hkv, bs, D), gen), _randn_bf16((NB, Hkv, bs, D), gen)
    lib_pool = pkv.Pool(NB, bs, B, maxb, w["order"])
    ref_pool = ocache.PagePool(NB, bs, B, maxb, w["order"])
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), (L + C).tolist(), table)
    for b in range(B):
        ref_pool.reserve(b, int(L[b]) + C)
    assert np.array_equal(table.cpu().numpy(), ref_pool.table)
    order_L = np.argsort(L, kind="stable")
    check = sorted({int(order_L[0]), int(order_L[-1])} | {int(order_L[i]) for i in (18, 37, 55, 73, 91, 110)})
    host = {}
    for b in check:
        ids = ref_pool.table[b, :-(-(int(L[b]) + C) // bs)]
        host[b] = (ids, _pages_host(kd, ids), _pages_host(vd, ids))
    # (i) chunk: append C tokens at p0 = L, causal attention of the C queries
    nk, nv = _randn_bf16((B, Hkv, C, D), gen), _randn_bf16((B, Hkv, C, D), gen)
    q = _randn_bf16((B, Hq, C, D), gen)
    nkh, nvh, qh = bits_host(nk), bits_host(nv), bits_host(q)
    with pkv.bind_writable(kd), pkv.bind_writable(vd):
        pkv.paged_cache_update(lib_pool, kd, table, nk, L.tolist(), C)
        pkv.paged_cache_update(lib_pool, vd, table, nv, L.tolist(), C)
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    pkv.chunk_attention(q, kd, vd, table, maxb, bs, L.tolist(), out, pool=lib_pool)
    got = onum.bf16_to_f64(bits_host(out))
    G = Hq // Hkv
    for b in check:
        ids, kp, vp = host[b]
        local = np.arange(len(ids), dtype=np.int32)[None]
        ocache.paged_cache_update(kp, local, nkh[b:b + 1], [int(L[b])], C, bs)
        ocache.paged_cache_update(vp, local, nvh[b:b + 1], [int(L[b])], C, bs)
        assert np.array_equal(_pages_host(kd, ids), kp) and np.array_equal(_pages_host(vd, ids), vp)
        K = onum.bf16_to_f64(ocache.paged_gather(kp, local[0], int(L[b]) + C, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(vp, local[0], int(L[b]) + C, bs))
        for t in (0, 1, 255, C - 1):
            last = int(L[b]) + t
            qt = onum.bf16_to_f64(qh[b, :, t])
            ref = np.stack([oattn.attend(qt[h], K[h // G, :last + 1], V[h // G, :last + 1], 1 / np.sqrt(D))
                            for h in range(Hq)])
            for h in range(Hq):
                s = K[h // G, :last + 1] @ qt[h] / np.sqrt(D)
                assert_bf16_pv_bound(got[b, h, t], ref[h], s, V[h // G, :last + 1])
    # (ii) decode over the full prefix + chunk (L + C tokens)
    dq = _randn_bf16((B, Hq, D), gen)
    dout = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, int((L + C).max())))
    pkv.paged_decode_attention(dq, kd, vd, table, maxb, bs, (L + C).tolist(), dout, ws, pool=lib_pool)
    dout32 = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    pkv.paged_decode_attention(dq, kd, vd, table, maxb, bs, (L + C).tolist(), dout32, ws, pool=lib_pool)
    assert np.array_equal(bits_host(dout), _bf16_round(dout32))
    torch.cuda.synchronize()
    dgot = dout32.double().cpu().numpy()
    dqh = onum.bf16_to_f64(bits_host(dq))
    for b in check:
        ids, kp, vp = host[b]
        local = np.arange(len(ids), dtype=np.int32)
        K = onum.bf16_to_f64(ocache.paged_gather(kp, local, int(L[b]) + C, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(vp, local, int(L[b]) + C, bs))
        ref = np.stack([oattn.attend(dqh[b, h], K[h // G], V[h // G], 1 / np.sqrt(D)) for h in range(Hq)])
        assert rel_err_rows(dgot[b], ref) <= F32_TOL, b
    # (iii) sampling of [128, 151936] logits ~ N(0, 3)
    logits = workloads.logits(w["seed"], B, w["vocab"])
    ld = torch.from_numpy(logits).to(DEV)
    ids = torch.empty((B,), dtype=torch.int64, device=DEV)
    sws = workspace(pkv.sample_workspace_size(B, w["vocab"]))
    pkv.sample(ld, 0.0, 5, ids, sws)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), osamp.greedy(logits))
    pkv.sample(ld, 0.7, 5, ids, sws)
    torch.cuda.synchronize()
    got_ids = ids.cpu().numpy()
    want = osamp.sample(logits, 0.7, 5)
    for b in np.nonzero(got_ids != want)[0]:
        sc = osamp.gumbel_scores(logits[b], 0.7, 5, b)
        assert abs(sc[got_ids[b]] - sc[want[b]]) <= 1e-5 * max(1.0, abs(sc[want[b]]))
    assert (got_ids == want).mean() >= 0.99


def test_mixed32k_full_size():
    """The mixed-format bench row: 32 x 32768 tokens in a full pool, BF16 prefix pages then INT8 K / UINT4 V
    pages chosen by the length-threshold selector, appended in the bench's chunks; sampled rows' pages
    bit for bit and their attention against the oracle."""
    require_gpu()
    from oracle import mixed as om
    w = workloads.mixed32k()
    rows = [0, 31]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(w.seed)
    kp = torch.zeros((w.NB, w.Hkv, w.bs, w.D), device=DEV, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    pd = pkv.mixed_page_desc(w.NB, DEV)
    pool = pkv.Pool(w.NB, w.bs, w.B, w.maxb, w.order)
    ref_pool = ocache.PagePool(w.NB, w.bs, w.B, w.maxb, w.order)
    table = torch.full((w.B, w.maxb), -1, device=DEV, dtype=torch.int32)
    pool.reserve(range(w.B), [w.L] * w.B, table)
    for b in range(w.B):
        ref_pool.reserve(b, w.L)
    assert np.array_equal(table.cpu().numpy(), ref_pool.table)
    fm = lambda t: pkv.page_format(*t)
    select = pkv.LengthThresholdSelector(w.threshold, (fm(w.early[0]), fm(w.early[1])), (fm(w.late[0]), fm(w.late[1])))
    refs = {b: om.MixedPool(w.maxb, w.Hkv, w.bs, w.D) for b in rows}
    local = np.arange(w.maxb, dtype=np.int32)[None]
    with pkv.bind_writable(kp), pkv.bind_writable(vp), pkv.bind_writable(pd):
        pos = 0
        while pos < w.L:
            n = w.threshold if pos < w.threshold else min(2048, w.L - pos)
            kv = (torch.randn((w.B, w.Hkv, n, w.D), generator=gen, device=DEV) * w.k_sigma).to(torch.bfloat16)
            vv = (torch.randn((w.B, w.Hkv, n, w.D), generator=gen, device=DEV) * w.v_sigma).to(torch.bfloat16)
            kb, vb = bits_host(kv), bits_host(vv)
            kf, vf = select(pos)
            pkv.mixed_cache_update(pool, kp, vp, pd, table, kv, vv, [pos] * w.B, n, kf, vf)
            okf, ovf = (w.early if pos < w.threshold else w.late)
            for b in rows:
                refs[b].append(local, kb[b:b + 1], vb[b:b + 1], [pos], n, om.Format(*okf), om.Format(*ovf))
            pos += n
    q = torch.randn((w.B, w.Hq, w.D), generator=gen, device=DEV).to(torch.bfloat16)
    qh = onum.bf16_to_f64(bits_host(q))
    out = torch.empty((w.B, w.Hq, w.D), device=DEV, dtype=torch.bfloat16)
    ws = workspace(pkv.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.L))
    pkv.paged_decode_attention_mixed(q, kp, vp, pd, table, w.maxb, w.bs, [w.L] * w.B, out, ws, pool=pool)
    out32 = torch.empty((w.B, w.Hq, w.D), device=DEV, dtype=torch.float32)
    pkv.paged_decode_attention_mixed(q, kp, vp, pd, table, w.maxb, w.bs, [w.L] * w.B, out32, ws, pool=pool)
    assert np.array_equal(bits_host(out), _bf16_round(out32))
    torch.cuda.synchronize()
    got = out32.double().cpu().numpy()
    for b in rows:
        ids = torch.from_numpy(ref_pool.table[b].astype(np.int64)).to(DEV)
        for name, t in (("k", kp), ("v", vp)):
            gb = bytes_host(t.index_select(0, ids).contiguous()).reshape(w.maxb, w.Hkv, -1)
            assert np.array_equal(gb, refs[b].data[name]), (b, name)
        ref = om.decode_attention(refs[b], qh[b:b + 1], local, [w.L])
        assert rel_err_rows(got[b], ref[0]) <= F32_TOL, b


def test_one_request_chunk_with_the_library_split():
    """One row of the Qwen shape at full size (16384-token prefix, 512-token chunk): the library's split over the
    keys (chosen from the launch size: one workgroup per K/V head and 128-token query tile, 32 in all) and its
    merge.  Queries at both ends and at the query-tile edges against the oracle over all 16896 keys."""
    require_gpu()
    w = workloads.qwen(B=1, lo=16384, hi=16384)
    B, Hq, Hkv, D, bs, C, maxb = w["B"], w["Hq"], w["Hkv"], w["D"], w["bs"], w["chunk"], w["maxb"]
    L = w["lengths"].astype(np.int32)
    NB = w["NB"]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(6)
    kd, vd = _randn_bf16((NB, Hkv, bs, D), gen), _randn_bf16((NB, Hkv, bs, D), gen)
    lib_pool = pkv.Pool(NB, bs, B, maxb, w["order"])
    ref_pool = ocache.PagePool(NB, bs, B, maxb, w["order"])
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), (L + C).tolist(), table)
    ref_pool.reserve(0, int(L[0]) + C)
    nk, nv = _randn_bf16((B, Hkv, C, D), gen), _randn_bf16((B, Hkv, C, D), gen)
    q = _randn_bf16((B, Hq, C, D), gen)
    with pkv.bind_writable(kd), pkv.bind_writable(vd):
        pkv.paged_cache_update_kv(lib_pool, kd, vd, table, nk, nv, L.tolist(), C)
    need = pkv.chunk_workspace_size(B, Hq, Hkv, C, 0)
    assert need > 0
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    pkv.chunk_attention(q, kd, vd, table, maxb, bs, L.tolist(), out, pool=lib_pool, workspace=workspace(need),
                        num_splits=0)
    got = onum.bf16_to_f64(bits_host(out))
    qh = bits_host(q)
    ids = ref_pool.table[0, :-(-(int(L[0]) + C) // bs)]
    local = np.arange(len(ids), dtype=np.int32)
    K = onum.bf16_to_f64(ocache.paged_gather(_pages_host(kd, ids), local, int(L[0]) + C, bs))
    V = onum.bf16_to_f64(ocache.paged_gather(_pages_host(vd, ids), local, int(L[0]) + C, bs))
    G = Hq // Hkv
    for t in (0, 1, 127, 128, 255, 256, 384, C - 1):
        last = int(L[0]) + t
        qt = onum.bf16_to_f64(qh[0, :, t])
        for h in range(Hq):
            ref = oattn.attend(qt[h], K[h // G, :last + 1], V[h // G, :last + 1], 1 / np.sqrt(D))
            s = K[h // G, :last + 1] @ qt[h] / np.sqrt(D)
            assert_bf16_pv_bound(got[0, h, t], ref, s, V[h // G, :last + 1])
