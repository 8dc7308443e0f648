"""Batches larger than the 256 rows one launch takes: the host splits them into launches whose row,
page-table, query and output offsets must line up.  Every row of a 300-row batch is checked against
the oracle for the paired paged append, paged decode (with and without splits), contiguous decode
(fast and generic kernels), INT4 decode and chunk attention (with and without a split over the keys)."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import affine as oaffine
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import numeric as onum
from tests.gpu_util import DEV, bf16_dev, bits_host, rel_err_rows, require_gpu, workspace
from tests.test_gpu_chunk import _assert_chunk_bound, _setup
from tests.test_gpu_decode import TOL, _contig_inputs, _out_f64, _paged_inputs, _paged_ref

pytestmark = pytest.mark.gpu

B = 300


def test_decode_and_paired_append_over_300_rows():
    require_gpu()
    Hkv, G, D, bs, maxb = 2, 2, 128, 16, 5
    Hq = Hkv * G
    lengths = synth.rng(1300).integers(1, maxb * bs - 1, size=B).astype(np.int32)
    d = _paged_inputs(1301, B, Hq, Hkv, D, bs, lengths, maxb, extra_blocks=B)
    ref = _paged_ref(d, lengths)
    for S in [0, 3]:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, S))
        pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out, ws,
                                   pool=d["pool"], num_splits=S)
        assert rel_err_rows(_out_f64(out), ref) <= TOL["f32"], S
    # one more token per row through the paired append: every byte of both pools
    new_len = (lengths + 1).tolist()
    d["pool"].reserve(range(B), new_len, d["table"])
    for b in range(B):
        d["ref_pool"].reserve(b, new_len[b])
    g = synth.rng(1302)
    kv = synth.f32_to_bf16_bits(synth.normal(g, (B, Hkv, 1, D)))
    vv = synth.f32_to_bf16_bits(synth.normal(g, (B, Hkv, 1, D)))
    with pkv.bind_writable(d["kp"]), pkv.bind_writable(d["vp"]):
        pkv.paged_cache_update_kv(d["pool"], d["kp"], d["vp"], d["table"], bf16_dev(kv), bf16_dev(vv), lengths, 1)
    ocache.paged_cache_update(d["kp_host"], d["ref_pool"].table, kv, lengths, 1, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp_host"], d["ref_pool"].table, vv, lengths, 1, bs, d["ref_pool"].held)
    assert np.array_equal(bits_host(d["kp"]), d["kp_host"]) and np.array_equal(bits_host(d["vp"]), d["vp_host"])


@pytest.mark.parametrize("S", [1, 2])         # without and with a split over the keys
def test_chunk_attention_over_300_rows(S):
    require_gpu()
    Hkv, G, D, bs, C = 2, 2, 128, 16, 3
    Hq = Hkv * G
    p0 = synth.rng(1310).integers(0, 70, size=B).astype(np.int32)
    maxb = -(-(int(p0.max()) + C) // bs) + 1
    d = _setup(1311, B, Hq, Hkv, D, bs, p0, C, maxb)
    with pkv.bind_writable(d["kd"]), pkv.bind_writable(d["vd"]):
        pkv.paged_cache_update_kv(d["lib_pool"], d["kd"], d["vd"], d["table"], bf16_dev(d["new_k"]),
                                  bf16_dev(d["new_v"]), p0, C)
    ocache.paged_cache_update(d["kp"], d["ref_pool"].table, d["new_k"], p0, C, bs, d["ref_pool"].held)
    ocache.paged_cache_update(d["vp"], d["ref_pool"].table, d["new_v"], p0, C, bs, d["ref_pool"].held)
    assert np.array_equal(bits_host(d["kd"]), d["kp"]) and np.array_equal(bits_host(d["vd"]), d["vp"])
    out = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device=DEV)
    ws = None if S == 1 else workspace(pkv.chunk_workspace_size(B, Hq, Hkv, C, S))
    pkv.chunk_attention(bf16_dev(d["q"]), d["kd"], d["vd"], d["table"], maxb, bs, p0, out, pool=d["lib_pool"],
                        workspace=ws, num_splits=S)
    got = onum.bf16_to_f64(bits_host(out))
    qh = onum.bf16_to_f64(d["q"])
    for b in range(B):
        L = int(p0[b]) + C
        K = onum.bf16_to_f64(ocache.paged_gather(d["kp"], d["ref_pool"].table[b], L, bs))
        V = onum.bf16_to_f64(ocache.paged_gather(d["vp"], d["ref_pool"].table[b], L, bs))
        ref = oattn.chunk_attention(qh[b], K, V, int(p0[b]))
        _assert_chunk_bound(got[b], ref, qh[b], K, V, int(p0[b]))


@pytest.mark.parametrize("D", [128, 8])       # the fast kernel and the generic one
def test_contiguous_decode_over_300_rows(D):
    require_gpu()
    Hkv, G, cap = 2, 2, 40
    Hq = Hkv * G
    lengths = synth.rng(1320, D).integers(1, cap + 1, size=B).astype(np.int32)
    q, kc, vc, qh, kh, vh = _contig_inputs(1321 + D, B, Hq, Hkv, D, cap, lengths)
    ref = oattn.decode_attention(qh, kh, vh, lengths)
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, 2))
    pkv.decode_attention(q.reshape(B, Hq, 1, D), kc, vc, lengths, out, ws, num_splits=2)
    assert rel_err_rows(_out_f64(out), ref) <= TOL["f32"]


def test_int4_decode_over_300_rows():
    require_gpu()
    Hkv, G, D, bs, maxb = 2, 4, 128, 16, 3
    Hq = Hkv * G
    lengths = synth.rng(1330).integers(1, maxb * bs + 1, size=B).astype(np.int32)
    NB = int(sum(-(-int(L) // bs) for L in lengths))
    order = synth.permutation(synth.rng(1331), NB)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    lib_pool = pkv.Pool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), lengths.tolist(), table)
    kc = np.zeros((NB, Hkv, bs, D // 2), np.uint8)
    vc = np.zeros_like(kc)
    kp = np.zeros((NB, Hkv, bs, D // 32, 2), np.uint16)
    vp = np.zeros_like(kp)
    k_log, v_log = [], []
    for b in range(B):
        L = int(lengths[b])
        ref_pool.reserve(b, L)
        g = synth.rng(1332, b)
        codes = [g.integers(0, 256, size=(1, Hkv, L, D // 2), dtype=np.uint8) for _ in range(2)]
        params = []
        for _ in range(2):
            prm = np.empty((1, Hkv, L, D // 32, 2), np.uint16)
            prm[..., 0] = synth.f16_bits(synth.uniform(g, (1, Hkv, L, D // 32), 0.01, 0.1))
            prm[..., 1] = synth.f16_bits(g.integers(0, 16, size=(1, Hkv, L, D // 32)).astype(np.float32))
            params.append(prm)
        for pool_arr, rows in ((kc, codes[0]), (vc, codes[1])):
            ocache.paged_cache_update(pool_arr, ref_pool.table[b:b + 1], rows, [0], L, bs)
        for pool_arr, rows in ((kp, params[0]), (vp, params[1])):
            ocache.paged_cache_update(pool_arr.reshape(NB, Hkv, bs, -1), ref_pool.table[b:b + 1],
                                      rows.reshape(1, Hkv, L, -1), [0], L, bs)
        k_log.append(oaffine.int4_dequant_rows(codes[0][0], params[0][0]))
        v_log.append(oaffine.int4_dequant_rows(codes[1][0], params[1][0]))
    q = synth.normal(synth.rng(1333), (B, Hq, D))
    ref = np.stack([np.stack([oattn.attend(q[b, h].astype(np.float64), k_log[b][h // G], v_log[b][h // G],
                                           1 / np.sqrt(D)) for h in range(Hq)]) for b in range(B)])
    f16 = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.float16)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, 2))
    pkv.paged_decode_attention_int4(torch.from_numpy(q).to(DEV), torch.from_numpy(kc).to(DEV), f16(kp),
                                    torch.from_numpy(vc).to(DEV), f16(vp), table, maxb, bs, lengths, out, ws,
                                    pool=lib_pool, num_splits=2)
    assert rel_err_rows(_out_f64(out), ref) <= TOL["int4"]
