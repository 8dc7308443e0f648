"""GPU parity of decode attention (contiguous, paged bf16, generic paths, INT4)
against the float64 oracle, the tiny stateful == stateless fixture, and the
invariances the method implies (split count, page order, layout)."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import affine as oaffine
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import numeric as onum
from oracle import stateless as ostate
from synth import workloads
from tests.gpu_util import DEV, bf16_dev, bits_host, bytes_host, rel_err_rows, require_gpu, sentinel_dev, workspace

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "int4": 1e-3}
# The decode kernels accumulate in float32 from exactly representable inputs,
# so f32 outputs meet the float32 bar; a 16-bit output adds one rounding to
# nearest, at most the unit roundoff times the element (2^-8 for bf16's 8
# significant bits, 2^-11 for f16's 11), which bounds the normwise error by
# that fraction of the row's largest element.  Tests with a bf16 output also
# check it bit for bit against the float32 output rounded once.
BF16_OUT = 2.0 ** -8 + 2e-5
F16_OUT = 2.0 ** -11 + 2e-5


def _out_f64(out: torch.Tensor) -> np.ndarray:
    if out.dtype == torch.bfloat16:
        return onum.bf16_to_f64(bits_host(out))
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def test_tiny_fixture_stateful_equals_stateless():
    """1-token prompt + 15 appends into capacity 16, attention after each, then the overflow step."""
    require_gpu()
    w = workloads.tiny()
    q, k, v = w["q"], w["k"], w["v"]
    cap = w["capacity"]
    ref = ostate.stateless_decode(q[:cap].astype(np.float64), k[:cap].astype(np.float64), v[:cap].astype(np.float64))
    kc = sentinel_dev((1, 1, cap, 4), torch.float32)         # 0xA5 bytes: untouched rows stay visible
    vc = sentinel_dev((1, 1, cap, 4), torch.float32)
    ws = workspace(pkv.decode_workspace_size(1, 1, 1, 4, cap))
    out = torch.empty((1, 1, 1, 4), device=DEV)
    with pkv.bind_writable(kc), pkv.bind_writable(vc):
        for t in range(cap):
            kt = torch.from_numpy(k[t]).reshape(1, 1, 1, 4).to(DEV)
            vt = torch.from_numpy(v[t]).reshape(1, 1, 1, 4).to(DEV)
            assert pkv.cache_update(kc, kt, [t], 1) == kc.data_ptr()
            assert pkv.cache_update(vc, vt, [t], 1) == vc.data_ptr()
            pkv.decode_attention(torch.from_numpy(q[t]).reshape(1, 1, 1, 4).to(DEV), kc, vc, [t + 1], out, ws)
            assert rel_err_rows(_out_f64(out), ref[t][None]) <= TOL["f32"], t
            # retained logical bytes grow by exactly one 16-byte row per tensor per step: rows 0..t hold
            # the appended values, every byte of rows t+1.. still holds the sentinel
            for dev_t, host_rows in ((kc, k), (vc, v)):
                got = bytes_host(dev_t).reshape(cap, 16)
                changed = (got != 0xA5).any(axis=1)
                assert int(changed.sum()) * 16 == 16 * (t + 1) and changed[:t + 1].all(), t
                assert np.array_equal(got[:t + 1], host_rows[:t + 1].astype(np.float32).view(np.uint8).reshape(-1, 16))
        before = (kc.clone(), vc.clone())
        with pytest.raises(pkv.PkvError) as e:
            pkv.cache_update(kc, torch.from_numpy(k[cap]).reshape(1, 1, 1, 4).to(DEV), [cap], 1)
        assert e.value.status == pkv.E_CAPACITY
        assert torch.equal(kc, before[0]) and torch.equal(vc, before[1])


def _contig_inputs(seed, B, Hq, Hkv, D, cap, lengths, kind="bf16"):
    g = synth.rng(seed)
    if kind == "bf16":
        kb = synth.f32_to_bf16_bits(synth.normal(g, (B, Hkv, cap, D)))
        vb = synth.f32_to_bf16_bits(synth.normal(g, (B, Hkv, cap, D)))
        qb = synth.f32_to_bf16_bits(synth.normal(g, (B, Hq, D)))
        return (bf16_dev(qb), bf16_dev(kb), bf16_dev(vb),
                onum.bf16_to_f64(qb), onum.bf16_to_f64(kb), onum.bf16_to_f64(vb))
    tdt = {"f32": torch.float32, "f16": torch.float16}[kind]
    kf, vf, qf = (synth.normal(g, s) for s in [(B, Hkv, cap, D), (B, Hkv, cap, D), (B, Hq, D)])
    if kind == "f16":
        kf, vf, qf = (x.astype(np.float16).astype(np.float32) for x in (kf, vf, qf))
    dev = [torch.from_numpy(x).to(DEV).to(tdt) for x in (qf, kf, vf)]
    return (*dev, qf.astype(np.float64), kf.astype(np.float64), vf.astype(np.float64))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_contiguous_bf16_matches_oracle(G):
    require_gpu()
    B, Hkv, D, cap = 4, 2, 128, 700
    Hq = Hkv * G
    lengths = np.array([1, 17, 333, 700], np.int32)
    q, kc, vc, qh, kh, vh = _contig_inputs(700 + G, B, Hq, Hkv, D, cap, lengths)
    ref = oattn.decode_attention(qh, kh, vh, lengths)
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap))
    pkv.decode_attention(q.reshape(B, Hq, 1, D), kc, vc, lengths, out, ws)
    assert rel_err_rows(_out_f64(out), ref) <= BF16_OUT
    out32 = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=DEV)
    pkv.decode_attention(q.reshape(B, Hq, 1, D), kc, vc, lengths, out32, ws)
    assert rel_err_rows(_out_f64(out32), ref) <= TOL["f32"]           # no bf16 output rounding
    # the bf16 output is the float32 result rounded once (same reduction order)
    assert np.array_equal(bits_host(out), bits_host(out32.to(torch.bfloat16)))


def test_split_count_does_not_change_the_result():
    require_gpu()
    B, Hq, Hkv, D, cap = 3, 8, 2, 128, 2000
    lengths = np.array([2000, 1003, 64], np.int32)
    q, kc, vc, qh, kh, vh = _contig_inputs(710, B, Hq, Hkv, D, cap, lengths)
    ref = oattn.decode_attention(qh, kh, vh, lengths)
    outs = []
    for S in [1, 2, 7, 16, 64, 0]:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, S))
        pkv.decode_attention(q, kc, vc, lengths, out, ws, num_splits=S)
        got = _out_f64(out)
        assert rel_err_rows(got, ref) <= TOL["f32"], S
        outs.append(got)
    for got in outs[1:]:
        assert rel_err_rows(got, outs[0]) <= 1e-5


def _encode(x32, kind):
    """float32 draws -> (storage array, exact float64 values) for the given element type."""
    if kind == "bf16":
        bits = synth.f32_to_bf16_bits(x32)
        return bits, onum.bf16_to_f64(bits)
    if kind == "f16":
        bits = synth.f16_bits(x32)
        return bits, onum.f16_to_f64(bits)
    return x32, x32.astype(np.float64)


def _to_dev(arr, kind):
    if kind == "bf16":
        return bf16_dev(arr)
    if kind == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.float16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _paged_inputs(seed, B, Hq, Hkv, D, bs, lengths, maxb, extra_blocks=3, order=None, kind="bf16"):
    """Logical rows on the host, laid out through the oracle pool; the library pool writes the device table."""
    g = synth.rng(seed)
    NB = int(sum(-(-int(L) // bs) for L in lengths)) + extra_blocks
    order = synth.permutation(g, NB) if order is None else order
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    lib_pool = pkv.Pool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), lengths.tolist(), table)
    k_log, v_log = [], []
    store = np.float32 if kind == "f32" else np.uint16
    kp = np.zeros((NB, Hkv, bs, D), store)
    vp = np.zeros((NB, Hkv, bs, D), store)
    for b in range(B):
        ref_pool.reserve(b, int(lengths[b]))
        kr, kf = _encode(synth.normal(synth.rng(seed, 1, b), (1, Hkv, int(lengths[b]), D)), kind)
        vr, vf = _encode(synth.normal(synth.rng(seed, 2, b), (1, Hkv, int(lengths[b]), D)), kind)
        ocache.paged_cache_update(kp, ref_pool.table[b:b + 1], kr, [0], int(lengths[b]), bs)
        ocache.paged_cache_update(vp, ref_pool.table[b:b + 1], vr, [0], int(lengths[b]), bs)
        k_log.append(kf[0])
        v_log.append(vf[0])
    assert np.array_equal(table.cpu().numpy(), ref_pool.table)
    qs, qh = _encode(synth.normal(synth.rng(seed, 3), (B, Hq, D)), kind)
    return dict(q=_to_dev(qs, kind), qh=qh, kp=_to_dev(kp, kind), vp=_to_dev(vp, kind), table=table,
                pool=lib_pool, ref_pool=ref_pool, k_log=k_log, v_log=v_log, NB=NB, order=order,
                kp_host=kp, vp_host=vp)


def _paged_ref(d, lengths, left_window=-1):
    out = []
    for b, L in enumerate(lengths):
        Hq = d["qh"].shape[1]
        G = Hq // d["k_log"][b].shape[0]
        lo = oattn.visible_begin(int(L) - 1, left_window)
        out.append(np.stack([oattn.attend(d["qh"][b, h], d["k_log"][b][h // G][lo:], d["v_log"][b][h // G][lo:],
                                          1 / np.sqrt(d["qh"].shape[2])) for h in range(Hq)]))
    return np.stack(out)


@pytest.mark.parametrize("G,bs", [(4, 16), (2, 16), (1, 32), (8, 64)])
def test_paged_bf16_matches_oracle(G, bs):
    require_gpu()
    B, Hkv, D, maxb = 6, 2, 128, 40
    Hq = Hkv * G
    lengths = np.array([1, 15, 16, 17, 300, 40 * bs - 3], np.int32)
    d = _paged_inputs(720 + G, B, Hq, Hkv, D, bs, lengths, maxb)
    ref = _paged_ref(d, lengths)
    for S in [0, 1, 5]:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, S))
        pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out, ws,
                                   pool=d["pool"], num_splits=S)
        assert rel_err_rows(_out_f64(out), ref) <= BF16_OUT, S
        out32 = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out32, ws,
                                   pool=d["pool"], num_splits=S)
        assert rel_err_rows(_out_f64(out32), ref) <= TOL["f32"], S


def test_page_order_and_layout_do_not_change_the_bits():
    """Two page permutations of the same logical rows, and the contiguous layout, give identical outputs."""
    require_gpu()
    B, Hq, Hkv, D, bs, maxb = 4, 16, 4, 128, 16, 20
    lengths = np.array([5, 160, 233, 320], np.int32)
    d1 = _paged_inputs(730, B, Hq, Hkv, D, bs, lengths, maxb)
    d2 = _paged_inputs(730, B, Hq, Hkv, D, bs, lengths, maxb, order=d1["order"][::-1].copy())
    assert not np.array_equal(d1["ref_pool"].table, d2["ref_pool"].table)
    cap = maxb * bs
    kc = np.zeros((B, Hkv, cap, D), np.uint16)
    vc = np.zeros((B, Hkv, cap, D), np.uint16)
    for b in range(B):
        L = int(lengths[b])
        kc[b, :, :L] = ocache.paged_gather(d1["kp_host"], d1["ref_pool"].table[b], L, bs)
        vc[b, :, :L] = ocache.paged_gather(d1["vp_host"], d1["ref_pool"].table[b], L, bs)
    outs = []
    for S in [0, 3]:
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, S))
        res = []
        for d in (d1, d2):
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
            pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out, ws,
                                       pool=d["pool"], num_splits=S)
            res.append(_out_f64(out))
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        pkv.decode_attention(d1["q"], bf16_dev(kc), bf16_dev(vc), lengths, out, ws, num_splits=S)
        res.append(_out_f64(out))
        assert np.array_equal(res[0], res[1]) and np.array_equal(res[0], res[2]), S
        outs.append(res[0])
    assert rel_err_rows(outs[0], _paged_ref(d1, lengths)) <= TOL["f32"]


@pytest.mark.parametrize("kind,D,bs,G", [("bf16", 64, 16, 4), ("bf16", 128, 8, 4), ("f32", 32, 16, 2),
                                         ("f16", 128, 16, 4), ("bf16", 128, 16, 3), ("f32", 256, 4, 1)])
def test_generic_paths_match_oracle(kind, D, bs, G):
    require_gpu()
    B, Hkv, maxb = 3, 2, 80
    Hq = Hkv * G
    cap = 250
    lengths = np.array([1, 129, 250], np.int32)
    tol = {"f32": TOL["f32"], "bf16": BF16_OUT, "f16": F16_OUT}[kind]
    q, kc, vc, qh, kh, vh = _contig_inputs(740 + D + bs, B, Hq, Hkv, D, cap, lengths, kind)
    ref = oattn.decode_attention(qh, kh, vh, lengths)
    out = torch.empty((B, Hq, D), dtype=q.dtype, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap))
    pkv.decode_attention(q, kc, vc, lengths, out, ws)
    torch.cuda.synchronize()
    assert rel_err_rows(out.double().cpu().numpy(), ref) <= tol
    d = _paged_inputs(741 + D + bs, B, Hq, Hkv, D, bs, lengths, maxb, kind=kind)
    out = torch.empty((B, Hq, D), dtype=q.dtype, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs))
    pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out, ws, pool=d["pool"])
    torch.cuda.synchronize()
    assert rel_err_rows(out.double().cpu().numpy(), _paged_ref(d, lengths)) <= tol


@pytest.mark.parametrize("kind,Dk,Dv,bs", [("bf16", 64, 128, 16), ("f32", 128, 48, 8), ("f16", 32, 256, 16)])
def test_value_head_size_of_its_own(kind, Dk, Dv, bs):
    """K and V head sizes differ (generic kernel), contiguous and paged, with and without splits."""
    require_gpu()
    B, Hq, Hkv, cap, maxb = 3, 8, 2, 300, 40
    lengths = np.array([1, 150, 300], np.int32)
    g = synth.rng(790 + Dk + Dv)
    qf, kf, vf = (synth.normal(g, sh) for sh in [(B, Hq, Dk), (B, Hkv, cap, Dk), (B, Hkv, cap, Dv)])
    (qs, qh), (ks, kh), (vs, vh) = (_encode(x, kind) for x in (qf, kf, vf))
    ref = oattn.decode_attention(qh, kh, vh, lengths)
    tol = {"f32": TOL["f32"], "bf16": BF16_OUT, "f16": F16_OUT}[kind]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[kind]
    for S in (0, 3):
        out = torch.empty((B, Hq, Dv), dtype=tdt, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, Dv, cap, S))
        pkv.decode_attention(_to_dev(qs, kind), _to_dev(ks, kind), _to_dev(vs, kind), lengths, out, ws, num_splits=S)
        torch.cuda.synchronize()
        assert rel_err_rows(out.double().cpu().numpy(), ref) <= tol, S
    # paged: the pools take each row's logical K / V through the oracle's page layout
    NB = int(sum(-(-int(L) // bs) for L in lengths)) + 2
    order = synth.permutation(g, NB)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    lib_pool = pkv.Pool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), lengths.tolist(), table)
    kp = np.zeros((NB, Hkv, bs, Dk), ks.dtype)
    vp = np.zeros((NB, Hkv, bs, Dv), vs.dtype)
    for b in range(B):
        L = int(lengths[b])
        ref_pool.reserve(b, L)
        ocache.paged_cache_update(kp, ref_pool.table[b:b + 1], ks[b:b + 1, :, :L], [0], L, bs)
        ocache.paged_cache_update(vp, ref_pool.table[b:b + 1], vs[b:b + 1, :, :L], [0], L, bs)
    out = torch.empty((B, Hq, Dv), dtype=tdt, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, Dv, maxb * bs))
    pkv.paged_decode_attention(_to_dev(qs, kind), _to_dev(kp, kind), _to_dev(vp, kind), table, maxb, bs, lengths,
                               out, ws, pool=lib_pool, left_window=120)
    torch.cuda.synchronize()
    ref_w = oattn.decode_attention(qh, kh, vh, lengths, left_window=120)
    assert rel_err_rows(out.double().cpu().numpy(), ref_w) <= tol


@pytest.mark.parametrize("G,bs", [(2, 16), (8, 32)])
def test_f16_fast_paged_matches_oracle(G, bs):
    require_gpu()
    B, Hkv, D, maxb = 4, 2, 128, 30
    Hq = Hkv * G
    lengths = np.array([1, 17, 300, 30 * bs - 5], np.int32)
    d = _paged_inputs(795 + G, B, Hq, Hkv, D, bs, lengths, maxb, kind="f16")
    ref = _paged_ref(d, lengths)
    for S in (0, 4):
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, S))
        pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out, ws,
                                   pool=d["pool"], num_splits=S)
        torch.cuda.synchronize()
        assert rel_err_rows(out.double().cpu().numpy(), ref) <= F16_OUT, S


@pytest.mark.parametrize("W", [0, 1, 63, 64, 65, 200, 5000])
def test_left_window_matches_oracle(W):
    """Left window W: the query at L - 1 sees keys [L - 1 - W, L - 1] (fast contiguous and paged paths,
    the generic path, auto and forced splits)."""
    require_gpu()
    B, Hkv, D, cap = 4, 2, 128, 700
    lengths = np.array([1, 70, 333, 700], np.int32)
    for G in (4, 2):
        Hq = Hkv * G
        q, kc, vc, qh, kh, vh = _contig_inputs(760 + W + G, B, Hq, Hkv, D, cap, lengths)
        ref = oattn.decode_attention(qh, kh, vh, lengths, left_window=W)
        for S in (0, 3):
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
            ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, S))
            pkv.decode_attention(q, kc, vc, lengths, out, ws, num_splits=S, left_window=W)
            assert rel_err_rows(_out_f64(out), ref) <= TOL["f32"], (G, S)
        d = _paged_inputs(770 + W + G, B, Hq, Hkv, D, 16, lengths, 48)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, 48 * 16))
        pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["table"], 48, 16, lengths, out, ws, pool=d["pool"],
                                   left_window=W)
        assert rel_err_rows(_out_f64(out), _paged_ref(d, lengths, W)) <= BF16_OUT, G
    # generic path: f32, D = 32, block size 8
    q, kc, vc, qh, kh, vh = _contig_inputs(780 + W, B, 4, 2, 32, cap, lengths, "f32")
    out = torch.empty((B, 4, 32), dtype=torch.float32, device=DEV)
    ws = workspace(pkv.decode_workspace_size(B, 4, 2, 32, cap))
    pkv.decode_attention(q, kc, vc, lengths, out, ws, left_window=W)
    assert rel_err_rows(_out_f64(out), oattn.decode_attention(qh, kh, vh, lengths, left_window=W)) <= TOL["f32"]


@pytest.mark.parametrize("G,bs", [(1, 16), (2, 32), (4, 16), (8, 16), (4, 64)])
def test_int4_paged_decode_matches_oracle(G, bs):
    require_gpu()
    Hkv, D = 2, 128
    B, Hq, maxb = 4, Hkv * G, -(-480 // bs) + 2
    lengths = np.array([1, 16, 250, 480], np.int32)
    g = synth.rng(750)
    NB = int(sum(-(-int(L) // bs) for L in lengths)) + 2
    order = synth.permutation(g, NB)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    lib_pool = pkv.Pool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    lib_pool.reserve(range(B), lengths.tolist(), table)
    # slots no row is written to hold arbitrary codes and NaN parameters: the
    # tail of a sequence's last page must not reach the output
    kc = synth.rng(750, 9).integers(0, 256, size=(NB, Hkv, bs, D // 2), dtype=np.uint8)
    vc = synth.rng(750, 10).integers(0, 256, size=(NB, Hkv, bs, D // 2), dtype=np.uint8)
    kp = np.full((NB, Hkv, bs, D // 32, 2), 0x7E00, np.uint16)
    vp = np.full_like(kp, 0x7E00)
    k_log, v_log = [], []
    for b in range(B):
        L = int(lengths[b])
        ref_pool.reserve(b, L)
        rows = {}
        for name, st in (("kc", 1), ("vc", 2)):
            rows[name] = synth.rng(750, st, b).integers(0, 256, size=(1, Hkv, L, D // 2), dtype=np.uint8)
        for name, st in (("kp", 3), ("vp", 4)):
            gg = synth.rng(750, st, b)
            p = np.empty((1, Hkv, L, D // 32, 2), np.uint16)
            p[..., 0] = synth.f16_bits(synth.uniform(gg, (1, Hkv, L, D // 32), 0.01, 0.1))
            p[..., 1] = synth.f16_bits(gg.integers(0, 16, size=(1, Hkv, L, D // 32)).astype(np.float32))
            rows[name] = p
        ocache.paged_cache_update(kc, ref_pool.table[b:b + 1], rows["kc"], [0], L, bs)
        ocache.paged_cache_update(vc, ref_pool.table[b:b + 1], rows["vc"], [0], L, bs)
        ocache.paged_cache_update(kp.reshape(NB, Hkv, bs, -1), ref_pool.table[b:b + 1],
                                  rows["kp"].reshape(1, Hkv, L, -1), [0], L, bs)
        ocache.paged_cache_update(vp.reshape(NB, Hkv, bs, -1), ref_pool.table[b:b + 1],
                                  rows["vp"].reshape(1, Hkv, L, -1), [0], L, bs)
        k_log.append(oaffine.int4_dequant_rows(rows["kc"][0], rows["kp"][0]))
        v_log.append(oaffine.int4_dequant_rows(rows["vc"][0], rows["vp"][0]))
    q = synth.normal(g, (B, Hq, D))
    ref = np.stack([np.stack([oattn.attend(q[b, h].astype(np.float64), k_log[b][h // G], v_log[b][h // G],
                                           1 / np.sqrt(D)) for h in range(Hq)]) for b in range(B)])
    kc_d, vc_d = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    kp_d = torch.from_numpy(kp.view(np.int16)).to(DEV).view(torch.float16)
    vp_d = torch.from_numpy(vp.view(np.int16)).to(DEV).view(torch.float16)
    for S in [0, 1, 4]:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, S))
        pkv.paged_decode_attention_int4(torch.from_numpy(q).to(DEV), kc_d, kp_d, vc_d, vp_d, table, maxb, bs,
                                        lengths, out, ws, pool=lib_pool, num_splits=S)
        assert rel_err_rows(_out_f64(out), ref) <= TOL["int4"], S
    for W in [0, 17, 100]:          # left window: keys [L - 1 - W, L - 1]
        ref_w = np.stack([np.stack([oattn.attend(q[b, h].astype(np.float64),
                                                 k_log[b][h // G][oattn.visible_begin(int(lengths[b]) - 1, W):],
                                                 v_log[b][h // G][oattn.visible_begin(int(lengths[b]) - 1, W):],
                                                 1 / np.sqrt(D)) for h in range(Hq)]) for b in range(B)])
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs))
        pkv.paged_decode_attention_int4(torch.from_numpy(q).to(DEV), kc_d, kp_d, vc_d, vp_d, table, maxb, bs,
                                        lengths, out, ws, pool=lib_pool, left_window=W)
        assert rel_err_rows(_out_f64(out), ref_w) <= TOL["int4"], W
