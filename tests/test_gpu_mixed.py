"""GPU parity of mixed-format pages against the oracle: appends and page
conversions bit for bit (pool bytes and page descriptors), decode attention
within tolerance, and the pages' four-step accuracy table through the GPU path."""
import struct

import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import mixed as omixed
from oracle import numeric as onum
from tests.gpu_util import DEV, bf16_dev, bits_host, bytes_host, rel_err_rows, require_gpu, workspace

pytestmark = pytest.mark.gpu

F = omixed.Format
TOL_F32 = 1e-5       # float32 output, against the oracle on exactly decoded values
TOL_BF16 = 2.0 ** -8 + 2e-5   # bf16 output: one rounding (unit roundoff 2^-8) of the float32 result
AFFINE = {"INT8": (0.02, -3), "UINT8": (0.02, 130), "INT4": (0.3, 1), "UINT4": (0.3, 8), "INT2": (0.8, 0),
          "UINT2": (0.8, 2)}
ALL = ["BF16", "F16"] + list(AFFINE)


def fmt(name):
    if name in AFFINE:
        s, z = AFFINE[name]
        return F(name, float(np.float32(s)), z)
    return F(name)


def lib_fmt(f: F):
    return pkv.page_format(f.storage, f.scale, f.zero_point)


class Case:
    """One mixed pool driven through the library and the oracle in lockstep."""

    def __init__(self, seed, B, Hkv, bs, NB, maxb, D=128):
        self.g = synth.rng(seed)
        self.B, self.H, self.bs, self.NB, self.maxb, self.D = B, Hkv, bs, NB, maxb, D
        order = synth.permutation(synth.rng(seed, 1), NB)
        self.pool = pkv.Pool(NB, bs, B, maxb, order)
        self.opool = ocache.PagePool(NB, bs, B, maxb, order)
        self.table = torch.zeros((B, maxb), dtype=torch.int32, device=DEV)
        self.k = torch.zeros((NB, Hkv, bs, D), dtype=torch.bfloat16, device=DEV)
        self.v = torch.zeros((NB, Hkv, bs, D), dtype=torch.bfloat16, device=DEV)
        self.desc = pkv.mixed_page_desc(NB, DEV)
        self.binds = [pkv.bind_writable(t) for t in (self.k, self.v, self.desc)]
        self.ref = omixed.MixedPool(NB, Hkv, bs, D)
        self.lens = np.zeros(B, np.int64)

    def append(self, n, kf: F, vf: F, sigma=1.0):
        B, H, D = self.B, self.H, self.D
        new = [int(L) + n for L in self.lens]
        self.pool.reserve(list(range(B)), new, self.table)
        for b in range(B):
            self.opool.reserve(b, new[b])
        kb = synth.f32_to_bf16_bits(synth.normal(self.g, (B, H, n, D), sigma))
        vb = synth.f32_to_bf16_bits(synth.normal(self.g, (B, H, n, D), sigma))
        pkv.mixed_cache_update(self.pool, self.k, self.v, self.desc, self.table, bf16_dev(kb), bf16_dev(vb),
                               self.lens.tolist(), n, lib_fmt(kf), lib_fmt(vf))
        self.ref.append(self.opool.table, kb, vb, self.lens, n, kf, vf)
        self.lens += n

    def check_storage(self):
        assert np.array_equal(self.pool.table(), self.opool.table)
        for name, t in (("k", self.k), ("v", self.v)):
            got = bytes_host(t).reshape(self.NB, self.H, -1)
            assert np.array_equal(got, self.ref.data[name]), name
        d = bytes_host(self.desc).reshape(self.NB, 16)
        for p in range(self.NB):
            for which, off_s, off_z, off_t in (("k", 0, 8, 12), ("v", 4, 10, 13)):
                f = self.ref.fmt[which][p]
                if f is None:
                    continue
                assert d[p, off_t] == pkv.PAGE_STORAGES[f.storage], (p, which)
                if f.affine:
                    assert struct.unpack("<f", d[p, off_s:off_s + 4].tobytes())[0] == np.float32(f.scale)
                    assert struct.unpack("<h", d[p, off_z:off_z + 2].tobytes())[0] == f.zero_point

    def attend(self, G, lens=None, window=-1, num_splits=0, out_dtype=torch.float32):
        lens = self.lens if lens is None else np.asarray(lens)
        Hq = self.H * G
        qb = synth.f32_to_bf16_bits(synth.normal(self.g, (self.B, Hq, self.D)))
        out = torch.empty((self.B, Hq, self.D), dtype=out_dtype, device=DEV)
        ws = workspace(pkv.decode_workspace_size(self.B, Hq, self.H, self.D, int(lens.max()), num_splits))
        pkv.paged_decode_attention_mixed(bf16_dev(qb), self.k, self.v, self.desc, self.table, self.maxb, self.bs,
                                         lens.tolist(), out, ws, pool=self.pool, num_splits=num_splits,
                                         left_window=window)
        ref = omixed.decode_attention(self.ref, onum.bf16_to_f64(qb), self.opool.table, lens, None, window)
        if out_dtype == torch.bfloat16:
            got = onum.bf16_to_f64(bits_host(out))
        else:
            torch.cuda.synchronize()
            got = out.double().cpu().numpy()
        return got, ref

    def close(self):
        for b in self.binds:
            b.close()


@pytest.mark.parametrize("kname", ALL)
def test_append_every_storage_bit_exact(kname):
    """Every storage as K (and a different one as V), ragged positions, pages
    continued across appends: pool bytes and descriptors equal the oracle's."""
    require_gpu()
    vname = ALL[(ALL.index(kname) + 3) % len(ALL)]
    c = Case(900 + ALL.index(kname), B=3, Hkv=2, bs=16, NB=40, maxb=8)
    try:
        c.append(5, fmt(kname), fmt(vname))
        c.append(13, fmt(vname), fmt(kname))        # fills the partial pages in their own format
        c.append(1, fmt("BF16"), fmt("INT2"))
        c.append(30, fmt(kname), fmt(vname), sigma=3.0)   # saturating values
        c.check_storage()
    finally:
        c.close()


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_over_mixed_pages_matches_oracle(G):
    require_gpu()
    c = Case(910 + G, B=4, Hkv=2, bs=16, NB=160, maxb=40)
    try:
        for i, n in enumerate([40, 17, 64, 3, 100, 9]):
            c.append(n, fmt(ALL[i % 8]), fmt(ALL[(i + 5) % 8]))
        got, ref = c.attend(G)
        assert rel_err_rows(got, ref) <= TOL_F32
        got, ref = c.attend(G, out_dtype=torch.bfloat16)
        assert rel_err_rows(got, ref) <= TOL_BF16
    finally:
        c.close()


@pytest.mark.parametrize("bs", [16, 32, 64])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_ragged_lengths_windows_and_splits(bs, splits):
    require_gpu()
    c = Case(920 + bs + splits, B=5, Hkv=2, bs=bs, NB=128, maxb=24)
    try:
        c.append(1, fmt("INT8"), fmt("UINT4"))
        c.append(200, fmt("UINT4"), fmt("INT8"))
        c.append(150, fmt("F16"), fmt("INT2"))
        lens = [1, 16, 17, 300, 351]
        for window in (-1, 0, 5, 64, 1000):
            got, ref = c.attend(4, lens=lens, window=window, num_splits=splits)
            assert rel_err_rows(got, ref) <= TOL_F32, window
    finally:
        c.close()


def test_all_bf16_pages_equal_the_bf16_kernel():
    """A pool of BF16 pages is a bf16 pool: the mixed kernel agrees with the
    plain paged kernel on the same bytes."""
    require_gpu()
    c = Case(930, B=3, Hkv=2, bs=16, NB=64, maxb=20)
    try:
        c.append(250, fmt("BF16"), fmt("BF16"))
        q = torch.randn((3, 8, 128), device=DEV).to(torch.bfloat16)
        o1 = torch.empty((3, 8, 128), device=DEV)
        o2 = torch.empty((3, 8, 128), device=DEV)
        ws = workspace(pkv.decode_workspace_size(3, 8, 2, 128, 250, 0))
        lens = [250, 100, 7]
        pkv.paged_decode_attention_mixed(q, c.k, c.v, c.desc, c.table, c.maxb, c.bs, lens, o1, ws)
        pkv.paged_decode_attention(q, c.k, c.v, c.table, c.maxb, c.bs, lens, o2, ws)
        torch.cuda.synchronize()
        assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)
    finally:
        c.close()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_page_conversion_bit_exact(seed):
    """Selected pages re-encoded (K and V to their own formats, or one kept),
    partial pages included, several conversions in a row; then attention."""
    require_gpu()
    c = Case(940 + seed, B=2, Hkv=2, bs=16, NB=48, maxb=12)
    g = synth.rng(941, seed)
    try:
        c.append(37, fmt("BF16"), fmt("BF16"))
        c.append(40, fmt("UINT4"), fmt("INT8"))
        table = c.opool.table
        for round_ in range(4):
            b = round_ % 2
            held = -(-int(c.lens[b]) // c.bs)
            blocks = sorted(g.choice(held, size=min(held, 3), replace=False).tolist())
            pages = [int(table[b, j]) for j in blocks]
            valid = [min(c.bs, int(c.lens[b]) - j * c.bs) for j in blocks]
            kf = fmt(ALL[int(g.integers(8))])
            vf = None if round_ == 2 else fmt(ALL[int(g.integers(8))])
            pkv.mixed_convert_pages(c.k, c.v, c.desc, pages, valid, lib_fmt(kf),
                                    None if vf is None else lib_fmt(vf))
            c.ref.convert(pages, valid, kf, vf)
            c.check_storage()
        got, ref = c.attend(2)
        assert rel_err_rows(got, ref) <= TOL_F32
    finally:
        c.close()


def test_worked_conversion_example_on_the_gpu():
    """The pages' example: a block to INT2 keys / UINT4 values, then FLOAT16 keys
    and BFLOAT16 values (hand-derived bytes in tests/golden)."""
    require_gpu()
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "mixed_convert_example.json")) as f:
        gx = json.load(f)
    D = 16                                    # the example's 4 values, then zeros
    k = torch.zeros((8, 1, 16, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((8, 1, 16, D), dtype=torch.bfloat16, device=DEV)
    d = pkv.mixed_page_desc(8, DEV)
    pool = pkv.Pool(8, 16, 1, 1, [3, 0, 1, 2, 4, 5, 6, 7])
    table = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    pool.reserve([0], [3], table)
    kv = np.zeros((1, 1, 3, D), np.float32)
    vv = np.zeros((1, 1, 3, D), np.float32)
    kv[0, 0, :, :4] = gx["k_values"]
    vv[0, 0, :, :4] = gx["v_values"]
    with pkv.bind_writable(k), pkv.bind_writable(v), pkv.bind_writable(d):
        pkv.mixed_cache_update(pool, k, v, d, table, bf16_dev(synth.f32_to_bf16_bits(kv)),
                               bf16_dev(synth.f32_to_bf16_bits(vv)), [0], 3, pkv.page_format("BF16"),
                               pkv.page_format("BF16"))
        ki, vu = gx["k_int2"], gx["v_uint4"]
        pkv.mixed_convert_pages(k, v, d, [3], [3], pkv.page_format("INT2", ki["scale"], ki["zero_point"]),
                                pkv.page_format("UINT4", vu["scale"], vu["zero_point"]))
        kb = bytes_host(k).reshape(8, -1)[3]
        vb = bytes_host(v).reshape(8, -1)[3]
        # D = 16 INT2 row = 4 bytes: the example's byte, then three bytes of zero codes
        assert [kb[4 * r] for r in range(4)] == [int(h, 16) for h in ki["row_bytes_hex"]]
        assert all(kb[4 * r + i] == 0 for r in range(4) for i in (1, 2, 3))
        assert [vb[8 * r:8 * r + 2].tobytes().hex() for r in range(4)] == vu["row_bytes_hex"]
        pkv.mixed_convert_pages(k, v, d, [3], [3], pkv.page_format("F16"), pkv.page_format("BF16"))
        k16 = bits_host(k)[3, 0, :4, :4]
        v16 = bits_host(v)[3, 0, :4, :4]
        assert k16.tolist() == [[int(h, 16) for h in r] for r in gx["k_f16_bits"]]
        assert v16.tolist() == [[int(h, 16) for h in r] for r in gx["v_bf16_bits"]]


def test_four_step_accuracy_table_on_the_gpu():
    """The pages' fixture (components +/-(0.173 * step), four steps, each of its
    storages): the GPU output after every step against unquantised attention
    within the table's tolerance, and against the oracle's mixed pages."""
    require_gpu()
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "quant_accuracy_table.json")) as f:
        tab = json.load(f)
    D = 128
    sign = np.array([(-1) ** d for d in range(D)], np.float32)
    for row in tab["rows"]:
        f = F(row["storage"], row["scale"], row["zero_point"])
        k = torch.zeros((4, 1, 16, D), dtype=torch.bfloat16, device=DEV)
        v = torch.zeros_like(k)
        d = pkv.mixed_page_desc(4, DEV)
        pool = pkv.Pool(4, 16, 1, 1)
        table = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
        ref = omixed.MixedPool(4, 1, 16, D)
        opool = ocache.PagePool(4, 16, 1, 1)
        exact = []
        with pkv.bind_writable(k), pkv.bind_writable(v), pkv.bind_writable(d):
            for step in range(1, 5):
                xb = synth.f32_to_bf16_bits(np.float32(tab["component_per_step"] * step) * sign)
                pool.reserve([0], [step], table)
                opool.reserve(0, step)
                xd = bf16_dev(xb.reshape(1, 1, 1, D))
                pkv.mixed_cache_update(pool, k, v, d, table, xd, xd, [step - 1], 1, lib_fmt(f), lib_fmt(f))
                ref.append(opool.table, xb.reshape(1, 1, 1, D), xb.reshape(1, 1, 1, D), [step - 1], 1, f, f)
                exact.append(onum.bf16_to_f64(xb))
                out = torch.empty((1, 1, D), device=DEV)
                ws = workspace(pkv.decode_workspace_size(1, 1, 1, D, 16, 0))
                pkv.paged_decode_attention_mixed(bf16_dev(xb.reshape(1, 1, D)), k, v, d, table, 1, 16, [step], out, ws)
                torch.cuda.synchronize()
                got = out.double().cpu().numpy()
                qx = onum.bf16_to_f64(xb)[None, None]
                E = np.array(exact)[None, None]
                dense = oattn.decode_attention(qx, E, E, [step])
                assert np.abs(got - dense).max() <= row["tolerance"], (row, step)
                mixed_ref = omixed.decode_attention(ref, qx, opool.table, [step])
                assert np.abs(got - mixed_ref).max() <= 1e-5, (row, step)
