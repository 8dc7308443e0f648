"""The device-driven decode step: K and V appended in one launch at positions
held in device memory, lengths advanced on the device, attention over device
lengths, sampling seeded from a device step counter.  Run eagerly and as a
captured HIP graph replayed over several advancing steps, it matches the
oracle's stateful loop each step (f32 output at the fp32 bar, cache bytes
bit for bit) and the replays equal the eager run bit for bit.  Device-side
checks: positions past capacity, unreserved pages and lengths past the bound
set the status word and write nothing."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import attention as oattn
from oracle import cache as ocache
from oracle import numeric as onum
from oracle import sampling as osamp
from tests.gpu_util import DEV, bf16_dev, bits_host, rel_err_rows, require_gpu, workspace

pytestmark = pytest.mark.gpu
F32_TOL = 1e-5


def _step_inputs(seed, steps, B, Hq, Hkv, D):
    g = synth.rng(seed, 50)
    q = synth.f32_to_bf16_bits(synth.normal(g, (steps, B, Hq, D)))
    k = synth.f32_to_bf16_bits(synth.normal(g, (steps, B, Hkv, 1, D)))
    v = synth.f32_to_bf16_bits(synth.normal(g, (steps, B, Hkv, 1, D)))
    return q, k, v


class _Contig:
    """Contiguous caches with a prefix per row, the oracle's copy, and the step's fixed device buffers."""

    def __init__(self, seed, B, Hq, Hkv, D, cap, L0):
        g = synth.rng(seed)
        self.B, self.Hq, self.Hkv, self.D, self.cap = B, Hq, Hkv, D, cap
        self.kh = np.zeros((B, Hkv, cap, D), np.uint16)
        self.vh = np.zeros_like(self.kh)
        for b in range(B):
            self.kh[b, :, :L0[b]] = synth.f32_to_bf16_bits(synth.normal(g, (Hkv, int(L0[b]), D)))
            self.vh[b, :, :L0[b]] = synth.f32_to_bf16_bits(synth.normal(g, (Hkv, int(L0[b]), D)))
        self.kc, self.vc = bf16_dev(self.kh), bf16_dev(self.vh)
        self.lens = torch.from_numpy(np.asarray(L0, np.int32)).to(DEV)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.step = torch.zeros(1, dtype=torch.int64, device=DEV)
        self.q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
        self.k = torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=DEV)
        self.v = torch.empty_like(self.k)
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
        self.ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap))
        self.binds = [pkv.bind_writable(self.kc), pkv.bind_writable(self.vc)]

    def run(self):
        """append K and V at lens, lens += 1 (and the step counter), attention over lens"""
        pkv.cache_update_kv_dev(self.kc, self.vc, self.k, self.v, self.lens, 1, self.status)
        pkv.advance(self.lens, 1, self.step)
        pkv.decode_attention_dev(self.q, self.kc, self.vc, self.lens, self.cap, self.out, self.status, self.ws)

    def close(self):
        for b in self.binds:
            b.close()


def _oracle_step(kh, vh, L, qs, ks, vs):
    """the oracle's stateful step: append at L, attention over L + 1 (f64)"""
    ocache.cache_update(kh, ks, L, 1)
    ocache.cache_update(vh, vs, L, 1)
    L = L + 1
    B, Hq, D = qs.shape
    G = Hq // kh.shape[1]
    qd = onum.bf16_to_f64(qs)
    ref = np.stack([np.stack([oattn.attend(qd[b, h], onum.bf16_to_f64(kh[b, h // G, :L[b]]),
                                           onum.bf16_to_f64(vh[b, h // G, :L[b]]), 1 / np.sqrt(D))
                              for h in range(Hq)]) for b in range(B)])
    return L, ref


@pytest.mark.parametrize("G", [4, 1])
def test_contiguous_device_step_eager_and_graph_replays(G):
    require_gpu()
    B, Hkv, D, cap, steps = 4, 2, 128, 700, 6
    Hq = Hkv * G
    L0 = np.array([1, 40, 333, 600], np.int32)
    qs, ks, vs = _step_inputs(880 + G, steps, B, Hq, Hkv, D)
    eager = _Contig(881, B, Hq, Hkv, D, cap, L0)
    graphed = _Contig(881, B, Hq, Hkv, D, cap, L0)
    kh, vh, L = eager.kh.copy(), eager.vh.copy(), L0.copy()
    # capture one step of the second instance (its buffers are fixed; the inputs are copied in per replay)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    for t in range(steps):
        for inst in (eager, graphed):
            inst.q.copy_(bf16_dev(qs[t]))
            inst.k.copy_(bf16_dev(ks[t]))
            inst.v.copy_(bf16_dev(vs[t]))
        eager.run()
        g.replay()
        torch.cuda.synchronize()
        L, ref = _oracle_step(kh, vh, L, qs[t], ks[t], vs[t])
        got = eager.out.double().cpu().numpy()
        assert rel_err_rows(got, ref) <= F32_TOL, t
        assert np.array_equal(graphed.out.cpu().numpy(), eager.out.cpu().numpy()), t
        assert np.array_equal(eager.lens.cpu().numpy(), L) and np.array_equal(graphed.lens.cpu().numpy(), L)
    for inst in (eager, graphed):
        assert np.array_equal(bits_host(inst.kc), kh) and np.array_equal(bits_host(inst.vc), vh)
        assert int(inst.status.item()) == 0 and int(inst.step.item()) == steps
        inst.close()


def test_paged_device_step_eager_and_graph_replays():
    """Paged pools: reserve the final lengths up front, then the captured step appends and attends as the rows
    grow across page boundaries (block size 16), in the bench's split configuration (bound = the longest row)."""
    require_gpu()
    B, Hq, Hkv, D, bs, steps = 4, 16, 4, 128, 16, 20
    L0 = np.array([1, 15, 250, 1000], np.int32)
    maxb = -(-(int(L0.max()) + steps) // bs) + 1
    g0 = synth.rng(890)
    NB = int(sum(-(-(int(x) + steps) // bs) for x in L0)) + 3
    order = synth.permutation(g0, NB)
    ref_pool = ocache.PagePool(NB, bs, B, maxb, order)
    kp = np.zeros((NB, Hkv, bs, D), np.uint16)
    vp = np.zeros_like(kp)
    k_log = [synth.f32_to_bf16_bits(synth.normal(synth.rng(890, 1, b), (1, Hkv, int(L0[b]), D))) for b in range(B)]
    v_log = [synth.f32_to_bf16_bits(synth.normal(synth.rng(890, 2, b), (1, Hkv, int(L0[b]), D))) for b in range(B)]
    for b in range(B):
        ref_pool.reserve(b, int(L0[b]) + steps)
        ocache.paged_cache_update(kp, ref_pool.table[b:b + 1], k_log[b], [0], int(L0[b]), bs)
        ocache.paged_cache_update(vp, ref_pool.table[b:b + 1], v_log[b], [0], int(L0[b]), bs)
    qs, ks, vs = _step_inputs(891, steps, B, Hq, Hkv, D)
    max_len = int(L0.max()) + steps

    def make():
        lib_pool = pkv.Pool(NB, bs, B, maxb, order)
        table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
        lib_pool.reserve(range(B), (L0 + steps).tolist(), table)
        st = dict(pool=lib_pool, table=table, kd=bf16_dev(kp), vd=bf16_dev(vp),
                  lens=torch.from_numpy(L0.copy()).to(DEV), status=torch.zeros(1, dtype=torch.int32, device=DEV),
                  q=torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV),
                  k=torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=DEV),
                  v=torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=DEV),
                  out=torch.empty((B, Hq, D), dtype=torch.float32, device=DEV),
                  ws=workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, max_len)))
        st["binds"] = [pkv.bind_writable(st["kd"]), pkv.bind_writable(st["vd"])]
        return st

    def run(st):
        pkv.paged_cache_update_kv_dev(st["pool"], st["kd"], st["vd"], st["table"], st["k"], st["v"], st["lens"], 1,
                                      st["status"])
        pkv.advance(st["lens"], 1)
        pkv.paged_decode_attention_dev(st["q"], st["kd"], st["vd"], st["table"], maxb, bs, st["lens"], max_len,
                                       st["out"], st["status"], st["ws"], pool=st["pool"])

    eager, graphed = make(), make()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graphed)
    torch.cuda.synchronize()
    kph, vph, L = kp.copy(), vp.copy(), L0.copy()
    G = Hq // Hkv
    for t in range(steps):
        for st in (eager, graphed):
            st["q"].copy_(bf16_dev(qs[t]))
            st["k"].copy_(bf16_dev(ks[t]))
            st["v"].copy_(bf16_dev(vs[t]))
        run(eager)
        g.replay()
        torch.cuda.synchronize()
        ocache.paged_cache_update(kph, ref_pool.table, ks[t], L, 1, bs, ref_pool.held)
        ocache.paged_cache_update(vph, ref_pool.table, vs[t], L, 1, bs, ref_pool.held)
        L = L + 1
        qd = onum.bf16_to_f64(qs[t])
        ref = np.stack([np.stack([oattn.attend(
            qd[b, h], onum.bf16_to_f64(ocache.paged_gather(kph, ref_pool.table[b], int(L[b]), bs)[h // G]),
            onum.bf16_to_f64(ocache.paged_gather(vph, ref_pool.table[b], int(L[b]), bs)[h // G]), 1 / np.sqrt(D))
            for h in range(Hq)]) for b in range(B)])
        got = eager["out"].double().cpu().numpy()
        assert rel_err_rows(got, ref) <= F32_TOL, t
        assert np.array_equal(graphed["out"].cpu().numpy(), eager["out"].cpu().numpy()), t
    for st in (eager, graphed):
        assert np.array_equal(bits_host(st["kd"]), kph) and np.array_equal(bits_host(st["vd"]), vph)
        assert int(st["status"].item()) == 0
        for bnd in st["binds"]:
            bnd.close()


def test_device_step_checks_set_the_status_word_and_write_nothing():
    require_gpu()
    B, Hq, Hkv, D, cap = 3, 4, 2, 128, 64
    inst = _Contig(895, B, Hq, Hkv, D, cap, np.array([10, 63, 5], np.int32))
    inst.k.copy_(torch.randn_like(inst.k, dtype=torch.float32).to(torch.bfloat16))
    inst.v.copy_(torch.randn_like(inst.v, dtype=torch.float32).to(torch.bfloat16))
    before = (inst.kc.clone(), inst.vc.clone())
    inst.lens.copy_(torch.tensor([10, 64, 5], dtype=torch.int32))         # row 1 is full: no row may be written
    pkv.cache_update_kv_dev(inst.kc, inst.vc, inst.k, inst.v, inst.lens, 1, inst.status)
    torch.cuda.synchronize()
    assert int(inst.status.item()) == pkv.E_CAPACITY
    assert torch.equal(inst.kc, before[0]) and torch.equal(inst.vc, before[1])
    # attention: a length past the bound leaves that row's output alone, the others are computed
    inst.status.zero_()
    inst.out.fill_(float("nan"))
    inst.lens.copy_(torch.tensor([10, 40, 5], dtype=torch.int32))
    pkv.decode_attention_dev(inst.q.normal_(), inst.kc, inst.vc, inst.lens, 32, inst.out, inst.status, inst.ws)
    torch.cuda.synchronize()
    assert int(inst.status.item()) == pkv.E_CAPACITY
    o = inst.out.cpu()
    assert torch.isnan(o[1]).all() and not torch.isnan(o[0]).any() and not torch.isnan(o[2]).any()
    inst.close()
    # paged: a page that was never reserved (-1 in the table) is reported and nothing is written
    NB, bs, maxb = 8, 16, 4
    pool = pkv.Pool(NB, bs, 2, maxb)
    table = torch.full((2, maxb), -1, dtype=torch.int32, device=DEV)
    pool.reserve([0, 1], [16, 16], table)
    kp = torch.zeros((NB, Hkv, bs, D), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    kv = torch.ones((2, Hkv, 1, D), dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    pos = torch.tensor([3, 16], dtype=torch.int32, device=DEV)             # row 1's second page is not reserved
    with pkv.bind_writable(kp), pkv.bind_writable(vp):
        pkv.paged_cache_update_kv_dev(pool, kp, vp, table, kv, kv, pos, 1, status)
    torch.cuda.synchronize()
    assert int(status.item()) == pkv.E_PAGE
    assert not kp.any() and not vp.any()


def test_sample_dev_follows_the_device_step_counter():
    """pkv_sample_dev at counter t equals pkv_sample with pkv_generate_step_seed(seed, t, B, V), and both equal
    the oracle's draw up to float32 near-ties; a captured draw + advance replays t = 0, 1, 2, ..."""
    require_gpu()
    B, V, T, seed = 16, 5000, 0.8, 77
    x = synth.normal(synth.rng(896), (B, V), 3.0)
    logits = torch.from_numpy(x).to(DEV)
    ws = workspace(pkv.sample_workspace_size(B, V))
    step = torch.zeros(1, dtype=torch.int64, device=DEV)
    ids = torch.empty(B, dtype=torch.int64, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.sample_dev(logits, T, seed, step, ids, ws)
        pkv.advance(None, 0, step)
    torch.cuda.synchronize()
    ref_ids = torch.empty(B, dtype=torch.int64, device=DEV)
    ws2 = workspace(pkv.sample_workspace_size(B, V))
    for t in range(4):
        g.replay()
        pkv.sample(logits, T, pkv.generate_step_seed(seed, t, B, V), ref_ids, ws2)
        torch.cuda.synchronize()
        got = ids.cpu().numpy()
        assert np.array_equal(got, ref_ids.cpu().numpy()), t
        want = osamp.sample(x, T, pkv.generate_step_seed(seed, t, B, V))
        for b in np.nonzero(got != want)[0]:
            sc = osamp.gumbel_scores(x[b], T, pkv.generate_step_seed(seed, t, B, V), b)
            assert abs(sc[got[b]] - sc[want[b]]) <= 1e-5 * max(1.0, abs(sc[want[b]]))
    assert int(step.item()) == 4


@pytest.mark.parametrize("G,D", [(4, 128), (1, 128), (2, 64)])
def test_fused_device_step_equals_the_three_launch_step(G, D):
    """`decode_step_dev` (append at the device positions fused into the attention) followed by the advance, eager
    and as a replayed graph, equals the append / advance / attention sequence bit for bit, step after step."""
    require_gpu()
    B, Hkv, cap, steps = 4, 2, 500, 5
    Hq = Hkv * G
    L0 = np.array([1, 63, 300, 490], np.int32)
    qs, ks, vs = _step_inputs(890 + G + D, steps, B, Hq, Hkv, D)
    insts = [_Contig(891, B, Hq, Hkv, D, cap, L0) for _ in range(3)]    # three launches; fused eager; fused graph

    def fused(inst):
        pkv.decode_step_dev(inst.kc, inst.vc, inst.k, inst.v, inst.lens, 1, inst.q, cap, inst.out, inst.status,
                            inst.ws)
        pkv.advance(inst.lens, 1, inst.step)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fused(insts[2])
    torch.cuda.synchronize()
    for t in range(steps):
        for inst in insts:
            inst.q.copy_(bf16_dev(qs[t]))
            inst.k.copy_(bf16_dev(ks[t]))
            inst.v.copy_(bf16_dev(vs[t]))
        insts[0].run()
        fused(insts[1])
        g.replay()
        torch.cuda.synchronize()
        for inst in insts[1:]:
            assert torch.equal(inst.out.view(torch.int32), insts[0].out.view(torch.int32)), t
            assert torch.equal(inst.lens, insts[0].lens), t
    for inst in insts[1:]:
        assert torch.equal(inst.kc.view(torch.int16), insts[0].kc.view(torch.int16))
        assert torch.equal(inst.vc.view(torch.int16), insts[0].vc.view(torch.int16))
        assert int(inst.status.item()) == 0 and int(inst.step.item()) == steps
    for inst in insts:
        inst.close()


def test_fused_device_step_rejects_a_row_past_the_bound():
    """A row whose position + 1 exceeds max_len writes neither its cache rows nor its output and sets the status
    word; the other rows step as usual."""
    require_gpu()
    B, Hkv, G, D, cap = 3, 2, 4, 128, 256
    Hq = Hkv * G
    L0 = np.array([10, 200, 100], np.int32)
    qs, ks, vs = _step_inputs(895, 1, B, Hq, Hkv, D)
    ref, bad = _Contig(896, B, Hq, Hkv, D, cap, L0), _Contig(896, B, Hq, Hkv, D, cap, L0)
    for inst in (ref, bad):
        inst.q.copy_(bf16_dev(qs[0]))
        inst.k.copy_(bf16_dev(ks[0]))
        inst.v.copy_(bf16_dev(vs[0]))
        inst.out.fill_(7.0)
    max_len = 200                          # row 1 would need 201
    pkv.decode_step_dev(ref.kc, ref.vc, ref.k, ref.v, ref.lens, 1, ref.q, 256, ref.out, ref.status, ref.ws)
    pkv.decode_step_dev(bad.kc, bad.vc, bad.k, bad.v, bad.lens, 1, bad.q, max_len, bad.out, bad.status, bad.ws)
    torch.cuda.synchronize()
    assert int(bad.status.item()) == pkv.E_CAPACITY and int(ref.status.item()) == 0
    kb, vb = bits_host(bad.kc), bits_host(bad.vc)
    assert np.array_equal(kb[1], bad.kh[1]) and np.array_equal(vb[1], bad.vh[1])     # row 1 untouched
    assert bool((bad.out[1] == 7.0).all())
    for b in (0, 2):
        assert np.array_equal(kb[b], bits_host(ref.kc)[b]) and np.array_equal(vb[b], bits_host(ref.vc)[b])
        assert rel_err_rows(bad.out[b].double().cpu().numpy(), ref.out[b].double().cpu().numpy()) <= F32_TOL
    for inst in (ref, bad):
        inst.close()
