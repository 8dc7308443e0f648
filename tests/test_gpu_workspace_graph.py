"""Workspace and graph-capture contracts of the split decode and the sampler:
results do not depend on what the caller's workspace held before the call
(it needs no initialisation), on one workspace serving calls of other
shapes, or on the calls being captured in a HIP graph and replayed several
times with eager calls on the same workspaces in between."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
import synth
from oracle import attention as oattn
from tests.gpu_util import DEV, rel_err_rows, require_gpu, workspace
from tests.test_gpu_decode import _contig_inputs, _out_f64

pytestmark = pytest.mark.gpu


def _fill(ws: torch.Tensor, how: str) -> None:
    if how == "zeros":
        ws.zero_()
    elif how == "ones":
        ws.fill_(0xFF)
    else:
        g = torch.Generator(device=DEV)
        g.manual_seed(5)
        ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device=DEV, dtype=torch.uint8))


def _contig_case(seed=720):
    B, Hq, Hkv, D, cap = 3, 8, 2, 128, 6000
    lengths = np.array([6000, 1500, 700], np.int32)
    q, kc, vc, qh, kh, vh = _contig_inputs(seed, B, Hq, Hkv, D, cap, lengths)
    return dict(B=B, Hq=Hq, Hkv=Hkv, D=D, cap=cap, lengths=lengths, q=q, kc=kc, vc=vc,
                ref=oattn.decode_attention(qh, kh, vh, lengths))


@pytest.mark.parametrize("S", [4, 64, 94])
def test_decode_result_does_not_depend_on_workspace_contents(S):
    require_gpu()
    c = _contig_case()
    ws = workspace(pkv.decode_workspace_size(c["B"], c["Hq"], c["Hkv"], c["D"], c["cap"], S))
    outs = []
    for how in ["zeros", "ones", "random", "reused"]:
        if how != "reused":
            _fill(ws, how)
        out = torch.empty((c["B"], c["Hq"], c["D"]), dtype=torch.float32, device=DEV)
        pkv.decode_attention(c["q"], c["kc"], c["vc"], c["lengths"], out, ws, num_splits=S)
        got = _out_f64(out)
        assert rel_err_rows(got, c["ref"]) <= 1e-5, how
        outs.append(got)
    for got in outs[1:]:
        assert np.array_equal(got, outs[0])     # the same split plan sums in the same order


def test_decode_shared_workspace_across_shapes():
    """Calls of different batch sizes and split counts take turns on one workspace."""
    require_gpu()
    c = _contig_case()
    ws = workspace(pkv.decode_workspace_size(c["B"], c["Hq"], c["Hkv"], c["D"], c["cap"], 64))
    _fill(ws, "random")
    for rep in range(2):
        for S, rows in [(16, 3), (5, 1), (64, 2), (0, 3)]:
            out = torch.empty((rows, c["Hq"], c["D"]), dtype=torch.float32, device=DEV)
            pkv.decode_attention(c["q"][:rows], c["kc"][:rows], c["vc"][:rows], c["lengths"][:rows], out, ws,
                                 num_splits=S)
            assert rel_err_rows(_out_f64(out), c["ref"][:rows]) <= 1e-5, (rep, S, rows)


def test_graph_replays_match_eager_calls():
    """Captured contiguous, paged bf16 and paged INT4 decode (split rows and their merge) and a
    greedy sample, replayed several times with eager calls on the same workspaces in between,
    give the eager results each time."""
    require_gpu()
    c = _contig_case(721)
    B, Hq, Hkv, D, cap = c["B"], c["Hq"], c["Hkv"], c["D"], c["cap"]
    S = 8
    ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, S))
    # INT4 pool, every page of every row written with random codes and parameters
    bs = 16
    maxb = -(-cap // bs)
    NB = int(sum(-(-int(L) // bs) for L in c["lengths"]))
    g = synth.rng(722)
    order = synth.permutation(g, NB)
    pool = pkv.Pool(NB, bs, B, maxb, order)
    table = torch.full((B, maxb), -1, dtype=torch.int32, device=DEV)
    pool.reserve(range(B), c["lengths"].tolist(), table)
    codes = [torch.from_numpy(g.integers(0, 256, size=(NB, Hkv, bs, D // 2), dtype=np.uint8)).to(DEV)
             for _ in range(2)]
    params = []
    for _ in range(2):
        p = np.empty((NB, Hkv, bs, D // 32, 2), np.uint16)
        p[..., 0] = synth.f16_bits(synth.uniform(g, (NB, Hkv, bs, D // 32), 0.01, 0.1))
        p[..., 1] = synth.f16_bits(g.integers(0, 16, size=(NB, Hkv, bs, D // 32)).astype(np.float32))
        params.append(torch.from_numpy(p.view(np.int16)).to(DEV).view(torch.float16))
    gt = torch.Generator(device=DEV)
    gt.manual_seed(724)
    kpool, vpool = (torch.randn((NB, Hkv, bs, D), generator=gt, device=DEV, dtype=torch.bfloat16) for _ in range(2))
    wsp = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap))
    q32 = c["q"].float()
    ws4 = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, S))
    V = 50000
    logits = torch.from_numpy(synth.normal(g, (B, V)) * 3).to(DEV)
    wss = workspace(pkv.sample_workspace_size(B, V))

    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    out4 = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    outp = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty(B, dtype=torch.int64, device=DEV)

    def calls():
        pkv.decode_attention(c["q"], c["kc"], c["vc"], c["lengths"], out, ws, num_splits=S)
        pkv.paged_decode_attention(c["q"], kpool, vpool, table, maxb, bs, c["lengths"], outp, wsp)
        pkv.paged_decode_attention_int4(q32, codes[0], params[0], codes[1], params[1], table, maxb, bs,
                                        c["lengths"], out4, ws4, num_splits=S)
        pkv.sample(logits, 0.0, 0, ids, wss)

    calls()
    torch.cuda.synchronize()
    want = (out.clone(), out4.clone(), ids.clone(), outp.clone())
    assert rel_err_rows(_out_f64(out), c["ref"]) <= 1e-5
    assert torch.equal(ids.cpu(), torch.argmax(logits, dim=1).cpu())

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, out4, outp):
            t.fill_(float("nan"))
        ids.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(out4, want[1]) and torch.equal(ids, want[2]), rep
        assert torch.equal(outp, want[3]), rep
        calls()                       # eager calls in between rewrite the same workspaces
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(out4, want[1]) and torch.equal(ids, want[2]), rep
        assert torch.equal(outp, want[3]), rep


@pytest.mark.parametrize("how", ["zeros", "ones", "random"])
def test_sample_result_does_not_depend_on_workspace_contents(how):
    require_gpu()
    B, V = 5, 151936
    g = synth.rng(723)
    logits = torch.from_numpy(synth.normal(g, (B, V)) * 3).to(DEV)
    ws = workspace(pkv.sample_workspace_size(B, V))
    ids = torch.empty(B, dtype=torch.int64, device=DEV)
    want = torch.argmax(logits, dim=1)
    for rep in range(2):
        _fill(ws, how)
        pkv.sample(logits, 0.0, 0, ids, ws)
        assert torch.equal(ids, want), rep
        pkv.sample(logits, 0.0, 0, ids, ws)     # reused as the call left it
        assert torch.equal(ids, want), rep
