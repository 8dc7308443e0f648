"""The fused decode step (`pkv_decode_step`): one launch that appends the new K/V rows into contiguous caches and
attends over the valid prefix.  It must leave the caches byte for byte and the output bit for bit as the
append followed by the attention call do (those two are checked against the oracle elsewhere; one case here is
checked against the oracle as well): fast and generic kernels, splits, windows whose first visible token lies
after some of the new rows, several new tokens, values at an odd element offset, and 300-row batches (two
launches)."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
from oracle import attention as oattn
from tests.gpu_util import DEV, rel_err_rows, require_gpu, workspace
from tests.test_gpu_decode import TOL

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _rand(gen, shape, dt, offset=0):
    x = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32).to(dt)
    if offset:          # the same values at an element offset of a larger buffer
        buf = torch.zeros(x.numel() + offset, dtype=dt, device=DEV)
        buf[offset:] = x.reshape(-1)
        x = buf[offset:].view(x.shape)
    return x


def _run(seed, B, Hq, Hkv, D, Dv, cap, pos, n, kind, S, W, out_kind="f32", offset=0):
    dt = DT[kind]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    kc = _rand(gen, (B, Hkv, cap, D), dt)
    vc = _rand(gen, (B, Hkv, cap, Dv), dt)
    kv = _rand(gen, (B, Hkv, n, D), dt, offset)
    vv = _rand(gen, (B, Hkv, n, Dv), dt, offset)
    q = _rand(gen, (B, Hq, D), dt)
    pos = [int(p) for p in pos]
    lens = [p + n for p in pos]
    caches = [(kc.clone(), vc.clone()) for _ in range(2)]
    outs = [torch.empty((B, Hq, Dv), dtype=DT[out_kind], device=DEV) for _ in range(2)]
    nbytes = pkv.decode_workspace_size(B, Hq, Hkv, D, cap, S)
    wss = [workspace(nbytes) for _ in range(2)]
    (k1, v1), (k2, v2) = caches
    with pkv.bind_writable(k1), pkv.bind_writable(v1):
        if D == Dv:
            pkv.cache_update_kv(k1, v1, kv, vv, pos, n)
        else:           # the paired append takes equal shapes only
            pkv.cache_update(k1, kv, pos, n)
            pkv.cache_update(v1, vv, pos, n)
    pkv.decode_attention(q, k1, v1, lens, outs[0], wss[0], num_splits=S, left_window=W)
    with pkv.bind_writable(k2), pkv.bind_writable(v2):
        pkv.decode_step(k2, v2, kv, vv, pos, n, q, outs[1], wss[1], num_splits=S, left_window=W)
    torch.cuda.synchronize()
    for a, b in ((k1, k2), (v1, v2), (outs[0], outs[1])):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    return dict(q=q, k=k2, v=v2, out=outs[1], lens=lens)


@pytest.mark.parametrize("kind,G,n,S", [("bf16", 4, 1, 0), ("bf16", 1, 5, 3), ("f16", 8, 1, 1), ("bf16", 2, 2, 7),
                                        ("bf16", 4, 70, 0)])
def test_fast_kernel_step_equals_append_then_attention(kind, G, n, S):
    require_gpu()
    B, Hkv, D, cap = 5, 2, 128, 900
    pos = [0, 63, 127, 700, 900 - n]
    r = _run(1400 + G + n + S, B, Hkv * G, Hkv, D, D, cap, pos, n, kind, S, -1)
    if kind == "bf16" and S == 0 and n == 1:         # and against the oracle
        qh = r["q"].double().cpu().numpy()
        kh = r["k"].double().cpu().numpy()
        vh = r["v"].double().cpu().numpy()
        ref = oattn.decode_attention(qh, kh, vh, np.array(r["lens"]))
        assert rel_err_rows(r["out"].double().cpu().numpy(), ref) <= TOL["f32"]


@pytest.mark.parametrize("kind,D,Dv,G,n,S", [("f32", 4, 4, 1, 1, 0), ("bf16", 64, 32, 2, 3, 2), ("f16", 8, 8, 4, 1, 5),
                                             ("f32", 128, 128, 2, 4, 0)])
def test_generic_kernel_step_equals_append_then_attention(kind, D, Dv, G, n, S):
    require_gpu()
    B, Hkv, cap = 4, 2, 300
    _run(1420 + D + Dv + n, B, Hkv * G, Hkv, D, Dv, cap, [0, 1, 150, cap - n], n, kind, S, -1)


@pytest.mark.parametrize("kind,D,W,n", [("bf16", 128, 0, 3), ("bf16", 128, 5, 8), ("f32", 16, 0, 2), ("bf16", 128, 40, 1)])
def test_window_step_writes_rows_before_the_visible_range(kind, D, W, n):
    """With a left window narrower than the new tokens, some new rows lie before the first split's range (which
    starts at the visible range's 64-token quantum); they are written all the same."""
    require_gpu()
    B, Hkv, G, cap = 4, 2, 2, 400
    pos = [64 - n + 1, 128 - n + 1, 200, cap - n]      # the last new row at a quantum start in the first two rows
    _run(1440 + D + W + n, B, Hkv * G, Hkv, D, D, cap, pos, n, kind, 0, W)


def test_unaligned_values_and_bf16_output():
    require_gpu()
    _run(1460, 3, 8, 2, 128, 128, 500, [10, 260, 499], 1, "bf16", 0, -1, out_kind="bf16", offset=1)


def test_300_rows_and_a_plain_decode():
    require_gpu()
    B = 300
    pos = np.random.default_rng(1470).integers(0, 197, size=B)
    _run(1471, B, 4, 2, 128, 128, 200, pos, 3, "bf16", 0, -1)
    _run(1472, B, 4, 2, 8, 8, 50, np.maximum(pos % 50, 1), 0, "f32", 2, -1)      # update_length 0


def test_step_errors_write_nothing():
    require_gpu()
    B, Hkv, Hq, D, cap = 2, 2, 4, 128, 512
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1480)
    kc, vc = _rand(gen, (B, Hkv, cap, D), torch.bfloat16), _rand(gen, (B, Hkv, cap, D), torch.bfloat16)
    kv, vv = _rand(gen, (B, Hkv, 2, D), torch.bfloat16), _rand(gen, (B, Hkv, 2, D), torch.bfloat16)
    q = _rand(gen, (B, Hq, D), torch.bfloat16)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    k0, v0 = kc.clone(), vc.clone()
    with pytest.raises(pkv.PkvError) as e:               # read-only caches
        pkv.decode_step(kc, vc, kv, vv, [3, 4], 2, q, out)
    assert e.value.status == pkv.E_READONLY
    with pkv.bind_writable(kc), pkv.bind_writable(vc):
        with pytest.raises(pkv.PkvError) as e:           # one row past the capacity
            pkv.decode_step(kc, vc, kv, vv, [3, cap - 1], 2, q, out)
        assert e.value.status == pkv.E_CAPACITY
        with pytest.raises(pkv.PkvError) as e:           # q inside a cache
            pkv.decode_step(kc, vc, kv, vv, [3, 4], 2, kc[0, 0, :B * Hq].reshape(B, Hq, D), out)
        assert e.value.status == pkv.E_ALIAS
        ws = workspace(pkv.decode_workspace_size(B, Hq, Hkv, D, cap, 4))
        with pytest.raises(pkv.PkvError) as e:           # workspace too small for four splits
            pkv.decode_step(kc, vc, kv, vv, [300, 400], 2, q, out, ws[:256], num_splits=4)
        assert e.value.status == pkv.E_NOMEM
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), k0.view(torch.int16)) and torch.equal(vc.view(torch.int16), v0.view(torch.int16))
