"""pkv_paged_decode_attention_noalloc (split partials in the library's static
device scratch) against pkv_paged_decode_attention with a caller workspace:
bit-identical outputs (same kernels, same split plan) on two calls in a row,
the second with fewer and shorter rows, both within the fp32 bar of the
oracle; a call whose partials exceed the scratch is rejected untouched."""
import numpy as np
import pytest
import torch

import place_persistent_kv_amd as pkv
from tests.gpu_util import DEV, require_gpu, workspace
from tests.test_gpu_decode import TOL, _out_f64, _paged_inputs, _paged_ref
from tests.gpu_util import rel_err_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S", [0, 7])
def test_noalloc_matches_the_workspace_entry_point(S):
    require_gpu()
    B, Hq, Hkv, D, bs, maxb = 6, 16, 4, 128, 16, 130
    lengths = np.array([2000, 1, 17, 700, 2063, 1024], np.int32)
    d = _paged_inputs(990 + S, B, Hq, Hkv, D, bs, lengths, maxb)
    ref = _paged_ref(d, lengths)
    for rows, lens in ((B, lengths), (3, np.array([1333, 1, 9], np.int32))):     # each row's reserved prefix
        q = d["q"][:rows].contiguous()
        want = torch.empty((rows, Hq, D), dtype=torch.float32, device=DEV)
        ws = workspace(pkv.decode_workspace_size(rows, Hq, Hkv, D, maxb * bs, S))
        pkv.paged_decode_attention(q, d["kp"], d["vp"], d["table"], maxb, bs, lens, want, ws, pool=d["pool"],
                                   num_splits=S)
        got = torch.full((rows, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        pkv.paged_decode_attention_noalloc(q, d["kp"], d["vp"], d["table"], maxb, bs, lens, got, pool=d["pool"],
                                           num_splits=S)
        assert np.array_equal(_out_f64(got), _out_f64(want)), rows
        if rows == B:
            assert rel_err_rows(_out_f64(got), ref) <= TOL["f32"]
        else:                                                  # shorter rows: the oracle over their prefixes
            sub = dict(d, qh=d["qh"][:rows], k_log=[d["k_log"][b][:, :lens[b]] for b in range(rows)],
                       v_log=[d["v_log"][b][:, :lens[b]] for b in range(rows)])
            assert rel_err_rows(_out_f64(got), _paged_ref(sub, lens)) <= TOL["f32"]


def test_noalloc_rejects_partials_larger_than_the_scratch():
    require_gpu()
    B, Hq, Hkv, D, bs, maxb = 12, 64, 8, 128, 16, 300
    lengths = np.full(B, 4096, np.int32)
    d = _paged_inputs(995, B, Hq, Hkv, D, bs, lengths, maxb, extra_blocks=0)
    S = 64                                      # 12 * 64 * 64 * 130 * 4 bytes > 16 MiB
    assert pkv.decode_workspace_size(B, Hq, Hkv, D, maxb * bs, S) > pkv.NOALLOC_SCRATCH_BYTES
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_decode_attention_noalloc(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out,
                                           pool=d["pool"], num_splits=S)
    assert e.value.status == pkv.E_NOMEM
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    pkv.paged_decode_attention_noalloc(d["q"], d["kp"], d["vp"], d["table"], maxb, bs, lengths, out,
                                       pool=d["pool"], num_splits=8)
    assert rel_err_rows(_out_f64(out), _paged_ref(d, lengths)) <= TOL["f32"]
