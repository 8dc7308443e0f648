"""Decode-step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload "paged32k": a paged bf16 KV pool of 65536 blocks x 16 tokens, 32
sequences of exactly 32768 tokens (the pool is full), 32 query / 8 KV heads,
head size 128.  One step is the whole decode hot path for the batch:

  1. in-place append of one K and one V row per sequence at position 32767
     (the last slot of each sequence's last page),
  2. paged decode attention over the 32768 valid tokens (split + merge),
  3. temperature-0.7 sampling of [32, 151936] float32 logits.

Inputs are synthetic (seeded, drawn on the device) and resident in HBM before
the timed region.  Prints one JSON line.  `value` is decode tokens/s of the
whole step (32 tokens per step); `roofline` reports the attention call, the
dominant kernel, against the 8 TB/s HBM peak.  `cpu_baseline` times the CPU
oracle (numpy, float64) on a bounded sample of the same step, on one core and
on every host core (up to 16 processes of one BLAS thread each, run before the
GPU is touched); `value` is the all-core rate, `one_core` the single-core one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode-attn tokens/s + achieved HBM GB/s (% peak), paged bf16 GQA at 32k ctx"
COUNTERS = os.path.join(ROOT, "profiles", "paged_decode_paged32k_counters.json")
KERNEL_SOURCES = ["place_persistent_kv_amd/csrc/decode.hip", "place_persistent_kv_amd/csrc/device_common.h"]

B, HQ, HKV, D, BS, NB, CTX, VOCAB = 32, 32, 8, 128, 16, 65536, 32768, 151936
TEMPERATURE = 0.7


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attention_algorithmic_bytes() -> int:
    """Bytes the attention of one step must move: every valid K and V row once,
    the page-table entries of the valid pages, the queries and the outputs."""
    kv = B * CTX * HKV * D * 2 * 2
    table = B * (CTX // BS) * 4
    q_out = B * HQ * D * 2 * 2
    return kv + table + q_out


def traffic_from_counters():
    """HBM bytes per attention dispatch from committed rocprofv3 counters, if they
    were taken on the current kernel source; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha") != kernel_source_sha():
        return None
    return int(c["hbm_bytes_per_dispatch"])


def run_gpu(steps: int, warmup: int, profile_copy: bool):
    import numpy as np
    import torch

    import place_persistent_kv_amd as pkv
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    maxb = CTX // BS
    k_pool = torch.randn((NB, HKV, BS, D), generator=gen, device=dev, dtype=torch.bfloat16)
    v_pool = torch.randn((NB, HKV, BS, D), generator=gen, device=dev, dtype=torch.bfloat16)
    q = torch.randn((B, HQ, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
    new_k = torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
    new_v = torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
    logits = torch.randn((B, VOCAB), generator=gen, device=dev, dtype=torch.float32) * 3.0
    out = torch.empty((B, HQ, 1, D), device=dev, dtype=torch.bfloat16)
    ids = torch.empty((B,), device=dev, dtype=torch.int64)
    order = synth.permutation(synth.rng(3, 1), NB)
    pool = pkv.Pool(NB, BS, B, maxb, order)
    table = torch.full((B, maxb), -1, device=dev, dtype=torch.int32)
    pool.reserve(range(B), [CTX] * B, table)
    assert pool.free_count() == 0
    ws = torch.empty(pkv.decode_workspace_size(B, HQ, HKV, D, CTX), device=dev, dtype=torch.uint8)
    sws = torch.empty(pkv.sample_workspace_size(B, VOCAB), device=dev, dtype=torch.uint8)
    pos = [CTX - 1] * B
    lens = [CTX] * B
    bk, bv = pkv.bind_writable(k_pool), pkv.bind_writable(v_pool)

    if profile_copy:  # a plain 1 GiB copy: the counter calibration kernel
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # four events per timed step, read after the run: no host synchronisation inside it
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(i, ev):
        if ev:
            ev[0].record(stream)
        pkv.paged_cache_update_kv(pool, k_pool, v_pool, table, new_k, new_v, pos, 1)
        if ev:
            ev[1].record(stream)
        pkv.paged_decode_attention(q, k_pool, v_pool, table, maxb, BS, lens, out, ws, pool=pool)
        if ev:
            ev[2].record(stream)
        pkv.sample(logits, TEMPERATURE, 1000 + i, ids, sws)
        if ev:
            ev[3].record(stream)

    # the same step as a captured HIP graph on the device-driven entry points: one fused K+V append at the
    # device positions, attention over the device lengths, a draw seeded from the device step counter
    pos_dev = torch.full((B,), CTX - 1, dtype=torch.int32, device=dev)
    len_dev = torch.full((B,), CTX, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    step_ctr = torch.zeros(1, dtype=torch.int64, device=dev)

    def step_dev():
        pkv.paged_cache_update_kv_dev(pool, k_pool, v_pool, table, new_k, new_v, pos_dev, 1, status)
        pkv.paged_decode_attention_dev(q, k_pool, v_pool, table, maxb, BS, len_dev, CTX, out, status, ws, pool=pool)
        pkv.sample_dev(logits, TEMPERATURE, 1000, step_ctr, ids, sws)
        pkv.advance(None, 0, step_ctr)

    for i in range(warmup):
        step(i, None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_dev()
    for i in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / steps
    assert int(status.item()) == 0
    free_before = torch.cuda.mem_get_info()[0]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    acc = [sum(ev[k].elapsed_time(ev[k + 1]) for ev in evs) for k in range(3)]
    total_ms = t_start.elapsed_time(t_end)
    alloc_delta = free_before - torch.cuda.mem_get_info()[0]
    bk.close()
    bv.close()
    return {
        "ms_per_step": total_ms / steps,
        "update_us": acc[0] / steps * 1e3,
        "attn_us": acc[1] / steps * 1e3,
        "sample_us": acc[2] / steps * 1e3,
        "graph_step_us": graph_ms * 1e3,
        "device_bytes_allocated_during_steps": int(max(alloc_delta, 0)),
    }


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host's cores
# ---------------------------------------------------------------------------
MAX_CPU_WORKERS = 16      # a host shares its cores among its GPUs: at most 16 oracle processes


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_CPU_WORKERS))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _cpu_loop(budget_s, body):
    """Run body(i) (which returns the units of work it did) under one BLAS thread until budget_s
    elapses; returns (calls, units, seconds)."""
    from threadpoolctl import threadpool_limits
    n, units = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            units += body(n)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return n, units, el


def _job_paged32k_step(worker=0):
    """Whole per-sequence decode steps of the paged32k workload: append one K/V row into the row's 2048
    pages, gather, 32-head attention over 32768 tokens, a T=0.7 draw over 151936 logits.  One token each."""
    import numpy as np
    import synth
    from oracle import attention, cache, numeric, sampling
    maxb = CTX // BS
    order = synth.permutation(synth.rng(3, 7, worker), maxb)
    opool = cache.PagePool(maxb, BS, 1, maxb, order)
    opool.reserve(0, CTX)
    g = synth.rng(3, 8, worker)
    k_pages = synth.f32_to_bf16_bits(synth.normal(g, (maxb, HKV, BS, D)))
    v_pages = synth.f32_to_bf16_bits(synth.normal(g, (maxb, HKV, BS, D)))
    q = synth.f32_to_bf16_bits(synth.normal(g, (HQ, D)))
    new_k = synth.f32_to_bf16_bits(synth.normal(g, (1, HKV, 1, D)))
    new_v = synth.f32_to_bf16_bits(synth.normal(g, (1, HKV, 1, D)))
    logits = synth.normal(g, (1, VOCAB), 3.0)
    G = HQ // HKV

    def body(i):
        cache.paged_cache_update(k_pages, opool.table, new_k, [CTX - 1], 1, BS, opool.held)
        cache.paged_cache_update(v_pages, opool.table, new_v, [CTX - 1], 1, BS, opool.held)
        K = numeric.bf16_to_f64(cache.paged_gather(k_pages, opool.table[0], CTX, BS))
        V = numeric.bf16_to_f64(cache.paged_gather(v_pages, opool.table[0], CTX, BS))
        qh = numeric.bf16_to_f64(q)
        for h in range(HQ):
            attention.attend(qh[h], K[h // G], V[h // G], 1.0 / np.sqrt(D))
        sampling.sample(logits, TEMPERATURE, i)
        return 1
    return body


def _job_decode_rows(L_list, Hq, Hkv, D, seed, worker=0):
    """Oracle attention of whole rows (all query heads) of the given lengths, in turn; one row each."""
    import numpy as np
    import synth
    from oracle import attention
    g = synth.rng(seed, 77, worker)
    Lmax = max(L_list)
    K = synth.normal(g, (Hkv, Lmax, D)).astype(np.float64)
    V = synth.normal(g, (Hkv, Lmax, D)).astype(np.float64)
    q = synth.normal(g, (Hq, D)).astype(np.float64)
    G = Hq // Hkv

    def body(i):
        L = L_list[i % len(L_list)]
        for h in range(Hq):
            attention.attend(q[h], K[h // G, :L], V[h // G, :L], 1.0 / np.sqrt(D))
        return 1
    return body


def _job_int4_rows(worker=0):
    """INT4 rows of the int4 workload (8192 tokens, 32 heads): exact dequantisation + attention; one row each."""
    import numpy as np
    import synth
    from oracle import affine, attention
    from synth import workloads
    spec = workloads.int4()
    Hq, Hkv, Di = spec.Hq, spec.Hkv, spec.D
    rows = [(spec.codes_row(b), spec.params_row(b), spec.v_codes_row(b), spec.v_params_row(b),
             synth.normal(synth.rng(4, 6, b), (Hq, Di)).astype(np.float64)) for b in (worker % spec.B,)]

    def body(i):
        kc, kp, vc, vp, qq = rows[i % len(rows)]
        K = affine.int4_dequant_rows(kc, kp)
        V = affine.int4_dequant_rows(vc, vp)
        for h in range(Hq):
            attention.attend(qq[h], K[h // (Hq // Hkv)], V[h // (Hq // Hkv)], 1 / np.sqrt(Di))
        return 1
    return body


def _job_chunk_queries(worker=0):
    """Causal chunk queries of a median Qwen-shaped row (16 heads each); flops of each query."""
    import numpy as np
    import synth as sy
    from oracle import attention
    from synth import workloads
    w = workloads.qwen()
    C, Hq, Hkv, Dq = w["chunk"], w["Hq"], w["Hkv"], w["D"]
    g = sy.rng(5, 78, worker)
    Lr = int(np.median(w["lengths"])) + C
    K = sy.normal(g, (Hkv, Lr, Dq)).astype(np.float64)
    V = sy.normal(g, (Hkv, Lr, Dq)).astype(np.float64)
    qq = sy.normal(g, (Hq, Dq)).astype(np.float64)
    G = Hq // Hkv

    def body(i):
        t = (i * 37) % C
        last = Lr - C + t
        for h in range(Hq):
            attention.attend(qq[h], K[h // G, :last + 1], V[h // G, :last + 1], 1 / np.sqrt(Dq))
        return 4.0 * Hq * Dq * (last + 1)
    return body


def _job_sample_rows(worker=0):
    """T=0.7 draws over one row of [*, 151936] N(0, 3) logits; one token each."""
    from oracle import sampling
    from synth import workloads
    w = workloads.qwen()
    x = workloads.logits(5 + worker, 4, w["vocab"])

    def body(i):
        sampling.sample(x[i % 4:i % 4 + 1], 0.7, i)
        return 1
    return body


def _job_mixed_rows(worker=0):
    """Oracle attention over one 32768-token row of the mixed32k workload's pages (decoded exactly); one row."""
    import numpy as np
    import synth
    from oracle import mixed as om
    from synth import workloads
    w = workloads.mixed32k()
    g = synth.rng(w.seed, 9, worker)
    opool = om.MixedPool(w.maxb, w.Hkv, w.bs, w.D)
    local = np.arange(w.maxb, dtype=np.int32)[None]
    p = 0
    while p < w.L:                  # one row of the workload, outside the timed loop
        n = w.threshold if p < w.threshold else min(4096, w.L - p)
        kf, vf = (w.early if p < w.threshold else w.late)
        kb = synth.f32_to_bf16_bits(synth.normal(g, (1, w.Hkv, n, w.D), w.k_sigma))
        vb = synth.f32_to_bf16_bits(synth.normal(g, (1, w.Hkv, n, w.D), w.v_sigma))
        opool.append(local, kb, vb, [p], n, om.Format(*kf), om.Format(*vf))
        p += n
    qh = synth.normal(g, (1, w.Hq, w.D)).astype(np.float64)

    def body(i):
        om.decode_attention(opool, qh, local, [w.L])
        return 1
    return body


def _job_tiny_steps(worker=0):
    """The tiny fixture's stateful loop: prompt + 15 appends into capacity 16, attention after each; one
    step each (a 16-step run per 16 calls)."""
    import numpy as np
    from oracle import attention, cache
    from synth import workloads
    w = workloads.tiny()
    cap = w["capacity"]
    q, k, v = (w[x].astype(np.float64) for x in ("q", "k", "v"))
    kc = np.zeros((1, 1, cap, 4))
    vc = np.zeros((1, 1, cap, 4))

    def body(i):
        t = i % cap
        cache.cache_update(kc, k[t].reshape(1, 1, 1, 4), [t], 1)
        cache.cache_update(vc, v[t].reshape(1, 1, 1, 4), [t], 1)
        attention.attend(q[t, 0], kc[0, 0, :t + 1], vc[0, 0, :t + 1], 0.5)
        return 1
    return body


_CPU_JOBS = {"paged32k_step": _job_paged32k_step, "decode_rows": _job_decode_rows, "int4_rows": _job_int4_rows,
             "chunk_queries": _job_chunk_queries, "sample_rows": _job_sample_rows, "mixed_rows": _job_mixed_rows,
             "tiny_steps": _job_tiny_steps}


def _cpu_worker(name, kw, worker, budget_s, barrier):
    """One oracle process: build the job, wait until every worker has built it, run it for budget_s."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    body = _CPU_JOBS[name](worker=worker, **kw)
    body(0)
    barrier.wait()
    _, units, el = _cpu_loop(budget_s, body)
    return units, el


def oracle_baseline(name, kw, unit, what, scale=1.0, budget_one=10.0, budget_all=8.0, all_cores=True):
    """The oracle's rate on one core and on every host core (one process per core, one BLAS thread each,
    running together).  `scale` converts job units to `unit`.  The all-core figure is `value`."""
    import concurrent.futures as cf
    import multiprocessing as mp
    body = _CPU_JOBS[name](**kw)
    body(0)
    n1, u1, el1 = _cpu_loop(budget_one, body)
    one = {"value": round(u1 / el1 * scale, 6), "cores": 1, "sample": f"{n1} calls in {el1:.1f} s"}
    res = {"value": one["value"], "unit": unit, "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
           "host_cpus": os.cpu_count(), "sample": f"{what}; 1 core: {n1} calls in {el1:.1f} s", "one_core": one}
    cores = host_cores()
    if not all_cores or cores < 2:
        return res
    ctx = mp.get_context("spawn")         # fresh interpreters: nothing of this process is inherited
    with ctx.Manager() as mgr:
        barrier = mgr.Barrier(cores)
        with cf.ProcessPoolExecutor(cores, mp_context=ctx) as ex:
            futs = [ex.submit(_cpu_worker, name, kw, wk, budget_all, barrier) for wk in range(cores)]
            out = [f.result() for f in futs]
    rate = sum(u / el for u, el in out) * scale
    res.update({"value": round(rate, 6), "cores": cores,
                "sample": f"{what}; {cores} processes together for {budget_all:.0f} s each "
                          f"({sum(u for u, _ in out):.0f} units), one BLAS thread each; "
                          f"1 core: {n1} calls in {el1:.1f} s"})
    return res


# ---------------------------------------------------------------------------
# Other rows of the decode path, one JSON line each (python bench.py --workload X)
# ---------------------------------------------------------------------------
def _timed(fn, steps, warmup, stream):
    """Average duration (us) of fn() over `steps` back-to-back calls: one pair of
    HIP events on the launch stream brackets all of them (a pair per call adds
    the event packets' own latency to every short call), with a device
    synchronisation before and after."""
    import torch
    for i in range(warmup):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def _line(metric, value, unit, steps, warmup, us, dtype, config, roofline, cpu=None, **extra):
    r = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
         "ms_per_step": round(us / 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
         "dtype": dtype, "data": "synthetic", "config": config, "roofline": roofline}
    r.update(extra)
    if cpu is not None:
        r["cpu_baseline"] = cpu
    return r


def _hbm_roofline(nbytes, us):
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}


def bench_contig(steps, warmup, cpu):
    """Contiguous bf16 cache [8, 8, 4096, 128]: append one K/V row + decode attention per step (one fused call;
    the two-call step is reported beside it).
    Six cache replicas are rotated so that each step reads K/V from HBM, not from the 256 MB MALL."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.contig()
    Bc, Hq, Hkv, Dc, cap, S = w["B"], w["Hq"], w["Hkv"], w["D"], w["cap"], w["steps"]
    L0 = w["lengths"].astype(np.int64)
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    R = 6
    kc = [torch.randn((Bc, Hkv, cap, Dc), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(R)]
    vc = [torch.randn((Bc, Hkv, cap, Dc), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(R)]
    q = torch.randn((Bc, Hq, 1, Dc), generator=gen, device=dev, dtype=torch.bfloat16)
    nk = torch.randn((Bc, Hkv, 1, Dc), generator=gen, device=dev, dtype=torch.bfloat16)
    nv = torch.randn((Bc, Hkv, 1, Dc), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((Bc, Hq, 1, Dc), device=dev, dtype=torch.bfloat16)
    ws = torch.empty(pkv.decode_workspace_size(Bc, Hq, Hkv, Dc, cap), device=dev, dtype=torch.uint8)
    binds = [pkv.bind_writable(t) for t in kc + vc]
    stream = torch.cuda.current_stream()

    def step(i, rot=True):          # the append fused into the attention launch
        r = i % R if rot else 0
        pos = (L0 + i % S).tolist()
        pkv.decode_step(kc[r], vc[r], nk, nv, pos, 1, q, out, ws)

    def step_two_calls(i):          # the K+V append and the attention as two calls
        r = i % R
        pos = (L0 + i % S).tolist()
        pkv.cache_update_kv(kc[r], vc[r], nk, nv, pos, 1)
        pkv.decode_attention(q, kc[r], vc[r], [p + 1 for p in pos], out, ws)

    def attn_only(i, rot=True):
        r = i % R if rot else 0
        pkv.decode_attention(q, kc[r], vc[r], (L0 + i % S + 1).tolist(), out, ws)

    us_step = _timed(step, steps, warmup, stream)
    us_two = _timed(step_two_calls, steps, warmup, stream)
    us_attn = _timed(attn_only, steps, warmup, stream)
    us_warm = _timed(lambda i: attn_only(i, False), steps, warmup, stream)
    # captured step per replica: the append fused into the attention at the replica's device positions, then
    # the positions + 1
    lens = [torch.from_numpy(L0.astype(np.int32)).to(dev) for _ in range(R)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    graphs = []
    for r in range(R):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            pkv.decode_step_dev(kc[r], vc[r], nk, nv, lens[r], 1, q, cap, out, status, ws)
            pkv.advance(lens[r], 1)
        graphs.append(gr)
    torch.cuda.synchronize()
    for r in range(R):
        lens[r].copy_(torch.from_numpy(L0.astype(np.int32)))
    us_graph = _timed(lambda i: graphs[i % R].replay(), steps, min(warmup, R), stream)
    assert int(status.item()) == 0
    for bnd in binds:
        bnd.close()
    mean_L = float(np.mean(L0 + (np.arange(steps) % S)[:, None] + 1))
    nbytes = int(mean_L * Bc * Hkv * Dc * 2 * 2 + Bc * Hq * Dc * 2 * 2)
    cpu_res = cpu
    return _line("decode tokens/s, contiguous bf16 GQA cache", Bc / (us_step * 1e-6), "tokens/s", steps, warmup,
                 us_step, "bf16", {"workload": "contig", "batch": Bc, "capacity": cap, "q_heads": Hq, "kv_heads": Hkv,
                                   "head_dim": Dc, "replicas_rotated": R},
                 _hbm_roofline(nbytes, us_attn), cpu_res, attn_us=round(us_attn, 2),
                 attn_us_warm=round(us_warm, 2), attn_algorithmic_bytes=nbytes, step_two_call_us=round(us_two, 2),
                 graph_step_us=round(us_graph, 2), graph_tokens_per_s=round(Bc / (us_graph * 1e-6), 1))


def bench_paged(steps, warmup, cpu):
    """Paged bf16 pool of 65536 x 16 tokens, 64 rows with lognormal(8, 1) lengths in [16, 32768]."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    spec = workloads.paged()
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    Bp, Hq, Hkv, Dp, bs, NBp, maxb = spec.B, spec.Hq, spec.Hkv, spec.D, spec.bs, spec.NB, spec.maxb
    L = spec.lengths.astype(np.int64)
    kd = torch.randn((NBp, Hkv, bs, Dp), generator=gen, device=dev, dtype=torch.bfloat16)
    vd = torch.randn((NBp, Hkv, bs, Dp), generator=gen, device=dev, dtype=torch.bfloat16)
    q = torch.randn((Bp, Hq, Dp), generator=gen, device=dev, dtype=torch.bfloat16)
    nk = torch.randn((Bp, Hkv, 1, Dp), generator=gen, device=dev, dtype=torch.bfloat16)
    nv = torch.randn((Bp, Hkv, 1, Dp), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((Bp, Hq, Dp), device=dev, dtype=torch.bfloat16)
    pool = pkv.Pool(NBp, bs, Bp, maxb, spec.order)
    table = torch.full((Bp, maxb), -1, device=dev, dtype=torch.int32)
    pool.reserve(range(Bp), L.tolist(), table)
    ws = torch.empty(pkv.decode_workspace_size(Bp, Hq, Hkv, Dp, int(L.max())), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    bk, bv = pkv.bind_writable(kd), pkv.bind_writable(vd)
    pos = (L - 1).tolist()

    def step(i):
        pkv.paged_cache_update_kv(pool, kd, vd, table, nk, nv, pos, 1)
        pkv.paged_decode_attention(q, kd, vd, table, maxb, bs, L.tolist(), out, ws, pool=pool)

    us_step = _timed(step, steps, warmup, stream)
    us_attn = _timed(lambda i: pkv.paged_decode_attention(q, kd, vd, table, maxb, bs, L.tolist(), out, ws,
                                                          pool=pool), steps, warmup, stream)
    bk.close()
    bv.close()
    nbytes = int(L.sum() * Hkv * Dp * 4 + sum(-(-int(x) // bs) for x in L) * 4 + Bp * Hq * Dp * 4)
    cpu_res = cpu
    return _line("decode tokens/s, paged bf16 GQA, lognormal contexts", Bp / (us_step * 1e-6), "tokens/s", steps,
                 warmup, us_step, "bf16", {"workload": "paged", "batch": Bp, "num_blocks": NBp, "block_size": bs,
                                           "q_heads": Hq, "kv_heads": Hkv, "head_dim": Dp,
                                           "mean_ctx": round(float(L.mean()), 1), "max_ctx": int(L.max())},
                 _hbm_roofline(nbytes, us_attn), cpu_res, attn_us=round(us_attn, 2), attn_algorithmic_bytes=nbytes)


def bench_int4(steps, warmup, cpu):
    """INT4 paged pool (16384 x 16 tokens), 32 rows x 8192 tokens: quantise-on-append + INT4 decode.
    Three pool replicas are rotated (each ~288 MB, the MALL is 256 MB)."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    spec = workloads.int4()
    dev = "cuda:0"
    Bi, Hq, Hkv, Di, bs, NBi, maxb = spec.B, spec.Hq, spec.Hkv, spec.D, spec.bs, spec.NB, spec.maxb
    L = spec.lengths.astype(np.int64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    R = 3

    def codes():
        return torch.randint(0, 256, (NBi, Hkv, bs, Di // 2), generator=gen, device=dev, dtype=torch.uint8)

    def params():
        p = torch.empty((NBi, Hkv, bs, Di // 32, 2), device=dev, dtype=torch.float16)
        p[..., 0].uniform_(0.01, 0.1, generator=gen)
        p[..., 1].copy_(torch.randint(0, 16, p[..., 1].shape, generator=gen, device=dev).to(torch.float16))
        return p
    kc, kp, vc, vp = [codes() for _ in range(R)], [params() for _ in range(R)], [codes() for _ in range(R)], \
        [params() for _ in range(R)]
    q = torch.randn((Bi, Hq, Di), generator=gen, device=dev, dtype=torch.float32)
    newv = torch.randn((Bi, Hkv, 1, Di), generator=gen, device=dev, dtype=torch.float32) * 0.3
    out = torch.empty((Bi, Hq, Di), device=dev, dtype=torch.float32)
    pool = pkv.Pool(NBi, bs, Bi, maxb, spec.order)
    table = torch.full((Bi, maxb), -1, device=dev, dtype=torch.int32)
    pool.reserve(range(Bi), L.tolist(), table)
    ws = torch.empty(pkv.decode_workspace_size(Bi, Hq, Hkv, Di, int(L.max())), device=dev, dtype=torch.uint8)
    binds = [pkv.bind_writable(t) for t in kc + kp + vc + vp]
    stream = torch.cuda.current_stream()
    s_bits = int(np.float16(0.05).view(np.uint16))
    z_bits = int(np.float16(8.0).view(np.uint16))
    pos = (L - 1).tolist()

    def attn(i):
        r = i % R
        pkv.paged_decode_attention_int4(q, kc[r], kp[r], vc[r], vp[r], table, maxb, bs, L.tolist(), out, ws,
                                        pool=pool)

    def step(i):
        r = i % R
        pkv.paged_cache_update_int4(pool, kc[r], kp[r], table, newv, s_bits, z_bits, pos, 1)
        pkv.paged_cache_update_int4(pool, vc[r], vp[r], table, newv, s_bits, z_bits, pos, 1)
        attn(i)

    us_step = _timed(step, steps, warmup, stream)
    us_attn = _timed(attn, steps, warmup, stream)
    for bnd in binds:
        bnd.close()
    nbytes = int(L.sum() * Hkv * 160 + Bi * (int(L[0]) // bs) * 4 + Bi * Hq * Di * 4 * 2)
    cpu_res = cpu
    return _line("decode tokens/s, paged INT4 blockwise-affine GQA", Bi / (us_step * 1e-6), "tokens/s", steps, warmup,
                 us_step, "int4/f32", {"workload": "int4", "batch": Bi, "ctx": int(L[0]), "num_blocks": NBi,
                                       "block_size": bs, "q_heads": Hq, "kv_heads": Hkv, "head_dim": Di,
                                       "replicas_rotated": R},
                 _hbm_roofline(nbytes, us_attn), cpu_res, attn_us=round(us_attn, 2), attn_algorithmic_bytes=nbytes)


def _qwen_pools(w, extra, layers, gen):
    import torch
    import place_persistent_kv_amd as pkv
    dev = "cuda:0"
    L = w["lengths"]
    bs = w["bs"]
    NBq = int(sum(-(-(int(x) + extra) // bs) for x in L))
    base_k = torch.randn((NBq, w["Hkv"], bs, w["D"]), generator=gen, device=dev, dtype=torch.bfloat16)
    base_v = torch.randn((NBq, w["Hkv"], bs, w["D"]), generator=gen, device=dev, dtype=torch.bfloat16)
    ks, vs = [base_k], [base_v]
    for _ in range(layers - 1):
        ks.append(base_k.clone())
        vs.append(base_v.clone())
    import synth
    pool = pkv.Pool(NBq, bs, w["B"], w["maxb"], synth.permutation(synth.rng(w["seed"], 1), NBq))
    table = torch.full((w["B"], w["maxb"]), -1, device=dev, dtype=torch.int32)
    pool.reserve(range(w["B"]), [int(x) + extra for x in L], table)
    return ks, vs, pool, table, NBq


def bench_qwen_decode(steps, warmup, cpu, layers=28):
    """28 layers of paged bf16 caches (one shared page table), 128 rows, 16/8 heads, ctx U[1024, 16384]:
    per layer an in-place K/V append and paged decode attention."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.qwen()
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    ks, vs, pool, table, NBq = _qwen_pools(w, 1, layers, gen)
    Bq, Hq, Hkv, Dq, bs, maxb = w["B"], w["Hq"], w["Hkv"], w["D"], w["bs"], w["maxb"]
    L = w["lengths"].astype(np.int64) + 1
    q = torch.randn((Bq, Hq, Dq), generator=gen, device=dev, dtype=torch.bfloat16)
    nk = torch.randn((Bq, Hkv, 1, Dq), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((Bq, Hq, Dq), device=dev, dtype=torch.bfloat16)
    ws = torch.empty(pkv.decode_workspace_size(Bq, Hq, Hkv, Dq, int(L.max())), device=dev, dtype=torch.uint8)
    binds = [pkv.bind_writable(t) for t in ks + vs]
    stream = torch.cuda.current_stream()
    pos = (L - 1).tolist()
    lens = L.tolist()

    def step(i):
        for layer in range(layers):
            pkv.paged_cache_update_kv(pool, ks[layer], vs[layer], table, nk, nk, pos, 1)
            pkv.paged_decode_attention(q, ks[layer], vs[layer], table, maxb, bs, lens, out, ws, pool=pool)

    us_step = _timed(step, steps, warmup, stream)
    us_attn = _timed(lambda i: pkv.paged_decode_attention(q, ks[i % layers], vs[i % layers], table, maxb, bs, lens,
                                                          out, ws, pool=pool), steps * 4, warmup, stream)
    # the 28-layer step as one captured graph on the device-driven calls (positions and lengths on the device;
    # they stay at the same token, as the eager step's do).  Device lengths are planned from their bound (the
    # longest row), so the split count is given: the number the host plan gives the longest rows.
    graph_splits = -(-int(L.max()) // max(384, -(-(-(-int(L.sum()) * Hkv // 1024)) // 64) * 64))
    pos_dev = torch.from_numpy((L - 1).astype(np.int32)).to(dev)
    len_dev = torch.from_numpy(L.astype(np.int32)).to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for layer in range(layers):
            pkv.paged_cache_update_kv_dev(pool, ks[layer], vs[layer], table, nk, nk, pos_dev, 1, status)
            pkv.paged_decode_attention_dev(q, ks[layer], vs[layer], table, maxb, bs, len_dev, int(L.max()), out,
                                           status, ws, pool=pool, num_splits=graph_splits)
    torch.cuda.synchronize()
    us_graph = _timed(lambda i: gr.replay(), steps, warmup, stream)
    assert int(status.item()) == 0
    for bnd in binds:
        bnd.close()
    nbytes = int(L.sum() * Hkv * Dq * 4 + sum(-(-int(x) // bs) for x in L) * 4 + Bq * Hq * Dq * 4)
    cpu_res = cpu
    return _line("decode tokens/s, Qwen-shaped 28-layer paged bf16 step", Bq / (us_step * 1e-6), "tokens/s", steps,
                 warmup, us_step, "bf16", {"workload": "qwen-decode", "layers": layers, "batch": Bq, "q_heads": Hq,
                                           "kv_heads": Hkv, "head_dim": Dq, "block_size": bs,
                                           "blocks_per_layer": NBq, "mean_ctx": round(float(L.mean()), 1)},
                 _hbm_roofline(nbytes, us_attn), cpu_res, attn_us_per_layer=round(us_attn, 2),
                 attn_algorithmic_bytes_per_layer=nbytes, graph_step_us=round(us_graph, 2),
                 graph_tokens_per_s=round(Bq / (us_graph * 1e-6), 1))


def bench_qwen_chunk(steps, warmup, cpu, constant=None):
    """One layer: a 512-token chunk appended in place to 128 paged rows (prefix U[1024, 16384]) and the
    causal chunk attention on the bf16 matrix cores.  `constant` (a float) replaces every input value with
    it: the calibration of the data-dependent clock only."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.qwen()
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    C = w["chunk"]
    ks, vs, pool, table, NBq = _qwen_pools(w, C, 1, gen)
    Bq, Hq, Hkv, Dq, bs, maxb = w["B"], w["Hq"], w["Hkv"], w["D"], w["bs"], w["maxb"]
    P0 = w["lengths"].astype(np.int64)
    q = torch.randn((Bq, Hq, C, Dq), generator=gen, device=dev, dtype=torch.bfloat16)
    nk = torch.randn((Bq, Hkv, C, Dq), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((Bq, Hq, C, Dq), device=dev, dtype=torch.bfloat16)
    if constant is not None:
        for t in ks + vs + [q, nk]:
            t.fill_(constant)
    binds = [pkv.bind_writable(t) for t in ks + vs]
    stream = torch.cuda.current_stream()
    p0 = P0.tolist()

    def attn(i):
        pkv.chunk_attention(q, ks[0], vs[0], table, maxb, bs, p0, out, pool=pool)

    def step(i):
        pkv.paged_cache_update_kv(pool, ks[0], vs[0], table, nk, nk, p0, C)
        attn(i)

    us_step = _timed(step, steps, warmup, stream)
    us_attn = _timed(attn, steps, warmup, stream)
    for bnd in binds:
        bnd.close()
    flops = 4.0 * Hq * Dq * float(np.sum(C * P0 + C * (C + 1) / 2))
    tflops = flops / (us_attn * 1e-6) / 1e12
    peak = 2500.0
    cpu_res = cpu
    return _line("causal chunk attention TFLOP/s (512-token chunk, MFMA bf16)", tflops, "TFLOP/s", steps, warmup,
                 us_step, "bf16", {"workload": "qwen-chunk", "batch": Bq, "chunk": C, "q_heads": Hq, "kv_heads": Hkv,
                                   "head_dim": Dq, "mean_prefix": round(float(P0.mean()), 1)},
                 {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                  "frac": round(tflops / peak, 4), "traffic": None}, cpu_res,
                 attn_us=round(us_attn, 2), step_us=round(us_step, 2), attn_flops=flops,
                 chunk_tokens_per_s=round(Bq * C / (us_step * 1e-6), 1))


def bench_qwen_chunk_1row(steps, warmup, cpu):
    """One request of the qwen-chunk shape: a 512-token chunk after a 16384-token prefix.  Its launch has
    one workgroup per (K/V head, 128-token query tile), 32 in all, so the library splits every workgroup's
    key range and merges the parts; the unsplit launch and a sweep of split counts are reported beside it."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.qwen(B=1, lo=16384, hi=16384)
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    C = w["chunk"]
    ks, vs, pool, table, NBq = _qwen_pools(w, C, 1, gen)
    Bq, Hq, Hkv, Dq, bs, maxb = w["B"], w["Hq"], w["Hkv"], w["D"], w["bs"], w["maxb"]
    P0 = w["lengths"].astype(np.int64)
    q = torch.randn((Bq, Hq, C, Dq), generator=gen, device=dev, dtype=torch.bfloat16)
    nk = torch.randn((Bq, Hkv, C, Dq), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((Bq, Hq, C, Dq), device=dev, dtype=torch.bfloat16)
    binds = [pkv.bind_writable(t) for t in ks + vs]
    stream = torch.cuda.current_stream()
    p0 = P0.tolist()
    sweep = [1, 2, 4, 8, 16]
    ws = torch.empty(max(pkv.chunk_workspace_size(Bq, Hq, Hkv, C, S) for S in sweep + [0]), dtype=torch.uint8,
                     device=dev)

    def attn(S):
        return lambda i: pkv.chunk_attention(q, ks[0], vs[0], table, maxb, bs, p0, out, pool=pool, workspace=ws,
                                             num_splits=S)

    def step(i):
        pkv.paged_cache_update_kv(pool, ks[0], vs[0], table, nk, nk, p0, C)
        attn(0)(i)

    us_step = _timed(step, steps, warmup, stream)
    us_auto = _timed(attn(0), steps, warmup, stream)
    us_sweep = {str(S): round(_timed(attn(S), steps, warmup, stream), 2) for S in sweep}
    for bnd in binds:
        bnd.close()
    flops = 4.0 * Hq * Dq * float(np.sum(C * P0 + C * (C + 1) / 2))
    tflops = flops / (us_auto * 1e-6) / 1e12
    peak = 2500.0
    return _line("causal chunk attention TFLOP/s (one request, 512-token chunk, MFMA bf16)", tflops, "TFLOP/s",
                 steps, warmup, us_step, "bf16",
                 {"workload": "qwen-chunk-1row", "batch": Bq, "chunk": C, "q_heads": Hq, "kv_heads": Hkv,
                  "head_dim": Dq, "prefix": int(P0[0])},
                 {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                  "frac": round(tflops / peak, 4), "traffic": None}, cpu,
                 attn_us=round(us_auto, 2), step_us=round(us_step, 2), attn_flops=flops,
                 attn_us_by_splits=us_sweep)


def bench_mfma_ceiling(steps, warmup, cpu):
    """What the matrix cores deliver on this board for the data the benchmarks use.  Dense bf16 MFMA work
    is limited by power before the published rate is reached, and the limit depends on the operands'
    bit activity: a plain 8192^3 bf16 GEMM (torch.matmul, the vendor library) is timed on N(0, 1)
    operands and on constant ones, and so is the Qwen-shaped chunk attention launch."""
    import torch
    n = 8192
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    a = torch.randn((n, n), generator=gen, device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), generator=gen, device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    flops = 2.0 * n ** 3
    us_normal = _timed(lambda i: torch.matmul(a, b, out=c), steps, warmup, stream)
    a.fill_(0.0115)
    b.fill_(0.0115)
    us_const = _timed(lambda i: torch.matmul(a, b, out=c), steps, warmup, stream)
    del a, b, c
    torch.cuda.empty_cache()
    chunk_normal = bench_qwen_chunk(steps, warmup, None)
    chunk_const = bench_qwen_chunk(steps, warmup, None, constant=0.0115)
    tf = flops / (us_normal * 1e-6) / 1e12
    return _line("bf16 dense GEMM TFLOP/s (8192^3, torch.matmul) on N(0, 1) operands", tf, "TFLOP/s", steps,
                 warmup, us_normal, "bf16", {"workload": "mfma-ceiling", "m": n, "n": n, "k": n},
                 {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                  "frac": round(tf / 2500.0, 4), "traffic": None}, cpu,
                 gemm_constant_tflops=round(flops / (us_const * 1e-6) / 1e12, 1),
                 chunk_normal_tflops=chunk_normal["value"], chunk_constant_tflops=chunk_const["value"])


def bench_sample(steps, warmup, cpu):
    """Greedy and T = 0.7 sampling of [128, 151936] float32 logits; four logit replicas are rotated
    (78 MB each) so the reads come from HBM."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.qwen()
    dev = "cuda:0"
    Bs, Vs = w["B"], w["vocab"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    R = 4
    lg = [torch.randn((Bs, Vs), generator=gen, device=dev) * 3.0 for _ in range(R)]
    ids = torch.empty((Bs,), device=dev, dtype=torch.int64)
    sws = torch.empty(pkv.sample_workspace_size(Bs, Vs), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    us_greedy = _timed(lambda i: pkv.sample(lg[i % R], 0.0, i, ids, sws), steps, warmup, stream)
    us_temp = _timed(lambda i: pkv.sample(lg[i % R], 0.7, i, ids, sws), steps, warmup, stream)
    nbytes = Bs * Vs * 4
    cpu_res = cpu
    return _line("sampling tokens/s, T=0.7 over [128, 151936] logits", Bs / (us_temp * 1e-6), "tokens/s", steps,
                 warmup, us_temp, "f32", {"workload": "sample", "batch": Bs, "vocab": Vs, "replicas_rotated": R},
                 _hbm_roofline(nbytes, us_temp), cpu_res, greedy_us=round(us_greedy, 2),
                 greedy_roofline=_hbm_roofline(nbytes, us_greedy), temperature_us=round(us_temp, 2))


def bench_window(steps, warmup, cpu):
    """paged32k pages (32 rows x 32768 tokens, full pool) with a left window of 4095: each query sees its
    last 4096 tokens, and the pages before the window are not read."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    import synth
    W = 4095
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    maxb = CTX // BS
    kp = torch.randn((NB, HKV, BS, D), generator=gen, device=dev, dtype=torch.bfloat16)
    vp = torch.randn((NB, HKV, BS, D), generator=gen, device=dev, dtype=torch.bfloat16)
    q = torch.randn((B, HQ, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((B, HQ, 1, D), device=dev, dtype=torch.bfloat16)
    pool = pkv.Pool(NB, BS, B, maxb, synth.permutation(synth.rng(3, 1), NB))
    table = torch.full((B, maxb), -1, device=dev, dtype=torch.int32)
    pool.reserve(range(B), [CTX] * B, table)
    ws = torch.empty(pkv.decode_workspace_size(B, HQ, HKV, D, CTX), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    us = _timed(lambda i: pkv.paged_decode_attention(q, kp, vp, table, maxb, BS, [CTX] * B, out, ws, pool=pool,
                                                     left_window=W), steps, warmup, stream)
    visible = W + 1
    nbytes = B * visible * HKV * D * 2 * 2 + B * (visible // BS) * 4 + B * HQ * D * 2 * 2
    cpu_res = cpu
    return _line("decode tokens/s, paged bf16 GQA, 32k context with a 4096-token left window", B / (us * 1e-6),
                 "tokens/s", steps, warmup, us, "bf16",
                 {"workload": "window", "batch": B, "ctx": CTX, "left_window": W, "q_heads": HQ, "kv_heads": HKV,
                  "head_dim": D, "block_size": BS, "num_blocks": NB},
                 _hbm_roofline(nbytes, us), cpu_res, attn_us=round(us, 2), attn_algorithmic_bytes=nbytes)


def bench_mixed(steps, warmup, cpu):
    """Mixed-format pages at the paged32k shapes (32 rows x 32768 tokens, a full 65536-page pool), appended
    through the library with the pages' length-threshold selector: the first 1024 tokens of a row in BF16
    pages, the rest with INT8 keys (0.01, 0) and UINT4 values (0.25, 8).  Times the decode attention."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.mixed32k()
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    kp = torch.zeros((w.NB, w.Hkv, w.bs, w.D), device=dev, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    pd = pkv.mixed_page_desc(w.NB, dev)
    pool = pkv.Pool(w.NB, w.bs, w.B, w.maxb, w.order)
    table = torch.full((w.B, w.maxb), -1, device=dev, dtype=torch.int32)
    pool.reserve(range(w.B), [w.L] * w.B, table)
    fm = lambda t: pkv.page_format(*t)
    select = pkv.LengthThresholdSelector(w.threshold, (fm(w.early[0]), fm(w.early[1])),
                                         (fm(w.late[0]), fm(w.late[1])))
    binds = [pkv.bind_writable(t) for t in (kp, vp, pd)]
    pos = 0
    while pos < w.L:
        n = w.threshold if pos < w.threshold else min(2048, w.L - pos)
        kv = (torch.randn((w.B, w.Hkv, n, w.D), generator=gen, device=dev) * w.k_sigma).to(torch.bfloat16)
        vv = (torch.randn((w.B, w.Hkv, n, w.D), generator=gen, device=dev) * w.v_sigma).to(torch.bfloat16)
        kf, vf = select(pos)
        pkv.mixed_cache_update(pool, kp, vp, pd, table, kv, vv, [pos] * w.B, n, kf, vf)
        pos += n
    del kv, vv
    q = torch.randn((w.B, w.Hq, w.D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.D), device=dev, dtype=torch.bfloat16)
    ws = torch.empty(pkv.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.L), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    lens = [w.L] * w.B
    us = _timed(lambda i: pkv.paged_decode_attention_mixed(q, kp, vp, pd, table, w.maxb, w.bs, lens, out, ws,
                                                           pool=pool), steps, warmup, stream)
    for b in binds:
        b.close()
    early, late = w.threshold, w.L - w.threshold
    row_bytes = w.D * 2 * 2 * early + (w.D * 1 + w.D // 2) * late       # K + V bytes of one (row, kv head)
    nbytes = w.B * w.Hkv * row_bytes + w.B * w.maxb * (4 + 16) + w.B * w.Hq * w.D * 2 * 2
    cpu_res = cpu
    return _line("decode tokens/s, paged GQA over mixed-format pages (BF16 prefix, INT8 K / UINT4 V), 32k context",
                 w.B / (us * 1e-6), "tokens/s", steps, warmup, us, "bf16/int8/uint4",
                 {"workload": "mixed", "batch": w.B, "ctx": w.L, "q_heads": w.Hq, "kv_heads": w.Hkv,
                  "head_dim": w.D, "block_size": w.bs, "num_blocks": w.NB, "dense_prefix": w.threshold,
                  "k_late": list(w.late[0]), "v_late": list(w.late[1])},
                 _hbm_roofline(nbytes, us), cpu_res, attn_us=round(us, 2), attn_algorithmic_bytes=nbytes)


def bench_generate(steps, warmup, cpu, layers=28, new_tokens=8):
    """The generation loop (pkv.generate) over the 28-layer Qwen-shaped paged caches: 128 rows with cached
    prefixes of U[1024, 16384] tokens, a one-token prompt, `new_tokens` iterations.  The model is synthetic:
    per layer q, k, v are embedding-table rows of the input token (random bf16 tables), each layer appends
    k, v in place and runs paged decode attention, and the logits are the last layer's output times a random
    bf16 LM head [2048, 151936]; EOS is the last vocabulary id.  `steps` timed generate calls."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.qwen()
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    Bq, Hq, Hkv, Dq, bs, maxb, V = w["B"], w["Hq"], w["Hkv"], w["D"], w["bs"], w["maxb"], w["vocab"]
    runs = warmup + steps
    ks, vs, pool, table, NBq = _qwen_pools(w, runs * new_tokens, layers, gen)
    emb_q = torch.randn((V, Hq, Dq), generator=gen, device=dev).to(torch.bfloat16)
    emb_k = torch.randn((V, Hkv, 1, Dq), generator=gen, device=dev).to(torch.bfloat16)
    emb_v = torch.randn((V, Hkv, 1, Dq), generator=gen, device=dev).to(torch.bfloat16)
    head = (torch.randn((Hq * Dq, V), generator=gen, device=dev) * 0.05).to(torch.bfloat16)
    out = torch.empty((Bq, Hq, Dq), device=dev, dtype=torch.bfloat16)
    L0 = w["lengths"].astype(np.int64)
    ws = torch.empty(pkv.decode_workspace_size(Bq, Hq, Hkv, Dq, int(L0.max()) + runs * new_tokens), device=dev,
                     dtype=torch.uint8)
    binds = [pkv.bind_writable(t) for t in ks + vs]
    state = {"L": L0.copy()}

    def forward(step, ids):
        tok = (ids[:, -1] if ids.dim() == 2 else ids).contiguous()
        q = emb_q.index_select(0, tok)
        k = emb_k.index_select(0, tok)
        v = emb_v.index_select(0, tok)
        pos = state["L"].tolist()
        lens = (state["L"] + 1).tolist()
        for layer in range(layers):
            pkv.paged_cache_update_kv(pool, ks[layer], vs[layer], table, k, v, pos, 1)
            pkv.paged_decode_attention(q, ks[layer], vs[layer], table, maxb, bs, lens, out, ws, pool=pool)
        state["L"] += 1
        return out.reshape(Bq, Hq * Dq) @ head

    prompt = torch.from_numpy(np.arange(Bq, dtype=np.int64)[:, None] * 7 % V).to(dev)
    for i in range(warmup):
        pkv.generate(forward, prompt, new_tokens, 0.7, 100 + i, V - 1)
    torch.cuda.synchronize()
    mean_L = float(state["L"].mean())
    t0 = time.perf_counter()
    produced = 0
    for i in range(steps):
        res = pkv.generate(forward, prompt, new_tokens, 0.7, 200 + i, V - 1)
        produced += Bq * (res.shape[1] - 1)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    for bnd in binds:
        bnd.close()
    iters = produced / Bq
    us_iter = el / iters * 1e6
    mean_ctx = mean_L + new_tokens * steps / 2
    nbytes = int(layers * (Bq * mean_ctx * Hkv * Dq * 4 + Bq * Hq * Dq * 4))    # attention bytes of one iteration
    cpu_res = cpu
    return _line("generated tokens/s, 28-layer Qwen-shaped generation loop (paged bf16, T=0.7, EOS)",
                 produced / el, "tokens/s", steps, warmup, el / steps * 1e6, "bf16",
                 {"workload": "generate", "layers": layers, "batch": Bq, "q_heads": Hq, "kv_heads": Hkv,
                  "head_dim": Dq, "block_size": bs, "vocab": V, "new_tokens": new_tokens,
                  "mean_ctx": round(mean_ctx, 1), "temperature": 0.7},
                 _hbm_roofline(nbytes, us_iter), cpu_res, us_per_iteration=round(us_iter, 1),
                 attn_algorithmic_bytes_per_iteration=nbytes)


# Context only (another machine, a CPU runtime): the pages' single four-token run of the tiny fixture on an
# AMD EPYC 9V74, latency per token in microseconds ("Persistent input/output feedback", opening section).
PAGES_TINY_US = {"stateful": [236.216, 34.542, 22.253, 20.891], "stateless": [358.640, 18.268, 6.079, 5.308],
                 "host": "AMD EPYC 9V74 (CPU runtime, single observations)"}


def bench_tiny(steps, warmup, cpu):
    """The tiny fixture (1 row, 1 head, D = 4, float32, capacity 16): a 1-token prompt then 15 appends, each
    step an in-place K and V append and decode attention over the valid prefix, then the append that would
    overflow capacity and is rejected.  Each of the `steps` runs starts from an empty cache.  Reports the
    host-observed latency of every step (issue to completion, what a caller waits per token) and its device
    time (HIP events around the step on the launch stream), and the rejected call's host time."""
    import numpy as np
    import torch
    import place_persistent_kv_amd as pkv
    from synth import workloads
    w = workloads.tiny()
    cap = w["capacity"]
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    qd = [torch.from_numpy(w["q"][t]).reshape(1, 1, 1, 4).to(dev) for t in range(cap + 1)]
    kd = [torch.from_numpy(w["k"][t]).reshape(1, 1, 1, 4).to(dev) for t in range(cap + 1)]
    vd = [torch.from_numpy(w["v"][t]).reshape(1, 1, 1, 4).to(dev) for t in range(cap + 1)]
    kc = torch.zeros((1, 1, cap, 4), device=dev)
    vc = torch.zeros((1, 1, cap, 4), device=dev)
    out = torch.empty((1, 1, 1, 4), device=dev)
    ws = torch.empty(max(256, pkv.decode_workspace_size(1, 1, 1, 4, cap)), device=dev, dtype=torch.uint8)
    bk, bv = pkv.bind_writable(kc), pkv.bind_writable(vc)
    host = np.zeros((steps, cap))
    host2 = np.zeros((steps, cap))
    devt = np.zeros((steps, cap))
    rejected = np.zeros(steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(cap)]

    def run(record, fused=True):
        # a step: the fused append + attention call (one launch); fused=False: the K+V append and the
        # attention as two calls
        for t in range(cap):
            t0 = time.perf_counter()
            evs[t][0].record(stream)
            if fused:
                pkv.decode_step(kc, vc, kd[t], vd[t], [t], 1, qd[t], out, ws)
            else:
                pkv.cache_update_kv(kc, vc, kd[t], vd[t], [t], 1)
                pkv.decode_attention(qd[t], kc, vc, [t + 1], out, ws)
            evs[t][1].record(stream)
            torch.cuda.synchronize()
            if record is not None:
                (host if fused else host2)[record, t] = (time.perf_counter() - t0) * 1e6
        if not fused:
            return
        t0 = time.perf_counter()
        try:
            pkv.decode_step(kc, vc, kd[cap], vd[cap], [cap], 1, qd[cap], out, ws)
            raise RuntimeError("the append past capacity was accepted")
        except pkv.PkvError as e:
            assert e.status == pkv.E_CAPACITY
        if record is not None:
            rejected[record] = (time.perf_counter() - t0) * 1e6
            for t in range(cap):
                devt[record, t] = evs[t][0].elapsed_time(evs[t][1]) * 1e3

    for _ in range(warmup):
        run(None)
        run(None, fused=False)
    free_before = torch.cuda.mem_get_info()[0]
    for i in range(steps):
        run(i, fused=False)
        run(i)
    alloc_delta = free_before - torch.cuda.mem_get_info()[0]
    before = (kc.clone(), vc.clone())
    try:
        pkv.decode_step(kc, vc, kd[cap], vd[cap], [cap], 1, qd[cap], out, ws)
    except pkv.PkvError:
        pass
    torch.cuda.synchronize()
    unchanged = bool(torch.equal(kc, before[0]) and torch.equal(vc, before[1]))
    # the same run as captured steps: one graph per step (its own inputs), positions held on the device (the
    # append fused into the attention at the device position, then the position + 1)
    kc2 = torch.zeros((1, 1, cap, 4), device=dev)
    vc2 = torch.zeros((1, 1, cap, 4), device=dev)
    bk2, bv2 = pkv.bind_writable(kc2), pkv.bind_writable(vc2)
    lens = torch.zeros(1, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out2 = torch.empty_like(out)
    graphs = []
    for t in range(cap):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            pkv.decode_step_dev(kc2, vc2, kd[t], vd[t], lens, 1, qd[t], cap, out2, status, ws)
            pkv.advance(lens, 1)
        graphs.append(gr)
    torch.cuda.synchronize()
    ghost = np.zeros((steps, cap))
    for i in range(-warmup, steps):
        lens.zero_()
        torch.cuda.synchronize()
        for t in range(cap):
            t0 = time.perf_counter()
            graphs[t].replay()
            torch.cuda.synchronize()
            if i >= 0:
                ghost[i, t] = (time.perf_counter() - t0) * 1e6
    graph_matches = bool(torch.equal(kc2, kc) and torch.equal(vc2, vc) and torch.equal(out2, out)) and \
        int(status.item()) == 0
    bk2.close()
    bv2.close()
    med_graph = np.median(ghost, axis=0)
    bk.close()
    bv.close()
    med_host = np.median(host, axis=0)
    med_dev = np.median(devt, axis=0)
    mean_us = float(med_host.mean())
    r = _line("tiny-fixture decode step latency (append K/V + attention), us per step", mean_us, "us/step", steps,
              warmup, mean_us * cap, "f32",
              {"workload": "tiny", "batch": 1, "heads": 1, "head_dim": 4, "capacity": cap,
               "steps_per_run": cap, "step": "in-place K and V append + decode attention (one fused call), then "
                                             "a rejected step"},
              {"bound": "latency", "achieved": None, "peak": None, "unit": None, "frac": None, "traffic": None},
              cpu, per_step_host_us=[round(float(x), 2) for x in med_host],
              per_step_device_us=[round(float(x), 2) for x in med_dev],
              two_call_per_step_host_us=[round(float(x), 2) for x in np.median(host2, axis=0)],
              two_call_mean_host_us=round(float(np.median(host2, axis=0).mean()), 2),
              first_token_host_us=round(float(med_host[0]), 2), token4_host_us=round(float(med_host[3]), 2),
              overflow_rejected_host_us=round(float(np.median(rejected)), 2),
              graph_per_step_host_us=[round(float(x), 2) for x in med_graph],
              graph_mean_host_us=round(float(med_graph.mean()), 2),
              graph_run_equals_eager_run=graph_matches,
              overflow_leaves_cache_unchanged=unchanged,
              device_bytes_allocated_during_steps=int(max(alloc_delta, 0)),
              pages_cpu_runtime_us_context=PAGES_TINY_US)
    r["higher_is_better"] = False
    return r


# ---------------------------------------------------------------------------
# The oracle's baseline for each row, in the row's own unit (CPU only: run before the GPU is touched)
# ---------------------------------------------------------------------------
def cpu_paged32k(steps, warmup):
    return oracle_baseline("paged32k_step", {}, "tokens/s",
                           "whole per-sequence decode steps of the paged32k workload (append a K/V row into the "
                           "row's 2048 pages, 32-head attention over 32768 tokens, a T=0.7 draw over 151936 "
                           "logits), numpy float64", budget_one=12.0)


def cpu_contig(steps, warmup):
    from synth import workloads
    w = workloads.contig()
    L = [int(x) for x in w["lengths"] + 16]
    return oracle_baseline("decode_rows", dict(L_list=L, Hq=w["Hq"], Hkv=w["Hkv"], D=w["D"], seed=1), "tokens/s",
                           "rows of 32-head decode attention at the workload's mid-run lengths")


def cpu_paged(steps, warmup):
    import numpy as np
    from synth import workloads
    spec = workloads.paged()
    L = spec.lengths
    med = int(L[np.argsort(L)[len(L) // 2]])
    return oracle_baseline("decode_rows", dict(L_list=[med], Hq=spec.Hq, Hkv=spec.Hkv, D=spec.D, seed=2),
                           "tokens/s", f"median-length rows ({med} tokens) of 32-head attention, scaled to the "
                           f"mean length {float(L.mean()):.0f}", scale=med / float(L.mean()))


def cpu_int4(steps, warmup):
    return oracle_baseline("int4_rows", {}, "tokens/s", "rows of the int4 workload (8192 tokens, 32 heads): exact "
                           "dequantisation + attention")


def cpu_qwen_decode(steps, warmup, layers=28):
    import numpy as np
    from synth import workloads
    w = workloads.qwen()
    L = w["lengths"].astype(np.int64) + 1
    med = int(np.median(L))
    return oracle_baseline("decode_rows", dict(L_list=[med], Hq=w["Hq"], Hkv=w["Hkv"], D=w["D"], seed=5),
                           "tokens/s", f"median-length rows ({med} tokens) of one layer's 16-head attention, "
                           f"scaled to {layers} layers and the mean length", scale=med / (layers * float(L.mean())))


def cpu_qwen_chunk(steps, warmup):
    return oracle_baseline("chunk_queries", {}, "TFLOP/s", "causal chunk queries (16 heads each) of a "
                           "median-length row", scale=1e-12)


def cpu_sample(steps, warmup):
    return oracle_baseline("sample_rows", {}, "tokens/s", "rows of T=0.7 draws over 151936 logits")


def cpu_window(steps, warmup):
    visible = 4096
    return oracle_baseline("decode_rows", dict(L_list=[visible], Hq=HQ, Hkv=HKV, D=D, seed=3), "tokens/s",
                           f"rows of 32-head attention over the {visible} visible tokens")


def cpu_mixed(steps, warmup):
    return oracle_baseline("mixed_rows", {}, "tokens/s", "rows of 32-head attention over one 32768-token row of "
                           "the workload's mixed pages (decoded exactly, float64)")


def cpu_generate(steps, warmup, layers=28, new_tokens=8):
    import numpy as np
    from synth import workloads
    w = workloads.qwen()
    L0 = w["lengths"].astype(np.int64)
    med = int(np.median(L0))
    mean_ctx = float(L0.mean()) + new_tokens * (warmup + steps / 2)
    return oracle_baseline("decode_rows", dict(L_list=[med], Hq=w["Hq"], Hkv=w["Hkv"], D=w["D"], seed=5),
                           "tokens/s", f"median-length rows of one layer's attention, scaled to {layers} layers and "
                           f"the mean context (the LM head and sampling are not included)",
                           scale=med / (layers * mean_ctx))


def cpu_tiny(steps, warmup):
    r = oracle_baseline("tiny_steps", {}, "steps/s", "the tiny fixture's stateful steps (append K and V, attention "
                        "over the valid prefix), numpy float64", budget_one=5.0, all_cores=False)
    r.update({"value": round(1e6 / r["value"], 3), "unit": "us/step"})
    r["one_core"]["value"] = r["value"]
    return r


WORKLOADS = {"contig": bench_contig, "paged": bench_paged, "int4": bench_int4, "qwen-decode": bench_qwen_decode,
             "qwen-chunk": bench_qwen_chunk, "qwen-chunk-1row": bench_qwen_chunk_1row, "sample": bench_sample,
             "window": bench_window, "mixed": bench_mixed, "generate": bench_generate, "tiny": bench_tiny,
             "mfma-ceiling": bench_mfma_ceiling}
CPU_BASELINES = {"paged32k": cpu_paged32k, "contig": cpu_contig, "paged": cpu_paged, "int4": cpu_int4,
                 "qwen-decode": cpu_qwen_decode, "qwen-chunk": cpu_qwen_chunk, "sample": cpu_sample,
                 "window": cpu_window, "mixed": cpu_mixed, "generate": cpu_generate, "tiny": cpu_tiny}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates rocprofv3 byte counters)")
    ap.add_argument("--workload", default="paged32k", choices=["paged32k", *WORKLOADS],
                    help="paged32k (default) is the headline decode step; the others measure the other rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the decode step would shard)", file=sys.stderr)
        sys.exit(2)
    # the oracle's timing runs first, before this process touches the GPU (its worker processes start fresh)
    cpu = None if args.no_cpu_baseline or args.workload not in CPU_BASELINES else \
        CPU_BASELINES[args.workload](args.steps, args.warmup)
    if args.workload != "paged32k":
        print(json.dumps(WORKLOADS[args.workload](args.steps, args.warmup, cpu)), flush=True)
        return

    g = run_gpu(args.steps, args.warmup, args.profile_copy)
    attn_bytes = attention_algorithmic_bytes()
    achieved = attn_bytes / (g["attn_us"] * 1e-6) / 1e9
    traffic = traffic_from_counters()
    result = {
        "metric": METRIC,
        "value": round(B / (g["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "paged32k", "batch": B, "ctx": CTX, "q_heads": HQ, "kv_heads": HKV,
                   "head_dim": D, "block_size": BS, "num_blocks": NB, "vocab": VOCAB,
                   "temperature": TEMPERATURE,
                   "step": "paged in-place K/V append + paged decode attention + sampling"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "attn_us": round(g["attn_us"], 2),
        "attn_tokens_per_s": round(B / (g["attn_us"] * 1e-6), 1),
        "update_us": round(g["update_us"], 2),
        "sample_us": round(g["sample_us"], 2),
        "graph_step_us": round(g["graph_step_us"], 2),
        "graph_tokens_per_s": round(B / (g["graph_step_us"] * 1e-6), 1),
        "attn_algorithmic_bytes": attn_bytes,
        "device_bytes_allocated_during_steps": g["device_bytes_allocated_during_steps"],
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
