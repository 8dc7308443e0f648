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
oracle (numpy, float64, one BLAS thread) on a bounded sample of the same step.
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
        pkv.paged_cache_update(pool, k_pool, table, new_k, pos, 1)
        pkv.paged_cache_update(pool, v_pool, table, new_v, pos, 1)
        if ev:
            ev[1].record(stream)
        pkv.paged_decode_attention(q, k_pool, v_pool, table, maxb, BS, lens, out, ws, pool=pool)
        if ev:
            ev[2].record(stream)
        pkv.sample(logits, TEMPERATURE, 1000 + i, ids, sws)
        if ev:
            ev[3].record(stream)

    for i in range(warmup):
        step(i, None)
    torch.cuda.synchronize()
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
        "device_bytes_allocated_during_steps": int(max(alloc_delta, 0)),
    }


def run_cpu_baseline(budget_s: float = 12.0):
    """Time the oracle on whole per-sequence decode steps of the same workload:
    append one K/V row into the row's 2048 pages, 32-head attention over 32768
    tokens, and a T=0.7 draw over 151936 logits.  One sequence's pages are
    generated once and reused; the oracle's work does not depend on the values."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import attention, cache, numeric, sampling

    maxb = CTX // BS
    order = synth.permutation(synth.rng(3, 7), maxb)
    opool = cache.PagePool(maxb, BS, 1, maxb, order)
    opool.reserve(0, CTX)
    g = synth.rng(3, 8)
    k_pages = synth.f32_to_bf16_bits(synth.normal(g, (maxb, HKV, BS, D)))
    v_pages = synth.f32_to_bf16_bits(synth.normal(g, (maxb, HKV, BS, D)))
    q = synth.f32_to_bf16_bits(synth.normal(g, (HQ, D)))
    new_k = synth.f32_to_bf16_bits(synth.normal(g, (1, HKV, 1, D)))
    new_v = synth.f32_to_bf16_bits(synth.normal(g, (1, HKV, 1, D)))
    logits = synth.normal(g, (1, VOCAB), 3.0)
    G = HQ // HKV
    rows = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            cache.paged_cache_update(k_pages, opool.table, new_k, [CTX - 1], 1, BS, opool.held)
            cache.paged_cache_update(v_pages, opool.table, new_v, [CTX - 1], 1, BS, opool.held)
            K = numeric.bf16_to_f64(cache.paged_gather(k_pages, opool.table[0], CTX, BS))
            V = numeric.bf16_to_f64(cache.paged_gather(v_pages, opool.table[0], CTX, BS))
            qh = numeric.bf16_to_f64(q)
            for h in range(HQ):
                attention.attend(qh[h], K[h // G], V[h // G], 1.0 / np.sqrt(D))
            sampling.sample(logits, TEMPERATURE, rows, )
            rows += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return {"value": rows / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} whole per-sequence decode steps of the paged32k workload "
                      f"(append K/V row, 32-head attention over 32768 tokens, T=0.7 draw over "
                      f"{VOCAB} logits) in {el:.1f} s, numpy float64 with 1 BLAS thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the decode step would shard)", file=sys.stderr)
        sys.exit(2)

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
        "attn_algorithmic_bytes": attn_bytes,
        "device_bytes_allocated_during_steps": g["device_bytes_allocated_during_steps"],
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
