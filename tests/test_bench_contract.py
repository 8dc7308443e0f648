"""The benchmark's output contract, checked on the CPU: one GPU only (a request for more exits with a
message), the JSON line's keys, the HBM roofline arithmetic, and the oracle baseline's structure (one
core and every host core, with the core count and CPU model recorded)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports nothing GPU-related at module level)

LINE_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
             "vs_baseline", "dtype", "data", "config", "roofline"}


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_json_line_carries_the_contract_keys():
    roof = bench._hbm_roofline(4_000_000_000, 1000.0)
    cpu = {"value": 1.0, "unit": "tokens/s", "cores": 8, "kind": "oracle", "sample": "x"}
    line = bench._line("m", 12.3456, "tokens/s", 10, 2, 1500.0, "bf16", {"workload": "w"}, roof, cpu, extra=1)
    assert LINE_KEYS <= set(line)
    assert line["n_gpus"] == 1 and line["steps"] == 10 and line["warmup"] == 2
    assert line["ms_per_step"] == 1.5
    assert line["higher_is_better"] is True and line["vs_baseline"] is None
    assert line["data"] == "synthetic" and line["config"] == {"workload": "w"}
    assert line["cpu_baseline"] is cpu and line["extra"] == 1
    json.dumps(line)                                  # serialisable as one line


def test_hbm_roofline_is_bytes_over_time_against_the_published_peak():
    roof = bench._hbm_roofline(4_295_753_728, 653.05)
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] == pytest.approx(4_295_753_728 / 653.05e-6 / 1e9, abs=0.05)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0, abs=1e-4)


def test_oracle_baseline_records_one_core_and_all_cores():
    res = bench.oracle_baseline("tiny_steps", {}, "steps/s", "tiny steps", budget_one=0.2, budget_all=0.3)
    assert res["kind"] == "oracle" and res["unit"] == "steps/s"
    assert res["one_core"]["cores"] == 1 and res["one_core"]["value"] > 0
    assert res["cores"] == bench.host_cores() and res["value"] > 0
    assert res["host_cpus"] == os.cpu_count() and isinstance(res["cpu_model"], str) and res["cpu_model"]
    if res["cores"] > 1:
        assert "processes together" in res["sample"]
