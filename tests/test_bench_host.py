"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the traffic
record's source-hash gate, the temperature trend and the oracle CPU baseline."""
import json
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_only_for_the_current_source(tmp_path):
    good = tmp_path / "good.json"
    bad = tmp_path / "bad.json"
    good.write_text(json.dumps({"source_sha256": bench.src_sha(bench.ATTN_SRC),
                                "hbm_bytes_per_launch": 123}))
    bad.write_text(json.dumps({"source_sha256": "0" * 64, "hbm_bytes_per_launch": 123}))
    assert bench.traffic_record(str(good))["hbm_bytes_per_launch"] == 123
    assert bench.traffic_record(str(bad)) is None
    assert bench.traffic_record(str(tmp_path / "missing.json")) is None


def test_temperature_trend():
    w = WORKLOADS["stepdllm_8k"]
    from block_sparse_attention_pooled_amd.inputs import head_temperatures
    t = head_temperatures(w.H, w.seed).numpy()
    kept = list((np.argsort(np.argsort(t)) + 1) * 10)       # rises with t_h
    r = bench.temperature_trend(w, kept, types.SimpleNamespace(columns=False))
    assert r["kept_vs_temperature_rank_corr"] == 1.0
    ts = [p[0] for p in r["kept_fraction_by_temperature"]]
    assert ts == sorted(ts) and len(ts) == w.H
    assert bench.temperature_trend(w, kept, types.SimpleNamespace(columns=True)) == {}
    assert bench.temperature_trend(WORKLOADS["tiny"], [1, 2],
                                   types.SimpleNamespace(columns=False)) == {}


def test_cpu_baseline_on_the_tiny_workload():
    w = WORKLOADS["tiny"]
    inputs0 = Trajectory(w).next()
    flops = 4.0 * w.B ** 2 * w.d * 16
    r = bench.cpu_baseline(inputs0, w, w.sparsities[0], flops, budget_s=5.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    phys = r["physical_cores_available"]
    assert phys is None or 1 <= phys <= len(os.sched_getaffinity(0))


def test_cpu_all_on_the_tiny_workload(capsys):
    bench.cpu_all(types.SimpleNamespace(cpu_budget_s=5.0), names=("tiny",))
    line = [x for x in capsys.readouterr().out.splitlines() if x.startswith("{")][-1]
    r = json.loads(line)
    assert r["kind"] == "oracle" and len(r["results"]) == 1
    t = r["results"][0]
    assert t["workload"] == "tiny" and t["sparse_step"] == "full" and t["dense_step"] == "full"
    assert t["mask_build_s"] >= 0 and t["sparse_tflops"] > 0 and t["dense_tflops"] > 0
