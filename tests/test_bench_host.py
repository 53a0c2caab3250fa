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


def _kind(dense, every):
    """The driver's step kind (0 dense, 1 anchor, 2 reuse) for a schedule."""
    def kind(t):
        if t < dense:
            return 0
        since = t - dense
        return 1 if since == 0 or (every > 0 and since % every == 0) else 2
    return kind


def test_timed_window_opens_on_an_anchor():
    T = 256
    k = _kind(0, 32)
    # The driver's short command (--warmup 5 --steps 20) times an anchor first.
    assert bench.window_start(lambda t: k(t % T), 5, T) == 32
    assert bench.window_start(lambda t: k(t % T), 512, T) == 512
    assert bench.window_start(lambda t: k(t % T), 0, T) == 0
    # The GQA schedule refreshes every 16 of 64 steps.
    k16 = _kind(0, 16)
    assert bench.window_start(lambda t: k16(t % 64), 17, 64) == 32
    # Dense steps first (the long configuration): the window opens on step 0
    # of the next pass, so it holds the dense steps and then the anchor.
    kd = _kind(26, 0)
    assert bench.window_start(lambda t: kd(t % 128), 5, 128) == 128
    assert bench.window_start(lambda t: kd(t % 128), 0, 128) == 0


def test_mask_build_bandwidth():
    w = WORKLOADS["stepdllm_8k"]
    r = bench.mask_build_bandwidth(w, 0.236, 0.136, False)
    want = (64 * 8192 * 128 * 2 + 64 * 128 * 128 * 4 + 4 * 32 * 128 * 128 * 4)
    assert r["mask_build_bytes"] == want
    assert abs(r["mask_build_gbs"] - want / 0.1e-3 / 1e9) < 0.1
    assert bench.mask_build_bandwidth(w, None, 0.136, False) == {}
    assert bench.mask_build_bandwidth(w, 0.236, 0.136, True) == {}


def test_data_path_block_units():
    """The data-path view of the bench line from a fixed probe output: a
    64-query workgroup fills 4*64*d bytes of K/V per kept block for
    4*64^2*d flops (bytes = flops/64); per-clock rates times CUs and clock
    give TB/s; 8 waves x 16 MFMAs of 32x32x16 per CU and iteration give the
    step's TFLOP/s."""
    paths = {"cus": 256,
             "fill": {"ns_per_iter": 491.6, "ghz": 2.301, "cycles_per_iter": 1131,
                      "bytes_per_clk_per_cu": 57.9},
             "b128": {"ns_per_iter": 138.9, "ghz": 2.180, "cycles_per_iter": 303,
                      "bytes_per_clk_per_cu": 216.5},
             "tr": {"ns_per_iter": 145.0, "ghz": 2.225, "cycles_per_iter": 323,
                    "bytes_per_clk_per_cu": 203.1},
             "step": {"ns_per_iter": 812.7, "ghz": 1.868, "cycles_per_iter": 1518},
             "mfma": {"ns_per_iter": 525.0, "ghz": 1.993, "cycles_per_iter": 1046},
             "stream_read_128mib": {"gbs_median": 5678, "gbs_best": 6226, "frac_of_8tbs": 0.71}}
    kept, d = 52429, 128
    flops = 4.0 * 64 * 64 * d * kept
    out = bench.data_path_block(paths, flops, 64, 0.14)
    assert out["fill_bytes_per_launch"] == kept * 2 * 64 * d * 2      # K and V tiles, bf16
    assert abs(out["fill_achieved_tbs"] - kept * 2 * 64 * d * 2 / 0.14e-3 / 1e12) < 1e-3
    assert abs(out["fill_peak_tbs"] - 57.9 * 256 * 2.301e9 / 1e12) < 1e-3
    assert abs(out["step_without_softmax_tflops"] - 8 * 16 * 32768 * 256 / 812.7e-9 / 1e12) < 0.1
    assert out["hbm_stream_read_gbs"] == 5678
    # 128-query workgroups (dense and column launches) fill half the bytes.
    assert bench.data_path_block(paths, flops, 128, 0.14)["fill_bytes_per_launch"] == \
        out["fill_bytes_per_launch"] / 2
    assert bench.data_path_block(paths, flops, 64, None)["fill_achieved_tbs"] is None


def test_shared_gqa_inputs():
    """dream_gqa_8k_shared: a KV group's query heads are one shared draw plus
    a small own draw (correlation sqrt(0.99)^2 = 0.99 before rounding) with one
    temperature per group; heads of different groups are independent."""
    import torch
    w = WORKLOADS["dream_gqa_8k_shared"]
    tr = Trajectory(w)
    G = w.H // w.Hkv
    assert torch.equal(tr.temps.view(w.Hkv, G), tr.temps.view(w.Hkv, G)[:, :1].expand(w.Hkv, G))
    assert len(set(tr.temps.view(w.Hkv, G)[:, 0].tolist())) == w.Hkv
    q = tr.next()[0].float()[:, :1024].reshape(w.H, -1)
    q = q / q.norm(dim=1, keepdim=True)
    c = q @ q.T
    g = torch.arange(w.H) // G
    same = (g.view(-1, 1) == g.view(1, -1)) & ~torch.eye(w.H, dtype=torch.bool)
    assert c[same].min() > 0.98
    assert c[g.view(-1, 1) != g.view(1, -1)].abs().max() < 0.02
