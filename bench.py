#!/usr/bin/env python3
"""Benchmark of the pooled block-sparse attention path on one MI355X.

Workload (default): the Step-dLLM headline attention layer shape -- H = 32
query/key heads, L = 8192 tokens, d = 128, 64-token blocks, 90% of the blocks
dropped under the global budget, 256 denoising steps with the mask rebuilt at
every 32nd (anchor) step.  Inputs are seeded synthetic Q/K/V with per-head
temperatures, per-step drift and abrupt redraws of Q/K at steps 64 and 160;
the whole 256-step trajectory is generated into HBM before timing, so every
timed step reads its own inputs.

A timed step is one denoising step through the step driver (anchor: pool,
score, select, lists, plan, then sparse attention; other steps: sparse
attention on the stored mask).  `value` is the effective throughput
4*B^2*d*K / (wall time per step), K = kept blocks.  The roofline object is for
the sparse attention kernel, timed with HIP events on the launch stream.
The CPU baseline runs the oracle (test infrastructure) on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn ms/step + effective TFLOP/s, L=8192 H=32 d=128 90% sparse"
METRIC_COLS = ("column-sparse attn (PulseCol variant) ms/step + effective TFLOP/s, "
               "L=8192 H=32 d=128 90% of key columns dropped")
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_pooled_amd", "csrc", "attn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_stepdllm_8k_traffic.json")
TRAFFIC_FILE_COLS = os.path.join(ROOT, "profiles", "col_attn_stepdllm_8k_traffic.json")



def physical_cores():
    """Distinct (socket, core) pairs among the CPUs this process may run on,
    from sysfs; None where the topology files are missing."""
    pairs = set()
    for c in os.sched_getaffinity(0):
        base = f"/sys/devices/system/cpu/cpu{c}/topology/"
        try:
            with open(base + "physical_package_id") as f1, open(base + "core_id") as f2:
                pairs.add((f1.read().strip(), f2.read().strip()))
        except OSError:
            return None
    return len(pairs) or None

def window_start(kind_at, warmup, T):
    """First step index t >= warmup at which the timed window opens: the
    trajectory's first step (t % T == 0) when the schedule starts with dense
    steps, else an anchor step.  kind_at(t) is the driver's step kind
    (0 dense, 1 anchor, 2 reuse)."""
    first = kind_at(0)
    for t in range(warmup, warmup + T):
        if (first == 0 and t % T == 0) or (first == 1 and kind_at(t) == 1):
            return t
    return warmup


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    # Two passes over the trajectory before timing: the first few hundred steps
    # of a process run 2-3% slower than later ones, whichever inputs they read.
    p.add_argument("--warmup", type=int, default=512)
    p.add_argument("--runs", type=int, default=1,
                   help="time the K steps this many times and report the median run")
    p.add_argument("--workload", default="stepdllm_8k")
    p.add_argument("--sparsity", type=float, default=None)
    p.add_argument("--traj-steps", type=int, default=None,
                   help="distinct input steps held in HBM (default: the workload's step count)")
    p.add_argument("--dense-iters", type=int, default=5)
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--mask-quality", action="store_true",
                   help="instead of the timing run: recall of the mask in use at every step "
                        "against the true block attention mass of that step (anchors and "
                        "staleness across each refresh interval)")
    p.add_argument("--per-head-budget", action="store_true",
                   help="uniform per-head budget (the baseline the head-adaptive one is "
                        "compared with) instead of the global budget")
    p.add_argument("--columns", action="store_true",
                   help="the column-sparse variant (PulseCol): per head the ceil((1-s)L) key "
                        "columns of largest pooled-query mass, refreshed at the same anchors")
    p.add_argument("--gqa-group", action="store_true",
                   help="GQA variant with group-shared K/V tiles against the per-head kernel, "
                        "at the workload's anchor for each of its sparsities")
    p.add_argument("--cpu-all", action="store_true",
                   help="time the CPU oracle on every configuration (host only, no GPU): one "
                        "mask build, one sparse and one dense step, row-sampled past a budget")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (for counter calibration)")
    return p.parse_args()


def mask_build_bandwidth(w, anchor_ms, attn_ms, columns):
    """Mask build of a block mask against HBM speed: its algorithmic bytes
    (Q and K read once, pooled means written, four fp32 passes over the
    H * nb^2 score matrix) over the measured build time (anchor step minus a
    reuse step)."""
    if columns or not (anchor_ms and attn_ms) or anchor_ms <= attn_ms:
        return {}
    nbytes = ((w.H + w.Hkv) * w.L * w.d * 2 + (w.H + w.Hkv) * w.nb * w.d * 4
              + 4 * w.H * w.nb * w.nb * 4)
    gbs = nbytes / ((anchor_ms - attn_ms) * 1e-3) / 1e9
    return {"mask_build_bytes": nbytes, "mask_build_gbs": round(gbs, 1),
            "mask_build_frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def near_ties(drv, w, dims, rel=1e-5, show=8):
    """Scores of the last anchor's pooled map within rel of the cut (the K-th
    largest), from the GPU's own scores and select state in the workspace:
    the count and the first few (flat index, score, kept)."""
    import torch
    from block_sparse_attention_pooled_amd import binding as B
    lay = B.workspace_layout(dims)
    n = w.H * w.nb * w.nb
    P = drv.ws[lay.scores:lay.scores + 4 * n].view(torch.float32)
    key = int(drv.ws[lay.select:lay.select + 4].view(torch.int32).item()) & 0xFFFFFFFF
    bits = key ^ 0x80000000 if key & 0x80000000 else ~key & 0xFFFFFFFF
    cut = struct.unpack("<f", struct.pack("<I", bits))[0]
    if not cut > 0:
        return {"near_ties": {"count": 0, "cut": cut, "listed": []}}
    idx = torch.nonzero(torch.abs(P - cut) <= rel * cut).view(-1)
    rp = drv.row_ptr.cpu()
    ci = drv.col_idx[:drv.K].cpu()
    listed = []
    for f in idx[:show].tolist():
        r, j = divmod(f, w.nb)
        kept = bool((ci[int(rp[r]):int(rp[r + 1])] == j).any())
        listed.append([f, float(P[f]), kept])
    return {"near_ties": {"count": int(idx.numel()), "cut": cut, "rel": rel, "listed": listed}}


def src_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def traffic_record(path=TRAFFIC_FILE):
    """HBM bytes per attention launch from committed counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != src_sha(ATTN_SRC):
        return None
    return rec


def sustained_mfma_rate():
    """Run the package's MFMA-rate probe (built beside the library): the bf16
    MFMA rate and shader clock the GPU holds under a pure MFMA load, for
    random and for zero operands.  None if the probe is not built."""
    import subprocess
    exe = os.path.join(ROOT, "block_sparse_attention_pooled_amd", "mfma_rate")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        print(f"bench.py: mfma_rate failed: {r.stderr.strip()}", file=sys.stderr)
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def data_path_rates():
    """Run the package's data-path probe (built beside the library): buffer->LDS
    fill and LDS read rates per CU at the attention kernel's occupancy, one
    step's reads, fills and matrix products without the softmax, and a
    streaming HBM read.  None if the probe is not built."""
    import subprocess
    exe = os.path.join(ROOT, "block_sparse_attention_pooled_amd", "path_rates")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        print(f"bench.py: path_rates failed: {r.stderr.strip()}", file=sys.stderr)
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def data_path_block(paths, flops_step, q_rows, attn_ms):
    """The bench line's view of the path the K/V tiles take into each CU,
    from the data-path probe's output.  A workgroup of q_rows query rows fills
    each kept key block's K and V tiles (4*q_rows*d bytes for 4*q_rows^2*d
    flops) into LDS once, so a launch fills flops/q_rows bytes."""
    cus = paths["cus"]
    fill_bytes = flops_step / q_rows
    step_flops_per_cu = 8 * 16 * 2 * 32 * 32 * 16   # 8 waves x 16 MFMAs per iteration
    return {
        "probe": "block_sparse_attention_pooled_amd/path_rates",
        "fill_bytes_per_launch": fill_bytes,
        "fill_achieved_tbs": round(fill_bytes / (attn_ms * 1e-3) / 1e12, 3) if attn_ms else None,
        "fill_bytes_per_clk_per_cu": paths["fill"]["bytes_per_clk_per_cu"],
        "fill_peak_tbs": round(paths["fill"]["bytes_per_clk_per_cu"] * cus *
                               paths["fill"]["ghz"] / 1e3, 3),
        "fill_ghz": paths["fill"]["ghz"],
        "lds_read_bytes_per_clk_per_cu": {"b128": paths["b128"]["bytes_per_clk_per_cu"],
                                          "tr16_b64": paths["tr"]["bytes_per_clk_per_cu"]},
        "step_without_softmax_tflops": round(step_flops_per_cu * cus /
                                             paths["step"]["ns_per_iter"] / 1e3, 1),
        "step_without_softmax_ghz": paths["step"]["ghz"],
        "hbm_stream_read_gbs": paths["stream_read_128mib"]["gbs_median"],
    }


def cpu_baseline(inputs0, w, sparsity, flops_per_step, budget_s, per_head=False):
    """The oracle as it stands, on the host cores: one full mask build on step-0
    Q/K plus sparse attention on a deterministic sample of rows, extrapolated
    to one step by kept blocks (the anchor's mask build amortised over the
    refresh period)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle as O
    from block_sparse_attention_pooled_amd.inputs import to_host_f32

    q, k, v = (to_host_f32(x) for x in inputs0)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    ref = O.build_mask(q, k, w.B, sparsity, per_head=per_head)
    t_mask = time.perf_counter() - t0
    rp, ci, K = ref["row_ptr"], ref["col_idx"], ref["K"]
    lens = np.diff(rp)
    nonempty = np.nonzero(lens)[0]
    order = np.random.default_rng(w.seed).permutation(nonempty)
    out = np.zeros(q.shape, np.float64)
    done_rows, done_pairs = 0, 0
    batch = threads * 2
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while done_rows < order.size and time.perf_counter() - t0 < budget_s:
            chunk = order[done_rows:done_rows + batch]
            list(ex.map(lambda r: O.sparse_attn(q, k, v, w.B, rp, ci, rows=[int(r)], out=out),
                        chunk))
            done_rows += chunk.size
            done_pairs += int(lens[chunk].sum())
    t_attn = time.perf_counter() - t0
    period = w.refresh_every if w.refresh_every > 0 else w.steps
    t_step = t_attn * K / max(done_pairs, 1) + t_mask / period
    return {
        "value": round(flops_per_step / t_step / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads, "physical_cores_available": physical_cores(),
        "kind": "oracle",
        "sample": (f"one full mask build on the step-0 Q/K ({t_mask:.2f} s, amortised over "
                   f"{period} steps) + fp64 sparse attention on {done_rows} of {nonempty.size} "
                   f"non-empty rows ({done_pairs} of {K} kept blocks, {t_attn:.2f} s), "
                   f"extrapolated to one step by kept blocks"),
        "ms_per_step": round(t_step * 1e3, 3),
    }


def cpu_baseline_cols(inputs0, w, sparsity, flops_per_step, budget_s):
    """The column-sparse variant's oracle on the host cores: one full column
    mask build on step-0 Q/K plus attention on a deterministic sample of query
    blocks, extrapolated to one step by query blocks (the mask build amortised
    over the refresh period)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle as O
    from block_sparse_attention_pooled_amd.inputs import to_host_f32

    q, k, v = (to_host_f32(x) for x in inputs0)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    _, cols, k_c = O.build_col_mask(q, k, w.B, sparsity)
    t_mask = time.perf_counter() - t0
    rows_all = w.H * w.nb
    order = np.random.default_rng(w.seed).permutation(rows_all)
    out = np.zeros(q.shape, np.float64)
    done = 0
    batch = threads * 2
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while done < rows_all and time.perf_counter() - t0 < budget_s:
            chunk = order[done:done + batch]
            list(ex.map(lambda r: O.col_attn(q, k, v, w.B, cols, rows=[int(r)], out=out), chunk))
            done += chunk.size
    t_attn = time.perf_counter() - t0
    period = w.refresh_every if w.refresh_every > 0 else w.steps
    t_step = t_attn * rows_all / max(done, 1) + t_mask / period
    return {
        "value": round(flops_per_step / t_step / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads, "physical_cores_available": physical_cores(),
        "kind": "oracle",
        "sample": (f"one full column mask build on the step-0 Q/K ({t_mask:.2f} s, amortised "
                   f"over {period} steps) + fp64 column attention on {done} of {rows_all} "
                   f"query blocks ({k_c} columns per head, {t_attn:.2f} s), extrapolated to "
                   f"one step by query blocks"),
        "ms_per_step": round(t_step * 1e3, 3),
    }


def mask_quality(args, w, sparsity, dev, T):
    """Recall of the mask in use at each denoising step: the share of the true
    block attention mass (full softmax map of that step's Q/K) that the kept
    blocks hold, averaged over all rows (an empty row recalls 0)."""
    import torch
    from block_sparse_attention_pooled_amd import binding as B
    from block_sparse_attention_pooled_amd.inputs import Trajectory

    dims = B.make_dims(w.H, w.Hkv, w.L, w.d, w.B)
    drv = B.Driver(dims, w.dense_steps, w.refresh_every, sparsity, device=dev,
                   per_head_budget=args.per_head_budget, column_sparse=args.columns)
    o = torch.empty(w.H, w.L, w.d, dtype=torch.bfloat16, device=dev)
    mass = torch.empty(w.H * w.nb * w.nb, dtype=torch.float32, device=dev)
    rec = torch.empty(w.H * w.nb, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    traj = Trajectory(w, dev)
    # The best mask of the same budget: top-K of the true mass map itself.
    best_rp = torch.empty(w.H * w.nb + 1, dtype=torch.int32, device=dev)
    best_ci = torch.empty(max(drv.K, 1), dtype=torch.int32, device=dev)
    best_ws = torch.empty(B.workspace_bytes(dims), dtype=torch.uint8, device=dev)
    best_at_anchor = []
    overlap, prev_keep = [], None      # kept set shared with the previous anchor
    per_step, kinds, mass_ms = [], [], []
    since_anchor = []
    last_anchor = None
    for t in range(T):
        q, k, v = traj.next()
        kind = drv.step_kind(t)
        drv.step(t, q, k, v, o, stream)
        if kind == 0:
            continue
        if kind == 1:
            last_anchor = t
            if args.columns:
                cols = drv.cols().cpu()
                keep = set((cols + (torch.arange(w.H).view(-1, 1) * w.L)).view(-1).tolist())
            else:
                rp = drv.row_ptr.cpu()
                ci = drv.col_idx[:drv.K].cpu()
                rows = torch.repeat_interleave(torch.arange(w.H * w.nb), rp[1:] - rp[:-1])
                keep = set((rows * w.nb + ci.long()).tolist())
            if prev_keep is not None:
                overlap.append(round(len(keep & prev_keep) / max(len(keep), 1), 5))
            prev_keep = keep
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.columns:
            # Recall of the kept columns straight from this step's Q/K.
            a.record(stream)
            B.col_recall(dims, q, k, drv.cols(), rec, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            mass_ms.append(a.elapsed_time(b))
            per_step.append(float(rec.mean()))
            kinds.append(kind)
            since_anchor.append(t - last_anchor)
            continue
        a.record(stream)
        B.block_mass(dims, q, k, mass, stream)
        b.record(stream)
        B.mask_recall(dims, mass, drv.row_ptr, drv.col_idx, rec, nnz=drv.K, stream=stream)
        torch.cuda.synchronize()
        mass_ms.append(a.elapsed_time(b))
        per_step.append(float(rec.mean()))
        if kind == 1:
            B.select_mask(dims, sparsity, mass, best_ws, best_rp, best_ci, stream=stream,
                          per_head=args.per_head_budget)
            B.mask_recall(dims, mass, best_rp, best_ci, rec, nnz=drv.K, stream=stream)
            torch.cuda.synchronize()
            best_at_anchor.append(float(rec.mean()))
        kinds.append(kind)
        since_anchor.append(t - last_anchor)
    R = w.refresh_every if w.refresh_every > 0 else max(since_anchor) + 1
    by_offset = []
    for off in range(R):
        xs = [r for r, s in zip(per_step, since_anchor) if s == off]
        by_offset.append(round(sum(xs) / len(xs), 5) if xs else None)
    at_anchor = [r for r, kd in zip(per_step, kinds) if kd == 1]
    last_in = [r for r, s in zip(per_step, since_anchor) if s == R - 1]
    mass_flops = 4.0 * w.H * w.L * w.L * w.d          # two score passes
    if args.columns:                                  # one full pass, then the kept columns
        mass_flops = 2.0 * w.H * w.L * w.d * (w.L + drv.k_c)
    mms = sorted(mass_ms)[len(mass_ms) // 2]
    result = {
        "metric": ("mask recall: share of the exact attention on the kept key columns"
                   if args.columns else
                   "mask recall: share of the true block attention mass on the kept blocks"),
        "value": round(sum(per_step) / len(per_step), 5),
        "unit": "fraction",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": len(per_step),
        "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "L": w.L, "d": w.d, "block": w.B,
                   "sparsity": sparsity,
                   **({"kept_columns_per_head": drv.k_c} if args.columns
                      else {"kept_blocks": drv.K}),
                   "budget": ("columns" if args.columns else
                              "per_head" if args.per_head_budget else "global"),
                   "refresh_every": w.refresh_every, "dense_steps": w.dense_steps},
        "recall_at_anchors": round(sum(at_anchor) / len(at_anchor), 5),
        "best_recall_same_budget_at_anchors": (
            round(sum(best_at_anchor) / len(best_at_anchor), 5) if best_at_anchor else None),
        "random_mask_recall": round(drv.k_c / w.L if args.columns
                                    else drv.K / (w.H * w.nb * w.nb), 5),
        "recall_last_step_of_interval": round(sum(last_in) / len(last_in), 5) if last_in else None,
        "recall_by_steps_since_anchor": by_offset,
        "anchor_overlap_with_previous": overlap,
        "recall_per_step": [round(x, 5) for x in per_step],
        ("col_recall_ms" if args.columns else "block_mass_ms"): round(mms, 4),
        ("col_recall_tflops" if args.columns else "block_mass_tflops"):
            round(mass_flops / (mms * 1e-3) / 1e12, 2),
    }
    print(json.dumps(result), flush=True)


def temperature_trend(w, per_head, args):
    """Per-head kept fraction of the last mask against the head's temperature
    t_h (workloads that draw temperatures, block masks): the pairs sorted by
    t_h and their Spearman rank correlation."""
    if args.columns or not w.temperatures:
        return {}
    import numpy as np
    from block_sparse_attention_pooled_amd.inputs import head_temperatures
    t = head_temperatures(w.H, w.seed).numpy().astype(np.float64)
    f = np.asarray(per_head, np.float64) / (w.nb * w.nb)
    rt, rf = np.argsort(np.argsort(t)), np.argsort(np.argsort(f, kind="stable"), kind="stable")
    rho = float(np.corrcoef(rt, rf)[0, 1]) if f.std() > 0 else None
    order = np.argsort(t)
    return {"kept_fraction_by_temperature": [[round(float(t[h]), 3), round(float(f[h]), 4)]
                                             for h in order],
            "kept_vs_temperature_rank_corr": round(rho, 4) if rho is not None else None}


CPU_ALL_WORKLOADS = ("tiny", "llada_2k", "stepdllm_8k", "dream_gqa_8k", "long_64k")


def cpu_all(args, names=CPU_ALL_WORKLOADS):
    """The oracle as it stands on the host cores, per configuration: one full
    mask build on the step-0 Q/K, then sparse and dense attention over seeded
    random rows until a time budget each, extrapolated to a whole step by kept
    pairs (sparse) or rows (dense) when the budget ends first."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle as O
    from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory, to_host_f32

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    budget = args.cpu_budget_s
    out = []

    def timed_rows(fn, order, weight, total_weight):
        done, acc, t0 = 0, 0, time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            while done < order.size and time.perf_counter() - t0 < budget:
                chunk = order[done:done + 2 * threads]
                list(ex.map(fn, chunk))
                done += chunk.size
                acc += int(weight[chunk].sum())
        t = time.perf_counter() - t0
        full = done == order.size
        return (t if full else t * total_weight / max(acc, 1)), full, done

    for name in names:
        w = WORKLOADS[name]
        s = w.sparsities[-1]
        q, k, v = (to_host_f32(x) for x in Trajectory(w).next())
        t0 = time.perf_counter()
        ref = O.build_mask(q, k, w.B, s)
        t_mask = time.perf_counter() - t0
        rp, ci, K = ref["row_ptr"], ref["col_idx"], ref["K"]
        lens = np.diff(rp)
        rng = np.random.default_rng(w.seed)
        nonempty = rng.permutation(np.nonzero(lens)[0])
        buf = np.zeros(q.shape, np.float64)
        t_sp, sp_full, sp_rows = timed_rows(
            lambda r: O.sparse_attn(q, k, v, w.B, rp, ci, rows=[int(r)], out=buf),
            nonempty, lens, K)
        rows = w.H * w.nb
        t_de, de_full, de_rows = timed_rows(
            lambda r: O.dense_attn(q, k, v, w.B, rows=[int(r)], out=buf),
            rng.permutation(rows), np.ones(rows, np.int64), rows)
        sp_flops = 4.0 * w.B ** 2 * w.d * K
        de_flops = 4.0 * w.H * w.L * w.L * w.d
        out.append({"workload": name, "H": w.H, "Hkv": w.Hkv, "L": w.L, "d": w.d, "B": w.B,
                    "sparsity": s, "mask_build_s": round(t_mask, 3),
                    "sparse_step_s": round(t_sp, 3), "sparse_step": (
                        "full" if sp_full else f"extrapolated from {sp_rows} rows"),
                    "sparse_tflops": round(sp_flops / t_sp / 1e12, 5),
                    "dense_step_s": round(t_de, 3), "dense_step": (
                        "full" if de_full else f"extrapolated from {de_rows} rows"),
                    "dense_tflops": round(de_flops / t_de / 1e12, 5)})
        print(f"cpu-all: {name} done", file=sys.stderr, flush=True)
        del q, k, v, buf, ref
    print(json.dumps({"metric": "CPU oracle time per configuration (fp64, host cores)",
                      "unit": "s", "higher_is_better": False, "kind": "oracle",
                      "cores": threads, "physical_cores_available": physical_cores(), "budget_s_per_part": budget, "results": out}),
          flush=True)


def gqa_group(args, w, dev):
    """Per-head sparse kernel against the group-shared variant on the anchor
    step's mask: kernel times, bit identity, K/V tiles streamed per kept pair."""
    import numpy as np
    import torch
    from block_sparse_attention_pooled_amd import binding as B
    from block_sparse_attention_pooled_amd.inputs import Trajectory
    q, k, v = Trajectory(w, dev).next()
    dims = B.make_dims(w.H, w.Hkv, w.L, w.d, w.B)
    G = w.H // w.Hkv
    sps = [args.sparsity] if args.sparsity is not None else list(w.sparsities)
    out = []

    def med(fn, reps=30):
        for _ in range(5):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(); fn(); b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]

    for s in sps:
        buf = B.MaskBuffers(dims, s, device=dev)
        B.build_mask(dims, s, q, k, buf.ws, buf.row_ptr, buf.col_idx)
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        t_head = med(lambda: B.sparse_attn(dims, q, k, v, buf.col_idx, buf.ws, o1, nnz=buf.K))
        t_group = med(lambda: B.sparse_attn_group(dims, q, k, v, buf.row_ptr, buf.col_idx, o2,
                                                  nnz=buf.K))
        rp = buf.row_ptr.cpu().numpy()
        ci = buf.col_idx[:buf.K].cpu().numpy()
        keep = np.zeros((w.H, w.nb, w.nb), bool)
        rows = np.repeat(np.arange(w.H * w.nb), np.diff(rp))
        keep.reshape(-1, w.nb)[rows, ci] = True
        union = 0
        for g in range(w.Hkv):
            for h0 in range(g * G, (g + 1) * G, 2):
                union += int(keep[h0:min(h0 + 2, (g + 1) * G)].any(axis=0).sum())
        flops = 4.0 * w.B ** 2 * w.d * buf.K
        out.append({"sparsity": s, "kept_blocks": buf.K,
                    "per_head_kernel_ms": round(t_head, 4), "group_kernel_ms": round(t_group, 4),
                    "per_head_tflops": round(flops / (t_head * 1e-3) / 1e12, 1),
                    "group_tflops": round(flops / (t_group * 1e-3) / 1e12, 1),
                    "identical_output": bool(torch.equal(o1, o2)),
                    "kv_tiles_per_kept_pair": round(union / buf.K, 4)})
    print(json.dumps({
        "metric": "GQA group-shared K/V tiles: kernel time against the per-head sparse kernel",
        "unit": "ms", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "Hkv": w.Hkv, "L": w.L, "d": w.d,
                   "block": w.B, "heads_per_workgroup": 2},
        "results": out}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported (a "
              "multi-GPU run would shard the layer by query head, one all-reduce of the "
              "select histogram per digit pass)", file=sys.stderr)
        sys.exit(2)

    if args.cpu_all:
        cpu_all(args)
        return

    import torch
    from block_sparse_attention_pooled_amd import binding as B
    from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory

    w = WORKLOADS[args.workload]
    sparsity = args.sparsity if args.sparsity is not None else w.sparsities[-1]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = args.traj_steps or w.steps
    if args.mask_quality:
        mask_quality(args, w, sparsity, dev, T)
        return
    if args.gqa_group:
        gqa_group(args, w, dev)
        return
    if args.columns and args.per_head_budget:
        print("bench.py: --columns already keeps the same number of columns per head",
              file=sys.stderr)
        sys.exit(2)

    # Inputs for every step of the trajectory, resident in HBM before timing.
    traj = Trajectory(w, dev)
    inputs = [traj.next() for _ in range(T)]
    del traj
    torch.cuda.synchronize()
    dims = B.make_dims(w.H, w.Hkv, w.L, w.d, w.B)
    drv = B.Driver(dims, w.dense_steps, w.refresh_every, sparsity, device=dev,
                   per_head_budget=args.per_head_budget, column_sparse=args.columns)
    o = torch.empty(w.H, w.L, w.d, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def run_step(t):
        p = t % T
        q, k, v = inputs[p]
        drv.step(p, q, k, v, o, stream)

    for t in range(args.warmup):
        run_step(t)
    torch.cuda.synchronize()

    # The timed window opens on an anchor: the first trajectory position at or
    # after the warm-up whose step builds a mask (dense steps first if the
    # schedule has them, as in the long configuration), so a window of any
    # length holds the mask builds the schedule makes in it.
    start = window_start(lambda p: drv.step_kind(p % T), args.warmup, T)
    K_steps = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K_steps)]
    kinds = [drv.step_kind((start + i) % T) for i in range(K_steps)]
    # HIP events on the launch stream: every anchor / dense step is bracketed
    # on its own, and each run of consecutive reuse steps (one sparse launch
    # each) as a whole, so the cost of a pair of events (about 6 us of stream
    # time) is spread over the run instead of counted in a single launch.
    opens = [kd != 2 or i == 0 or kinds[i - 1] != 2 for i, kd in enumerate(kinds)]
    closes = [kd != 2 or i == K_steps - 1 or kinds[i + 1] != 2 for i, kd in enumerate(kinds)]
    # --runs R > 1 repeats the timed region R times (the same K steps) and
    # takes the median run's wall time; the events are those of the last run.
    walls = []
    for _ in range(max(1, args.runs)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K_steps):
            if opens[i]:
                ev[i][0].record(stream)
            run_step(start + i)
            if closes[i]:
                ev[i][1].record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    wall = sorted(walls)[len(walls) // 2]
    ms_per_step = wall * 1e3 / K_steps
    spans = []                      # (kind, first step, last step, ms)
    i = 0
    while i < K_steps:
        j = i
        while not closes[j]:
            j += 1
        spans.append((kinds[i], i, j, ev[i][0].elapsed_time(ev[j][1])))
        i = j + 1

    def mean(xs):
        return sum(xs) / len(xs) if xs else None

    reuse = [(j - i + 1, ms) for kd, i, j, ms in spans if kd == 2]
    n_reuse_timed = sum(n for n, _ in reuse)
    attn_ms = sum(ms for _, ms in reuse) / n_reuse_timed if n_reuse_timed else None
    anchor_ms = mean([ms for kd, _, _, ms in spans if kd == 1])
    dense_step_ms = mean([ms for kd, _, _, ms in spans if kd == 0])
    n_anchor = sum(1 for kd in kinds if kd == 1)
    # One refresh interval of the schedule (an anchor then R - 1 reuse steps),
    # from the measured anchor-step and reuse-step times: the per-step cost
    # over the whole trajectory, whatever the window length.
    R = w.refresh_every
    interval_ms = ((anchor_ms + (R - 1) * attn_ms) / R
                   if (R > 0 and anchor_ms and attn_ms) else None)

    Kkept = drv.K
    if args.columns:
        # Every query token attends to the k_c kept columns of its head.
        per_head = [drv.k_c] * w.H
        flops_step = 4.0 * w.L * w.d * drv.k_c * w.H
    else:
        # Kept blocks per head in the mask left by the last anchor before timing ended.
        rp = drv.row_ptr.cpu()
        per_head = [int(rp[(h + 1) * w.nb] - rp[h * w.nb]) for h in range(w.H)]
        flops_step = 4.0 * w.B * w.B * w.d * Kkept
    ph_mean = sum(per_head) / len(per_head)
    ph_cv = (sum((x - ph_mean) ** 2 for x in per_head) / len(per_head)) ** 0.5 / ph_mean
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    # Whole-step roofline: each timed step at its bound (kept flops at the bf16
    # peak or its Q/K/V/O bytes at HBM speed, whichever is longer; a dense step
    # likewise), plus each anchor's mask build at HBM speed (Q and K read once,
    # pooled means written, about four passes over the score matrix). Block
    # masks only: a column step moves the kept K/V rows and its anchor scores
    # every key, which this byte count does not describe.
    attn_bytes = (2 * w.H + 2 * w.Hkv) * w.L * w.d * 2
    mask_bytes = ((w.H + w.Hkv) * w.L * w.d * 2 + (w.H + w.Hkv) * w.nb * w.d * 4
                  + 4 * w.H * w.nb * w.nb * 4)
    ideal_s = 0.0
    for kd in kinds:
        f = 4.0 * w.H * w.L * w.L * w.d if kd == 0 else flops_step
        ideal_s += max(f / (PEAK_BF16_TFLOPS * 1e12), attn_bytes / (PEAK_HBM_GBS * 1e9))
        if kd == 1:
            ideal_s += mask_bytes / (PEAK_HBM_GBS * 1e9)
    ideal_ms_step = ideal_s * 1e3 / K_steps

    # Same-GPU dense baseline on the step-0 inputs.
    q0, k0, v0 = inputs[0]
    od = torch.empty_like(o)
    B.dense_attn(dims, q0, k0, v0, od, stream)
    torch.cuda.synchronize()
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.dense_iters)]
    for a, b in dev_ev:
        a.record(stream)
        B.dense_attn(dims, q0, k0, v0, od, stream)
        b.record(stream)
    torch.cuda.synchronize()
    dense_ms = mean([a.elapsed_time(b) for a, b in dev_ev])
    dense_flops = 4.0 * w.H * w.L * w.L * w.d

    # The sparse kernel on the last anchor's mask, with one step's inputs
    # repeated (the 256 MB last-level cache then holds them), timed as one run
    # of 32 launches: against kernel_ms, where every step reads fresh inputs
    # from HBM, the share of a launch that waits on HBM.
    resident_ms = None
    if attn_ms and not args.columns:
        qL, kL, vL = inputs[(start + K_steps - 1) % T]
        for _ in range(3):
            B.sparse_attn(dims, qL, kL, vL, drv.col_idx, drv.ws, o, nnz=drv.K, stream=stream)
        ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ra.record(stream)
        for _ in range(32):
            B.sparse_attn(dims, qL, kL, vL, drv.col_idx, drv.ws, o, nnz=drv.K, stream=stream)
        rb.record(stream)
        torch.cuda.synchronize()
        resident_ms = ra.elapsed_time(rb) / 32

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    attn_tflops = flops_step / (attn_ms * 1e-3) / 1e12 if attn_ms else None
    trec = None
    if (w.name, w.d, w.B, sparsity) == ("stepdllm_8k", 128, 64, 0.9):
        trec = traffic_record(TRAFFIC_FILE_COLS if args.columns else TRAFFIC_FILE)
    mode = "cols" if args.columns else "sparse"
    # Column rows of a head share one key list: with 64-token blocks they run
    # as 128-query workgroups (the library's launch choice, same output).
    inst_b = 128 if (args.columns and w.B == 64 and w.L % 128 == 0) else w.B
    roofline = {
        "bound": "mfma",
        "kernel": f"k_attn<{w.d},{inst_b},{mode}>",
        "achieved": round(attn_tflops, 3) if attn_tflops else None,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4) if attn_tflops else None,
        "traffic": trec["hbm_bytes_per_launch"] if trec else None,
        "l2_hit_rate": trec.get("l2_hit_rate") if trec else None,
        "algorithmic_flops_per_launch": flops_step,
        "kernel_ms": round(attn_ms, 5) if attn_ms else None,
        "kernel_launches_timed": n_reuse_timed,
    }
    if resident_ms:
        roofline["kernel_ms_resident_inputs"] = round(resident_ms, 5)
        roofline["fresh_input_cost"] = round(attn_ms / resident_ms - 1.0, 4)
    # What the chip sustains under pure MFMA load (power-limited clock with
    # real-valued operands), measured after the timed region.
    rate = sustained_mfma_rate()
    if rate:
        roofline["sustained_mfma"] = {
            "random_bf16_tflops": rate["random"]["tflops"], "random_ghz": rate["random"]["ghz"],
            "zero_bf16_tflops": rate["zero"]["tflops"], "zero_ghz": rate["zero"]["ghz"],
            "probe": "block_sparse_attention_pooled_amd/mfma_rate"}
        if attn_tflops:
            roofline["frac_of_sustained_random"] = round(attn_tflops / rate["random"]["tflops"], 4)
    # The path the K/V tiles take into each CU: at 64-token blocks as many
    # fill cycles per CU as matrix cycles per SIMD.
    paths = data_path_rates()
    if paths:
        roofline["data_path"] = data_path_block(paths, flops_step, inst_b, attn_ms)

    result = {
        "metric": (METRIC_COLS if args.columns else METRIC) if w.name == "stepdllm_8k" else
                  (f"{'column' if args.columns else 'block'}-sparse attn ms/step + effective "
                   f"TFLOP/s, {w.name} (L={w.L} H={w.H} Hkv={w.Hkv} d={w.d} B={w.B}, "
                   f"s={sparsity})"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "Hkv": w.Hkv, "L": w.L, "d": w.d, "block": w.B,
                   "sparsity": sparsity,
                   **({"kept_columns_per_head": drv.k_c} if args.columns
                      else {"kept_blocks": Kkept}),
                   "budget": ("columns" if args.columns else
                              "per_head" if args.per_head_budget else "global"),
                   "refresh_every": w.refresh_every, "dense_steps": w.dense_steps,
                   "distinct_input_steps": T, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kept_per_head": {"min": min(per_head), "max": max(per_head),
                          "cv": round(ph_cv, 4)},
        **temperature_trend(w, per_head, args),
        "empty_rows": (None if args.columns else
                       int((drv.row_ptr[1:] == drv.row_ptr[:-1]).sum().item())),
        **({} if args.columns or args.per_head_budget else near_ties(drv, w, dims)),
        "timed_window": {"first_step": start % T, "anchor_steps": n_anchor,
                         "dense_steps": sum(1 for kd in kinds if kd == 0),
                         "reuse_steps": sum(1 for kd in kinds if kd == 2)},
        "anchor_step_ms": round(anchor_ms, 5) if anchor_ms else None,
        "mask_build_ms": round(anchor_ms - attn_ms, 5) if (anchor_ms and attn_ms) else None,
        **mask_build_bandwidth(w, anchor_ms, attn_ms, args.columns),
        "anchors_timed": n_anchor,
        "ms_per_step_refresh_interval": round(interval_ms, 5) if interval_ms else None,
        "dense_step_ms": round(dense_step_ms, 5) if dense_step_ms else None,
        "dense_kernel_ms": round(dense_ms, 5),
        "dense_kernel_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 3),
        "dense_kernel_frac": round(dense_flops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "speedup_vs_dense_kernel": round(dense_ms / attn_ms, 3) if attn_ms else None,
        "speedup_vs_dense_per_step": round(dense_ms / ms_per_step, 3),
        **({"runs_ms_per_step": [round(x * 1e3 / K_steps, 5) for x in walls]}
           if len(walls) > 1 else {}),
        "step_roofline": (None if args.columns else
                          {"ideal_ms_per_step": round(ideal_ms_step, 5),
                           "frac": round(ideal_ms_step / ms_per_step, 4)}),
    }
    if not args.no_cpu_baseline and args.columns:
        result["cpu_baseline"] = cpu_baseline_cols(inputs[0], w, sparsity, flops_step,
                                                   args.cpu_budget_s)
    elif not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inputs[0], w, sparsity, flops_step, args.cpu_budget_s,
                                              per_head=args.per_head_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
