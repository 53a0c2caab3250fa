"""Full-size workloads through the step driver, against the oracle.

Masks are compared in full at the anchors (bit-exact except scores within 1e-5
of the cut, which are listed); outputs on sampled rows the oracle computes one
by one (all rows of some heads, the longest lists, seeded random rows), in the
launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_anchor(drv, w, sparsity, q, k, label):
    """Mask built by the driver at an anchor vs the oracle's, plus the oracle's
    select on the GPU's own scores (exact)."""
    qf, kf = PT.oracle_inputs(q, k)
    ref = O.build_mask(qf, kf, w.B, sparsity)
    K = ref["K"]
    assert K == drv.K
    rp = drv.row_ptr.cpu().numpy()
    ci = drv.col_idx[:K].cpu().numpy()
    PT.check_csr_form(rp, ci, K, w.nb)
    keep = PT.keep_from_csr(rp, ci, w.H, w.nb)
    keep_ref = PT.keep_from_csr(ref["row_ptr"], ref["col_idx"], w.H, w.nb)
    listed = PT.compare_masks(keep, keep_ref, ref["P"], K)
    # The GPU's own scores (left in the workspace) select exactly the GPU mask.
    lay = B.workspace_layout(drv.dims)
    P_gpu = drv.ws[lay.scores:lay.scores + 4 * w.H * w.nb * w.nb].view(torch.float32)
    P_gpu = P_gpu.cpu().numpy().reshape(w.H, w.nb, w.nb)
    assert np.array_equal(O.select(P_gpu, K), keep)
    rel = float(np.max(np.abs(P_gpu.astype(np.float64) - ref["P"]) / ref["P"]))
    assert rel <= PT.score_rel_bound(w.nb), rel
    work_ref, n_ref = O.plan(rp, w.H, w.nb, w.B)
    work = drv.ws[lay.work:lay.work + 4 * work_ref.size].view(torch.int32).cpu().numpy()
    assert np.array_equal(work, work_ref)
    print(f"{label}: K={K} near-tie differences={len(listed)} {listed[:8]} "
          f"empty rows={int((np.diff(rp) == 0).sum())} max score rel diff={rel:.2e}", flush=True)
    return rp, ci


def _check_rows(o, q, k, v, w, rp, ci, rows, label):
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    out = np.zeros(qf.shape, np.float64)
    PT.oracle_rows_parallel(O.sparse_attn, rows, q=qf, k=kf, v=vf, B=w.B, row_ptr=rp,
                            col_idx=ci, out=out)
    sel = PT.token_mask_for_rows(rows, w.H, w.nb, w.B)
    stats = PT.check_outputs(o, out, sel)
    print(f"{label}: {len(rows)} rows {stats}", flush=True)


def _run(w, sparsity, last_step, mask_steps, out_steps, heads=(0,)):
    traj = Trajectory(w, DEV)
    dims = B.make_dims(w.H, w.Hkv, w.L, w.d, w.B)
    drv = B.Driver(dims, w.dense_steps, w.refresh_every, sparsity, device=DEV)
    o = torch.empty(w.H, w.L, w.d, dtype=torch.bfloat16, device=DEV)
    rp = ci = None
    for t in range(last_step + 1):
        q, k, v = traj.next()
        kind = drv.step_kind(t)
        print(f"{w.name} s={sparsity} step {t} kind {kind}", flush=True)
        drv.step(t, q, k, v, o)
        torch.cuda.synchronize()
        if kind == 1:
            if t in mask_steps:
                rp, ci = _check_anchor(drv, w, sparsity, q, k, f"{w.name} anchor {t}")
            else:
                rp = drv.row_ptr.cpu().numpy()
                ci = drv.col_idx[:drv.K].cpu().numpy()
        if t in out_steps:
            if kind == 0:
                qf, kf, vf = PT.oracle_inputs(q, k, v)
                rows = np.array([0, w.rows // 3, w.rows - 1, w.nb + 1], np.int32)
                out = np.zeros(qf.shape, np.float64)
                PT.oracle_rows_parallel(O.dense_attn, rows, q=qf, k=kf, v=vf, B=w.B, out=out)
                stats = PT.check_outputs(o, out, PT.token_mask_for_rows(rows, w.H, w.nb, w.B))
                print(f"{w.name} dense step {t}: {stats}", flush=True)
            else:
                rows = PT.sample_rows(rp, w.H, w.nb, heads=heads, seed=t)
                _check_rows(o, q, k, v, w, rp, ci, rows, f"{w.name} step {t}")


@pytest.mark.timeout(600)
def test_llada_2k():
    w = WORKLOADS["llada_2k"]
    _run(w, w.sparsities[0], 7, mask_steps={0}, out_steps={0, 7}, heads=range(w.H))


@pytest.mark.timeout(900)
def test_stepdllm_8k_anchors_and_resample():
    """The whole 256-step trajectory: the mask at all 8 anchors (the Q/K
    redraws at 64 and 160 included), outputs at the first step, the last
    step before the first refresh, both redraws and the last step."""
    w = WORKLOADS["stepdllm_8k"]
    _run(w, w.sparsities[0], 255, mask_steps=set(range(0, 256, 32)),
         out_steps={0, 31, 64, 160, 255}, heads=(0, 17))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("sparsity", WORKLOADS["dream_gqa_8k"].sparsities)
def test_dream_gqa_8k(sparsity):
    """64 steps per sparsity: the mask at its 4 anchors, outputs at the first
    and last steps."""
    w = WORKLOADS["dream_gqa_8k"]
    _run(w, sparsity, 63, mask_steps={0, 16, 32, 48}, out_steps={0, 63}, heads=(0, 6, 7))


@pytest.mark.timeout(900)
def test_long_64k_dense_then_sparse():
    w = WORKLOADS["long_64k"]
    _run(w, w.sparsities[0], 127, mask_steps={26}, out_steps={0, 26, 27, 127}, heads=())


@pytest.mark.timeout(900)
def test_stepdllm_8k_structured_across_a_redraw():
    """Block-structured inputs (concentrated attention); Q/K are redrawn at
    step 80, inside the interval of the anchor at 64, so step 95 runs on a
    stale mask and step 96 rebuilds it."""
    w = WORKLOADS["stepdllm_8k_structured"]
    _run(w, w.sparsities[0], 96, mask_steps={0, 96}, out_steps={0, 95, 96}, heads=(0, 5))
