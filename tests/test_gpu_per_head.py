"""The uniform per-head budget (each head keeps its own ceil((1-s)*nb^2)
largest pooled scores) on the GPU against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [
    (2, 2, 256, 64, 64, 1.0),
    (4, 2, 37 * 64, 128, 64, 2.0),
    (3, 1, 5 * 128, 64, 128, 1.5),
    (7, 7, 3 * 128, 128, 128, 0.7),
]
SHAPE_IDS = [f"H{s[0]}kv{s[1]}L{s[2]}d{s[3]}B{s[4]}" for s in SHAPES]


def _qkv(shape, seed):
    H, Hkv, L, d, blk, qs = shape
    return random_qkv(H, Hkv, L, d, seed, device=DEV, q_scale=qs, sinks=True)


def _compare_per_head(keep, keep_ref, P_ref, k_h):
    """Masks agree head by head, except at oracle scores within rounding of that
    head's own cut."""
    listed = []
    for h in range(keep.shape[0]):
        listed += PT.compare_masks(keep[h:h + 1], keep_ref[h:h + 1], P_ref[h:h + 1], k_h)
    return listed


def _check_head_state(state, P, k_h):
    """Per-head select state: cut key of the k_h-th largest, count above, ties."""
    H = P.shape[0]
    st = state.reshape(H, 8).view(np.uint32)
    for h in range(H):
        if k_h == 0:
            assert st[h, 2] == 0 and st[h, 3] == 0
            continue
        vals = np.sort(P[h].reshape(-1))[::-1]
        cut = np.float32(vals[k_h - 1])
        assert st[h, 0] == (cut.view(np.uint32) | np.uint32(0x80000000)), h
        assert int(st[h, 1]) == int((P[h] > cut).sum())
        assert int(st[h, 1]) + int(st[h, 2]) == k_h == int(st[h, 3])


@pytest.mark.parametrize("s", [0.0, 0.5, 0.9, 0.97])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_per_head_selection_bit_exact_on_gpu_scores(shape, s):
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 212)
    m = PT.GpuMask(q, k, blk, s, per_head=True)
    P = m.P()
    k_h = O.keep_count(m.nb * m.nb, s)
    assert m.K == H * k_h
    rp, ci = m.csr()
    PT.check_csr_form(rp, ci, m.K, m.nb)
    keep_ref = O.select_per_head(P, k_h)
    assert np.array_equal(m.keep(), keep_ref)
    assert np.all(m.keep().reshape(H, -1).sum(axis=1) == k_h)
    rp_ref, ci_ref = O.csr(keep_ref)
    assert np.array_equal(rp, rp_ref) and np.array_equal(ci, ci_ref)
    _check_head_state(m.buf.head_select().cpu().numpy(), P, k_h)
    # The work order is the usual plan of this mask.
    work_ref, n_ref = O.plan(rp, H, m.nb, blk)
    assert np.array_equal(m.buf.work().cpu().numpy(), work_ref)


def _tie_scores(H, nb, levels, seed):
    rng = np.random.default_rng(seed)
    lv = np.sort(rng.random(levels)).astype(np.float32)
    return lv[rng.integers(0, levels, size=(H, nb, nb))]


@pytest.mark.parametrize("case", [
    ("few_levels", 4, 9, 3), ("many_ties", 2, 64, 2), ("all_equal", 3, 16, 1),
    ("one_block", 5, 1, 2), ("ragged", 6, 70, 50), ("big_head", 2, 1024, 7),
])
@pytest.mark.parametrize("s", [0.0, 0.25, 0.5, 0.9, 0.999999])
def test_per_head_selection_on_injected_scores(case, s):
    name, H, nb, levels = case
    P = _tie_scores(H, nb, levels, 17 + nb)
    dims = B.make_dims(H, H, nb * 64, 64, 64)
    buf = B.MaskBuffers(dims, s, device=DEV, per_head=True)
    B.select_mask(dims, s, torch.from_numpy(P.reshape(-1)).to(DEV), buf.ws, buf.row_ptr,
                  buf.col_idx, per_head=True)
    torch.cuda.synchronize()
    k_h = O.keep_count(nb * nb, s)
    assert buf.K == H * k_h
    rp = buf.row_ptr.cpu().numpy()
    ci = buf.col_idx[:buf.K].cpu().numpy()
    PT.check_csr_form(rp, ci, buf.K, nb)
    assert np.array_equal(PT.keep_from_csr(rp, ci, H, nb), O.select_per_head(P, k_h)), name
    _check_head_state(buf.head_select().cpu().numpy(), P, k_h)


@pytest.mark.parametrize("s", [0.5, 0.9])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_per_head_driver_step_matches_oracle(shape, s):
    """Anchor step through the driver with the per-head budget, element by
    element against the oracle on the same mask."""
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 313)
    dims = B.dims_of(q, k, blk)
    drv = B.Driver(dims, 0, 4, s, device=DEV, per_head_budget=True)
    o = torch.empty_like(q)
    drv.step(0, q, k, v, o)
    torch.cuda.synchronize()
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    ref = O.build_mask(qf, kf, blk, s, per_head=True)
    assert ref["K"] == drv.K
    nb = L // blk
    rp = drv.row_ptr.cpu().numpy()
    ci = drv.col_idx[:drv.K].cpu().numpy()
    PT.check_csr_form(rp, ci, drv.K, nb)
    keep = PT.keep_from_csr(rp, ci, H, nb)
    # Masks agree except where the pooled scores sit within rounding of the cut.
    listed = _compare_per_head(keep, PT.keep_from_csr(ref["row_ptr"], ref["col_idx"], H, nb),
                               ref["P"], drv.K // H)
    assert len(listed) <= 2, listed
    out = O.sparse_attn(qf, kf, vf, blk, rp, ci)
    PT.check_outputs(o, out, np.ones((H, L), bool))
    # A reuse step keeps the mask.
    drv.step(1, q, k, v, o)
    torch.cuda.synchronize()
    PT.check_outputs(o, out, np.ones((H, L), bool))


@pytest.mark.timeout(900)
def test_per_head_budget_8k_anchor():
    """The 8K workload's first anchor under the uniform budget: full mask
    against the oracle and sampled rows of the attention."""
    w = WORKLOADS["stepdllm_8k"]
    s = w.sparsities[0]
    traj = Trajectory(w, DEV)
    q, k, v = traj.next()
    dims = B.make_dims(w.H, w.Hkv, w.L, w.d, w.B)
    drv = B.Driver(dims, w.dense_steps, w.refresh_every, s, device=DEV, per_head_budget=True)
    o = torch.empty_like(q)
    drv.step(0, q, k, v, o)
    torch.cuda.synchronize()
    qf, kf = PT.oracle_inputs(q, k)
    ref = O.build_mask(qf, kf, w.B, s, per_head=True)
    assert ref["K"] == drv.K == w.H * O.keep_count(w.nb * w.nb, s)
    rp = drv.row_ptr.cpu().numpy()
    ci = drv.col_idx[:drv.K].cpu().numpy()
    PT.check_csr_form(rp, ci, drv.K, w.nb)
    keep = PT.keep_from_csr(rp, ci, w.H, w.nb)
    keep_ref = PT.keep_from_csr(ref["row_ptr"], ref["col_idx"], w.H, w.nb)
    listed = _compare_per_head(keep, keep_ref, ref["P"], drv.K // w.H)
    per_head = keep.reshape(w.H, -1).sum(axis=1)
    assert np.all(per_head == O.keep_count(w.nb * w.nb, s))
    print(f"per-head anchor: K={drv.K} near-tie differences={len(listed)}", flush=True)
    rows = PT.sample_rows(rp, w.H, w.nb, heads=(0, 9), seed=3)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    out = np.zeros(qf.shape, np.float64)
    PT.oracle_rows_parallel(O.sparse_attn, rows, q=qf, k=kf, v=vf, B=w.B, row_ptr=rp,
                            col_idx=ci, out=out)
    stats = PT.check_outputs(o, out, PT.token_mask_for_rows(rows, w.H, w.nb, w.B))
    print(f"per-head anchor: {len(rows)} rows {stats}", flush=True)
