"""Per-kernel parity of the HIP library against the oracle, through the C ABI,
at sizes the oracle finishes in seconds (several tiles plus ragged tails)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (H, Hkv, L, d, block, q_scale): tiles + ragged block counts (nb = 37, 5, 33, 1).
SHAPES = [
    (2, 2, 256, 64, 64, 1.0),
    (4, 2, 37 * 64, 128, 64, 2.0),
    (3, 1, 5 * 128, 64, 128, 1.5),
    (2, 2, 33 * 64, 128, 64, 3.0),
    (4, 4, 128, 128, 128, 1.0),
    (7, 7, 3 * 128, 128, 128, 0.7),
    (6, 2, 6 * 64, 128, 64, 1.2),      # GQA, 64-token blocks, L a multiple of 128
]
SHAPE_IDS = [f"H{s[0]}kv{s[1]}L{s[2]}d{s[3]}B{s[4]}" for s in SHAPES]


def _qkv(shape, seed):
    H, Hkv, L, d, blk, qs = shape
    return random_qkv(H, Hkv, L, d, seed, device=DEV, q_scale=qs, sinks=True)


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_pool_bit_exact_and_scores_close(shape):
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 101)
    m = PT.GpuMask(q, k, blk, 0.5)
    qf, kf = PT.oracle_inputs(q, k)
    qb_ref, kb_ref = O.pool(qf, blk), O.pool(kf, blk)
    qb, kb = m.buf.pooled()
    # Block sums run in the same ascending order on both sides: identical bits.
    assert np.array_equal(qb.cpu().numpy().reshape(qb_ref.shape), qb_ref)
    assert np.array_equal(kb.cpu().numpy().reshape(kb_ref.shape), kb_ref)
    P_ref = O.scores(qb_ref, kb_ref)
    P = m.P()
    assert np.array_equal(P, m.buf.scores().cpu().numpy().reshape(P.shape))
    rel = np.max(np.abs(P.astype(np.float64) - P_ref) / P_ref)
    print(f"max relative score difference {rel:.3g} (bound {PT.score_rel_bound(m.nb):.3g})")
    assert rel <= PT.score_rel_bound(m.nb), rel


@pytest.mark.parametrize("s", [0.0, 0.5, 0.9, 0.97])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_selection_bit_exact_on_gpu_scores(shape, s):
    """The oracle's select run on the GPU's own scores gives exactly the GPU mask."""
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 202)
    m = PT.GpuMask(q, k, blk, s)
    P = m.P()
    K = O.keep_count(P.size, s)
    assert K == m.K
    rp, ci = m.csr()
    PT.check_csr_form(rp, ci, K, m.nb)
    keep_ref = O.select(P, K)
    assert np.array_equal(m.keep(), keep_ref)
    rp_ref, ci_ref = O.csr(keep_ref)
    assert np.array_equal(rp, rp_ref) and np.array_equal(ci, ci_ref)
    # Select state: cut key is the K-th largest's bits, count above + ties kept = K.
    st = m.buf.select_state().cpu().numpy().view(np.uint32)
    if K > 0:
        cut = np.float32(O.cut_value(P, K))
        assert st[0] == (cut.view(np.uint32) | np.uint32(0x80000000))
        assert int(st[1]) == int((P > cut).sum())
        assert int(st[1]) + int(st[2]) == K


def _tie_scores(H, nb, levels, seed):
    rng = np.random.default_rng(seed)
    lv = np.sort(rng.random(levels)).astype(np.float32)
    return lv[rng.integers(0, levels, size=(H, nb, nb))]


@pytest.mark.parametrize("case", [
    ("few_levels", 4, 9, 3), ("many_ties", 2, 64, 2), ("all_equal", 3, 16, 1),
    ("one_block", 5, 1, 2), ("ragged", 6, 70, 50),
])
@pytest.mark.parametrize("s", [0.0, 0.25, 0.5, 0.9, 0.999999])
def test_selection_on_injected_scores(case, s):
    name, H, nb, levels, = case[0], case[1], case[2], case[3]
    P = _tie_scores(H, nb, levels, 7 + nb)
    dims = B.make_dims(H, H, nb * 64, 64, 64)
    buf = B.MaskBuffers(dims, s, device=DEV)
    B.select_mask(dims, s, torch.from_numpy(P.reshape(-1)).to(DEV), buf.ws, buf.row_ptr,
                  buf.col_idx)
    torch.cuda.synchronize()
    K = O.keep_count(P.size, s)
    assert K == buf.K
    rp = buf.row_ptr.cpu().numpy()
    ci = buf.col_idx[:K].cpu().numpy()
    PT.check_csr_form(rp, ci, K, nb)
    assert np.array_equal(PT.keep_from_csr(rp, ci, H, nb), O.select(P, K)), name


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_plan_matches_oracle(shape):
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 303)
    m = PT.GpuMask(q, k, blk, 0.8)
    rp, ci = m.csr()
    meta = m.buf.work_meta().cpu().numpy()
    work_ref, n_ref = O.plan(rp, H, L // blk, blk)
    assert np.array_equal(m.buf.work().cpu().numpy(), work_ref)
    assert int(meta[0]) * 8 == work_ref.size and int(meta[1]) == n_ref
    _check_records(m.buf.work_rec().cpu().numpy(), work_ref, rp, ci)


@pytest.mark.parametrize("s", [0.0, 0.5, 0.93, 1.0])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_mask_build_plan_equals_plan_launch(shape, s):
    """The global-budget mask build plans from the records and head counts
    its list launch wrote (one launch, every workgroup redoing the die part);
    a separate plan launch on the lists it wrote (die part, then rows) gives
    the same work order, records and meta words, including K = 0 and every
    block kept."""
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 505)
    m = PT.GpuMask(q, k, blk, s)
    fused = (m.buf.work().clone(), m.buf.work_rec().clone(), m.buf.work_meta()[:8].clone())
    B.plan(m.dims, m.buf.row_ptr, m.buf.col_idx, m.buf.ws, nnz=m.K)
    torch.cuda.synchronize()
    assert torch.equal(fused[0], m.buf.work())
    assert torch.equal(fused[1], m.buf.work_rec())
    assert torch.equal(fused[2], m.buf.work_meta()[:8])


@pytest.mark.parametrize("H", [255, 256, 257, 300])
def test_mask_build_plan_many_heads(H):
    """Around the one-launch plan's head limit (256; past it the mask build
    plans in two launches): the oracle's work order and records, and the
    same order from a separate plan launch."""
    shape = (H, H, 3 * 64, 64, 64, 1.0)
    q, k, v = _qkv(shape, 707)
    m = PT.GpuMask(q, k, 64, 0.7)
    rp, ci = m.csr()
    work_ref, n_ref = O.plan(rp, H, 3, 64)
    work = m.buf.work().cpu().numpy()
    assert np.array_equal(work, work_ref)
    assert int(m.buf.work_meta().cpu().numpy()[1]) == n_ref
    _check_records(m.buf.work_rec().cpu().numpy(), work_ref, rp, ci)
    fused = (m.buf.work_rec().clone(), m.buf.work_meta()[:8].clone())
    B.plan(m.dims, m.buf.row_ptr, m.buf.col_idx, m.buf.ws, nnz=m.K)
    torch.cuda.synchronize()
    assert np.array_equal(m.buf.work().cpu().numpy(), work)
    assert torch.equal(fused[0], m.buf.work_rec())
    assert torch.equal(fused[1], m.buf.work_meta()[:8])


@pytest.mark.parametrize("H,nb,blk", [(64, 320, 64), (28, 129, 128), (3, 1024, 64), (13, 7, 128)])
def test_plan_many_rows_and_lengths(H, nb, blk):
    """Injected lists with every length 0..nb, ragged head counts per die."""
    rng = np.random.default_rng(9)
    lens = rng.integers(0, nb + 1, size=H * nb)
    lens[rng.random(H * nb) < 0.3] = 0
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = rng.integers(0, nb, size=max(int(rp[-1]), 1)).astype(np.int32)
    dims = B.make_dims(H, H, nb * blk, 64, blk)
    buf = B.MaskBuffers(dims, 0.5, device=DEV)
    B.plan(dims, torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV), buf.ws,
           nnz=int(rp[-1]))
    torch.cuda.synchronize()
    work_ref, n_ref = O.plan(rp, H, nb, blk)
    assert np.array_equal(buf.work().cpu().numpy(), work_ref)
    assert int(buf.work_meta().cpu().numpy()[1]) == n_ref
    _check_records(buf.work_rec().cpu().numpy(), work_ref, rp, ci)


def _check_records(rec, work, rp, ci):
    """Each work position's record: row, list bounds, first two block ids
    (16 bits each, 0 past the list); padding has row -1 and zeros."""
    assert rec.shape == (work.size, 4)
    assert np.array_equal(rec[:, 0], work)
    pad = work < 0
    assert np.all(rec[pad, 1:] == 0)
    rows = work[~pad]
    lo, hi = rp[rows], rp[rows + 1]
    assert np.array_equal(rec[~pad, 1], lo) and np.array_equal(rec[~pad, 2], hi)
    ci_pad = np.concatenate([ci, [0, 0]])
    id0 = np.where(hi > lo, ci_pad[lo], 0)
    id1 = np.where(hi > lo + 1, ci_pad[np.minimum(lo + 1, ci_pad.size - 1)], 0)
    assert np.array_equal(rec[~pad, 3], id0 | (id1 << 16))


def _attn_case(shape, s, seed):
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, seed)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    ref = O.build_mask(qf, kf, blk, s)
    return q, k, v, qf, kf, vf, ref


@pytest.mark.parametrize("s", [0.5, 0.9])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_sparse_attention_on_oracle_mask(shape, s):
    H, Hkv, L, d, blk, _ = shape
    q, k, v, qf, kf, vf, ref = _attn_case(shape, s, 404)
    dims = B.dims_of(q, k, blk)
    buf = B.MaskBuffers(dims, s, device=DEV)
    rp = torch.from_numpy(ref["row_ptr"]).to(DEV)
    ci = torch.from_numpy(np.concatenate([ref["col_idx"], [0]]).astype(np.int32)).to(DEV)
    B.plan(dims, rp, ci, buf.ws, nnz=ref["K"])
    o = torch.full_like(q, float("nan"))
    B.sparse_attn(dims, q, k, v, ci, buf.ws, o, nnz=ref["K"])
    torch.cuda.synchronize()
    o_ref = O.sparse_attn(qf, kf, vf, blk, ref["row_ptr"], ref["col_idx"])
    PT.check_outputs(o, o_ref)


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_dense_attention(shape):
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 505)
    dims = B.dims_of(q, k, blk)
    o = torch.full_like(q, float("nan"))
    B.dense_attn(dims, q, k, v, o)
    torch.cuda.synchronize()
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    PT.check_outputs(o, O.dense_attn(qf, kf, vf, blk))


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_sparsity_zero_equals_dense(shape):
    """s = 0 keeps every block; the sparse kernel then runs the dense kernel's
    exact operation sequence."""
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 606)
    dims = B.dims_of(q, k, blk)
    buf = B.MaskBuffers(dims, 0.0, device=DEV)
    B.build_mask(dims, 0.0, q, k, buf.ws, buf.row_ptr, buf.col_idx)
    o_s, o_d = torch.empty_like(q), torch.empty_like(q)
    B.sparse_attn(dims, q, k, v, buf.col_idx, buf.ws, o_s)
    B.dense_attn(dims, q, k, v, o_d)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d)


@pytest.mark.timeout(600)
def test_largest_block_count():
    """nb = 1024, the most the library takes (L = 65536 in 64-token blocks),
    with GQA: the mask build (each score workgroup holds 16 rows of 1024
    scores in LDS), the plan records and the sparse attention on sampled rows
    against the oracle."""
    H, Hkv, L, d, blk, s = 2, 1, 65536, 128, 64, 0.9
    q, k, v = random_qkv(H, Hkv, L, d, 909, device=DEV, q_scale=2.0, sinks=True)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    ref = O.build_mask(qf, kf, blk, s)
    m = PT.GpuMask(q, k, blk, s)
    assert m.nb == 1024 and m.K == ref["K"]
    rp, ci = m.csr()
    PT.check_csr_form(rp, ci, m.K, m.nb)
    keep = m.keep()
    PT.compare_masks(keep, PT.keep_from_csr(ref["row_ptr"], ref["col_idx"], H, m.nb),
                     ref["P"], m.K)
    assert np.array_equal(O.select(m.P(), m.K), keep)
    lay = B.workspace_layout(m.dims)
    work_ref, _ = O.plan(rp, H, m.nb, blk)
    work = m.buf.ws[lay.work:lay.work + 4 * work_ref.size].view(torch.int32).cpu().numpy()
    assert np.array_equal(work, work_ref)
    o = torch.full_like(q, float("nan"))
    B.sparse_attn(m.dims, q, k, v, m.buf.col_idx, m.buf.ws, o, nnz=m.K)
    torch.cuda.synchronize()
    rows = PT.sample_rows(rp, H, m.nb, heads=(), seed=9)
    out = np.zeros(qf.shape, np.float64)
    PT.oracle_rows_parallel(O.sparse_attn, rows, q=qf, k=kf, v=vf, B=blk, row_ptr=rp,
                            col_idx=ci, out=out)
    PT.check_outputs(o, out, PT.token_mask_for_rows(rows, H, m.nb, blk))


def test_zero_budget_keeps_nothing():
    """s = 1 leaves K = 0: no digit pass runs, every row is empty, the plan's
    records have empty lists and the sparse launch writes zeros over the
    NaN-filled output."""
    H, Hkv, L, d, blk = 4, 2, 8 * 64, 64, 64
    s = 1.0
    q, k, v = _qkv((H, Hkv, L, d, blk, 1.0), 808)
    dims = B.dims_of(q, k, blk)
    nb = L // blk
    assert B.keep_count(dims, s) == 0 == O.keep_count(H * nb * nb, s)
    buf = B.MaskBuffers(dims, s, device=DEV)
    B.build_mask(dims, s, q, k, buf.ws, buf.row_ptr, buf.col_idx)
    o = torch.full_like(q, float("nan"))
    B.sparse_attn(dims, q, k, v, buf.col_idx, buf.ws, o, nnz=0)
    torch.cuda.synchronize()
    rp = buf.row_ptr.cpu().numpy()
    assert not rp.any()
    work_ref, n_ref = O.plan(rp, H, nb, blk)
    assert np.array_equal(buf.work().cpu().numpy(), work_ref) and n_ref == 0
    _check_records(buf.work_rec().cpu().numpy(), work_ref, rp, np.zeros(1, np.int32))
    assert torch.equal(o, torch.zeros_like(o))


def test_stale_plan_is_flagged():
    """A sparse launch checks the plan's tag.  On another col_idx array (same
    contents), another nnz, every row outputs zeros and bit 0 of the check
    word is set; with one row's first list entry rewritten in place after
    planning, that row outputs zeros, bit 1 is set and every other row is
    unchanged; a new plan clears the word and restores the output."""
    H, Hkv, L, d, blk = 4, 2, 8 * 64, 128, 64
    q, k, v = _qkv((H, Hkv, L, d, blk, 2.0), 515)
    m = PT.GpuMask(q, k, blk, 0.7)
    nb = L // blk
    ref = torch.empty_like(q)
    B.sparse_attn(m.dims, q, k, v, m.buf.col_idx, m.buf.ws, ref, nnz=m.K)
    torch.cuda.synchronize()
    assert m.buf.plan_check() == 0
    other = m.buf.col_idx.clone()
    o = torch.full_like(q, float("nan"))
    B.sparse_attn(m.dims, q, k, v, other, m.buf.ws, o, nnz=m.K)
    torch.cuda.synchronize()
    assert m.buf.plan_check() == 1
    assert torch.equal(o, torch.zeros_like(o))
    B.plan(m.dims, m.buf.row_ptr, other, m.buf.ws, nnz=m.K)
    o.fill_(float("nan"))
    B.sparse_attn(m.dims, q, k, v, other, m.buf.ws, o, nnz=m.K)
    torch.cuda.synchronize()
    assert m.buf.plan_check() == 0 and torch.equal(o, ref)
    o.fill_(float("nan"))
    B.sparse_attn(m.dims, q, k, v, other, m.buf.ws, o, nnz=m.K - 1)
    torch.cuda.synchronize()
    assert m.buf.plan_check() == 1 and torch.equal(o, torch.zeros_like(o))
    B.plan(m.dims, m.buf.row_ptr, other, m.buf.ws, nnz=m.K)
    rp, ci = m.csr()
    lens = np.diff(rp)
    r = int(np.argmax(lens))
    assert lens[r] >= 2 and lens[r] < nb
    ci2 = ci.copy()
    ci2[rp[r]] = int(np.setdiff1d(np.arange(nb), ci[rp[r]:rp[r + 1]])[0])
    other.copy_(torch.from_numpy(ci2))
    o.fill_(float("nan"))
    B.sparse_attn(m.dims, q, k, v, other, m.buf.ws, o, nnz=m.K)
    torch.cuda.synchronize()
    assert m.buf.plan_check() == 2
    h, i = divmod(r, nb)
    rows = o.view(H, nb, blk, d)
    assert torch.equal(rows[h, i], torch.zeros_like(rows[h, i]))
    keep = torch.ones(H, nb, dtype=torch.bool)
    keep[h, i] = False
    assert torch.equal(rows[keep], ref.view(H, nb, blk, d)[keep])


def test_dropped_block_is_detected():
    """Mutation: remove one kept block from the longest row of the mask given
    to the GPU; the comparison with the oracle on the full mask must fail."""
    shape = (4, 2, 16 * 64, 128, 64, 2.0)
    q, k, v, qf, kf, vf, ref = _attn_case(shape, 0.75, 707)
    blk = 64
    rp, ci = ref["row_ptr"].copy(), ref["col_idx"].copy()
    lens = np.diff(rp)
    r = int(np.argmax(lens))
    drop = rp[r] + lens[r] // 2
    ci_mut = np.delete(ci, drop)
    rp_mut = rp.copy()
    rp_mut[r + 1:] -= 1
    dims = B.dims_of(q, k, blk)
    buf = B.MaskBuffers(dims, 0.75, device=DEV)
    rpt = torch.from_numpy(rp_mut).to(DEV)
    cit = torch.from_numpy(ci_mut.astype(np.int32)).to(DEV)
    B.plan(dims, rpt, cit, buf.ws)
    o = torch.empty_like(q)
    B.sparse_attn(dims, q, k, v, cit, buf.ws, o)
    torch.cuda.synchronize()
    o_ref = O.sparse_attn(qf, kf, vf, blk, ref["row_ptr"], ref["col_idx"])
    with pytest.raises(AssertionError):
        PT.check_outputs(o, o_ref)
    # ... while the mutated mask itself is reproduced.
    PT.check_outputs(o, O.sparse_attn(qf, kf, vf, blk, rp_mut, ci_mut))


def test_worked_example_w1_on_gpu():
    import oracle_pins as pins
    q, k, v, keep_want = pins.worked_example_w1()
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in (q, k, v))
    m = PT.GpuMask(qd, kd, 64, 0.5)
    assert np.array_equal(m.keep(), keep_want)
    o = torch.empty_like(qd)
    B.sparse_attn(m.dims, qd, kd, vd, m.buf.col_idx, m.buf.ws, o)
    torch.cuda.synchronize()
    on = o.cpu().to(torch.float64).numpy()
    for i in range(4):
        want = v[0, i * 64:(i + 1) * 64].astype(np.float64).mean(axis=0)
        assert np.max(np.abs(on[0, i * 64:(i + 1) * 64] - want)) < 1e-2
    assert np.max(np.abs(on[1, :192] - v[1].astype(np.float64).mean(axis=0))) < 1e-2
    assert np.all(on[1, 192:] == 0)


def test_constant_values_and_zero_queries():
    """V = c gives O = c exactly on non-empty rows: the normaliser sums the
    same bf16-rounded weights that enter the value product, so O^T and l
    differ only by fp32 rounding (far below half a bf16 ulp of c = -1.5),
    and the bf16 output rounds back to c; Q = 0 gives the mean of V over the
    kept blocks."""
    H, Hkv, L, d, blk = 4, 2, 8 * 64, 128, 64
    q, k, v = random_qkv(H, Hkv, L, d, 808, device=DEV, q_scale=2.0)
    vc = torch.full_like(v, -1.5)
    m = PT.GpuMask(q, k, blk, 0.7)
    o = torch.empty_like(q)
    B.sparse_attn(m.dims, q, k, vc, m.buf.col_idx, m.buf.ws, o)
    torch.cuda.synchronize()
    nonempty = np.diff(m.csr()[0]) > 0
    on = o.cpu().to(torch.float32).numpy().reshape(H * (L // blk), blk, d)
    assert np.all(on[nonempty] == -1.5) and np.all(on[~nonempty] == 0)
    z = torch.zeros_like(q)
    B.sparse_attn(m.dims, z, k, v, m.buf.col_idx, m.buf.ws, o)
    torch.cuda.synchronize()
    qf, kf, vf = PT.oracle_inputs(z, k, v)
    rp, ci = m.csr()
    PT.check_outputs(o, O.sparse_attn(qf, kf, vf, blk, rp, ci))


def test_determinism():
    shape = (4, 2, 37 * 64, 128, 64, 2.0)
    q, k, v = _qkv(shape, 909)
    outs = []
    for _ in range(2):
        m = PT.GpuMask(q, k, 64, 0.9)
        o = torch.empty_like(q)
        B.sparse_attn(m.dims, q, k, v, m.buf.col_idx, m.buf.ws, o)
        torch.cuda.synchronize()
        outs.append((m.P(), m.csr(), m.buf.work().cpu().numpy(), o.cpu()))
    a, b = outs
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1][0], b[1][0]) and np.array_equal(a[1][1], b[1][1])
    assert np.array_equal(a[2], b[2]) and torch.equal(a[3], b[3])


def test_tiny_workload_end_to_end():
    """The tiny workload: one anchor step, mask and outputs against the oracle."""
    w = WORKLOADS["tiny"]
    q, k, v = Trajectory(w, DEV).next()
    drv = B.Driver(B.dims_of(q, k, w.B), w.dense_steps, w.refresh_every, w.sparsities[0])
    o = torch.empty_like(q)
    drv.step(0, q, k, v, o)
    torch.cuda.synchronize()
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    ref = O.build_mask(qf, kf, w.B, w.sparsities[0])
    keep = PT.keep_from_csr(drv.row_ptr.cpu().numpy(), drv.col_idx[:drv.K].cpu().numpy(),
                            w.H, w.nb)
    PT.compare_masks(keep, O.select(ref["P"], ref["K"]), ref["P"], ref["K"])
    PT.check_outputs(o, O.sparse_attn(qf, kf, vf, w.B, ref["row_ptr"], ref["col_idx"]))
    o_d = torch.empty_like(q)
    B.dense_attn(drv.dims, q, k, v, o_d)
    torch.cuda.synchronize()
    PT.check_outputs(o_d, O.dense_attn(qf, kf, vf, w.B))


@pytest.mark.parametrize("sign", [1.0, -1.0], ids=["rising", "falling"])
@pytest.mark.parametrize("d,blk", [(128, 64), (64, 128)])
def test_scores_moving_past_the_rescale_margin(d, blk, sign):
    """Every key shares one direction with every query and its score moves by
    about 0.45 natural units per key, about 21 log2 units per 32-key chunk.
    That is past the lazy rescale's margin of 8, so with rising scores the
    running max moves at every chunk of every row and O and the normaliser
    are rescaled each time, by factors down to about 2^-21 per chunk.  With
    falling scores the first chunk holds the max and every later weight
    underflows.  Sparse and dense, against the oracle.  The sparse mask is the
    library's at s = 0.5.  Most pooled scores underflow to exact zeros, so the
    ties at zero fill the budget in flat order: the first rows keep every
    block, and the others keep their few nonzero blocks."""
    H, Hkv, L = 2, 2, 1024
    g = torch.Generator().manual_seed(1212)
    e = torch.ones(d, dtype=torch.float64) / math.sqrt(d)
    a = sign * 0.45 * math.sqrt(d) / 4.0 * torch.arange(L, dtype=torch.float64)
    q = 4.0 * e.expand(H, L, d) + 0.05 * torch.randn(H, L, d, generator=g, dtype=torch.float64)
    k = a.view(1, L, 1) * e.view(1, 1, d) + 0.05 * torch.randn(Hkv, L, d, generator=g,
                                                                dtype=torch.float64)
    v = torch.randn(Hkv, L, d, generator=g, dtype=torch.float64)
    q, k, v = (x.to(torch.bfloat16).to(DEV) for x in (q, k, v))
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    m = PT.GpuMask(q, k, blk, 0.5)
    o = torch.full_like(q, float("nan"))
    B.sparse_attn(m.dims, q, k, v, m.buf.col_idx, m.buf.ws, o)
    torch.cuda.synchronize()
    rp, ci = m.csr()
    PT.check_outputs(o, O.sparse_attn(qf, kf, vf, blk, rp, ci))
    od = torch.full_like(q, float("nan"))
    B.dense_attn(m.dims, q, k, v, od)
    torch.cuda.synchronize()
    PT.check_outputs(od, O.dense_attn(qf, kf, vf, blk))
