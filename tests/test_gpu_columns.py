"""The column-sparse variant on the GPU against the oracle, through the C ABI:
column masses of the pooled queries, the per-head column select, column-sparse
attention (gathered key columns, ragged last chunk) and the driver's column
mode."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as pins
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
    (8, 8, 41 * 64, 128, 64, 3.0),     # 41 pooled queries: a ragged 32-query tile
    (2, 2, 160 * 64, 64, 64, 1.0),     # 5 tiles: a second group of four with one tile
]
SHAPE_IDS = [f"H{s[0]}kv{s[1]}L{s[2]}d{s[3]}B{s[4]}" for s in SHAPES]

# Masses: fp32 scores from exact bf16 products, fp32 exp2 and sums against the
# fp64 definition on the same bf16-rounded pooled queries.
MASS_REL, MASS_ABS = 1e-4, 1e-9


def _qkv(shape, seed):
    H, Hkv, L, d, blk, qs = shape
    return random_qkv(H, Hkv, L, d, seed, device=DEV, q_scale=qs, sinks=True)


class GpuCols:
    """Build the column mask of (q, k) on the GPU and fetch the outputs."""

    def __init__(self, q, k, blk, sparsity):
        self.dims = B.dims_of(q, k, blk)
        self.H, self.L = q.shape[0], q.shape[1]
        self.k_c = B.keep_count_columns(self.dims, sparsity)
        self.ws = torch.empty(B.workspace_bytes(self.dims), dtype=torch.uint8, device=DEV)
        self.buf = torch.empty(max(self.H * self.k_c, 1), dtype=torch.int32, device=DEV)
        self.c = torch.empty(self.H * self.L, dtype=torch.float32, device=DEV)
        B.build_col_mask(self.dims, sparsity, q, k, self.ws, self.buf, self.c)
        torch.cuda.synchronize()

    def cols_t(self):
        return self.buf[:self.H * self.k_c].view(self.H, self.k_c)

    def cols(self):
        return self.cols_t().cpu().numpy()

    def scores(self):
        return self.c.cpu().numpy().reshape(self.H, self.L)


def _check_cols_form(cols, k_c, L):
    assert cols.shape[1] == k_c
    assert np.all((cols >= 0) & (cols < L))
    assert np.all(np.diff(cols, axis=1) > 0)


def _compare_cols(cols_gpu, cols_ref, c_ref, k_c):
    """Per head, equal kept sets except at oracle masses within rounding of
    that head's cut; returns the listed near-ties."""
    H, L = c_ref.shape
    listed = []
    for h in range(H):
        kg = np.zeros((1, L), np.uint8)
        kr = np.zeros((1, L), np.uint8)
        kg[0, cols_gpu[h]] = 1
        kr[0, cols_ref[h]] = 1
        listed += [(h,) + t for t in PT.compare_masks(kg, kr, c_ref[h:h + 1], k_c)]
    return listed


def _check_mass(got, want):
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= MASS_ABS + MASS_REL * want), float((err / want).max())


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_column_masses_match_oracle(shape):
    H, Hkv, L, d, blk, _ = shape
    q, k, _ = _qkv(shape, 611)
    m = GpuCols(q, k, blk, 0.9)
    qf, kf = PT.oracle_inputs(q, k)
    want = O.col_scores(qf, kf, blk)
    got = m.scores()
    _check_mass(got, want)
    assert np.max(np.abs(got.sum(axis=1) - 1.0)) < 1e-4
    # Deterministic: a second build gives the same bits.
    m2 = GpuCols(q, k, blk, 0.9)
    assert torch.equal(m.c, m2.c) and torch.equal(m.cols_t(), m2.cols_t())


@pytest.mark.parametrize("s", [0.0, 0.5, 0.9, 0.97])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_column_selection_bit_exact_on_gpu_masses(shape, s):
    H, Hkv, L, d, blk, _ = shape
    q, k, _ = _qkv(shape, 612)
    m = GpuCols(q, k, blk, s)
    assert m.k_c == O.keep_count(L, s)
    cols = m.cols()
    _check_cols_form(cols, m.k_c, L)
    # The oracle's select on the GPU's own masses gives the same lists.
    assert np.array_equal(cols, O.col_select(m.scores(), m.k_c))
    # Against the oracle's whole pipeline: equal except within rounding of a cut.
    qf, kf = PT.oracle_inputs(q, k)
    c_ref, cols_ref, k_c = O.build_col_mask(qf, kf, blk, s)
    assert k_c == m.k_c
    listed = _compare_cols(cols, cols_ref, c_ref, k_c)
    assert len(listed) <= 2, listed


@pytest.mark.parametrize("H,L,blk", [(3, 256, 64), (2, 8192, 64), (5, 320 * 64, 64)])
def test_column_select_on_injected_ties(H, L, blk):
    """Masses with massive exact ties: the kept set is the top-k_c under (value
    descending, column ascending) for k_c from 0 to L, including the chunk
    edges 31, 32, 33."""
    dims = B.make_dims(H, H, L, 64, blk)
    rng = np.random.default_rng(L + H)
    vals = (rng.integers(0, 7, size=(H, L)) / 8.0).astype(np.float32)
    vals[0] = rng.random(L).astype(np.float32)
    ws = torch.empty(B.workspace_bytes(dims), dtype=torch.uint8, device=DEV)
    sc = torch.from_numpy(vals.reshape(-1)).to(DEV)
    for want_k in (0, 1, 31, 32, 33, L // 3, L - 1, L):
        s = (L - want_k) / L
        k_c = B.keep_count_columns(dims, s)
        assert k_c == want_k
        buf = torch.full((max(H * k_c, 1),), -7, dtype=torch.int32, device=DEV)
        B.select_col_mask(dims, s, sc, ws, buf)
        torch.cuda.synchronize()
        got = buf[:H * k_c].view(H, k_c).cpu().numpy()
        assert np.array_equal(got, O.col_select(vals, k_c)), want_k
        if k_c == 0:
            assert int(buf[0].item()) == -7    # nothing written


def _random_cols(H, L, k_c, rng, shuffle=False):
    cols = np.stack([np.sort(rng.choice(L, k_c, replace=False)) for _ in range(H)])
    if shuffle:
        for h in range(H):
            rng.shuffle(cols[h])
    return np.ascontiguousarray(cols, dtype=np.int32)


@pytest.mark.timeout(600)
def test_column_variant_at_the_largest_block_count():
    """L = 65536 in 64-token blocks (nb = 1024, the most the library takes),
    with GQA: the column masses, the kept columns (the oracle's except within
    rounding of a cut) and column attention on sampled rows, against the
    oracle (its fp32 masses, which hold the fp64 definition to ~1e-6)."""
    H, Hkv, L, d, blk, s = 2, 1, 65536, 128, 64, 0.9
    q, k, v = random_qkv(H, Hkv, L, d, 919, device=DEV, q_scale=2.0, sinks=True)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    m = GpuCols(q, k, blk, s)
    c_ref, cols_ref, k_c = O.build_col_mask(qf, kf, blk, s)
    assert m.k_c == k_c == 6554
    _check_mass(m.scores(), c_ref.astype(np.float64))
    cols = m.cols()
    _check_cols_form(cols, k_c, L)
    assert np.array_equal(cols, O.col_select(m.scores(), k_c))
    assert len(_compare_cols(cols, cols_ref, c_ref, k_c)) <= 2
    o = torch.empty_like(q)
    B.col_attn(m.dims, q, k, v, m.cols_t(), o)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(9).choice(H * (L // blk), 48, replace=False))
    want = O.col_attn(qf, kf, vf, blk, cols, rows=rows.astype(np.int32))
    PT.check_outputs(o, want, PT.token_mask_for_rows(rows, H, L // blk, blk))


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_column_attention_matches_oracle(shape):
    """Ragged column counts (one partial chunk, exact chunks, under one chunk),
    ascending and shuffled lists, against fp64 attention on the same lists."""
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 613)
    dims = B.dims_of(q, k, blk)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    rng = np.random.default_rng(L + d)
    for k_c, shuffle in ((1, False), (5, False), (32, False), (33, True), (L // 3, False),
                         (L - 7, True)):
        cols = _random_cols(H, L, k_c, rng, shuffle)
        o = torch.empty_like(q)
        B.col_attn(dims, q, k, v, torch.from_numpy(cols).to(DEV), o)
        torch.cuda.synchronize()
        want = O.col_attn(qf, kf, vf, blk, cols)
        PT.check_outputs(o, want)


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_column_attention_edges(shape):
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 614)
    dims = B.dims_of(q, k, blk)
    # Every column, in order: the dense kernel's key sequence, bit for bit.
    allc = torch.arange(L, dtype=torch.int32, device=DEV).repeat(H, 1).contiguous()
    o = torch.empty_like(q)
    od = torch.empty_like(q)
    B.col_attn(dims, q, k, v, allc, o)
    B.dense_attn(dims, q, k, v, od)
    torch.cuda.synchronize()
    assert torch.equal(o, od)
    # No column: zeros.
    o.fill_(1.0)
    B.col_attn(dims, q, k, v, torch.empty((H, 0), dtype=torch.int32, device=DEV), o, k_c=0)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(o)) == 0
    # Deterministic.
    cols = torch.from_numpy(_random_cols(H, L, 45, np.random.default_rng(3))).to(DEV)
    B.col_attn(dims, q, k, v, cols, o)
    B.col_attn(dims, q, k, v, cols, od)
    torch.cuda.synchronize()
    assert torch.equal(o, od)


def test_worked_example_w3_on_gpu():
    """Two strong columns: k_c = 2 keeps keys 5 and 70, k_c = 3 adds key 0 (the
    lowest of the tied rest); every query's output is the closed-form mix."""
    qn, kn, vn = pins.worked_example_w3()
    q, k, v = (torch.from_numpy(x).to(DEV).to(torch.bfloat16) for x in (qn, kn, vn))
    for s, want in ((1 - 2 / 128, [5, 70]), (1 - 3 / 128, [0, 5, 70])):
        m = GpuCols(q, k, 64, s)
        assert list(m.cols()[0]) == want
    m = GpuCols(q, k, 64, 1 - 2 / 128)
    o = torch.empty_like(q)
    B.col_attn(m.dims, q, k, v, m.cols_t(), o)
    torch.cuda.synchronize()
    want = O.col_attn(qn, kn, vn, 64, np.array([[5, 70]], np.int32))
    PT.check_outputs(o, want)
    on = o.float().cpu().numpy()[0]
    w5 = np.exp(0.75) / (np.exp(0.75) + np.exp(0.5))
    assert np.max(np.abs(on[:, 1] - (w5 * 5 + (1 - w5) * 70) / 64)) < 1e-2
    assert np.all(on[:, 2] == 1.0)


@pytest.mark.parametrize("s", [0.5, 0.9])
@pytest.mark.parametrize("shape", SHAPES[:4], ids=SHAPE_IDS[:4])
def test_column_driver_matches_oracle(shape, s):
    """Anchor then reuse step in the driver's column mode, element by element
    against the oracle on the GPU's own columns."""
    H, Hkv, L, d, blk, _ = shape
    q, k, v = _qkv(shape, 615)
    dims = B.dims_of(q, k, blk)
    drv = B.Driver(dims, 0, 4, s, device=DEV, column_sparse=True)
    assert drv.k_c == O.keep_count(L, s) and drv.row_ptr is None
    o = torch.empty_like(q)
    drv.step(0, q, k, v, o)
    torch.cuda.synchronize()
    cols = drv.cols().cpu().numpy()
    _check_cols_form(cols, drv.k_c, L)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    c_ref, cols_ref, _ = O.build_col_mask(qf, kf, blk, s)
    assert len(_compare_cols(cols, cols_ref, c_ref, drv.k_c)) <= 2
    want = O.col_attn(qf, kf, vf, blk, cols)
    PT.check_outputs(o, want)
    # The reuse step keeps the columns: new V, same lists.
    v2 = torch.randn_like(v.float()).to(torch.bfloat16)
    drv.step(1, q, k, v2, o)
    torch.cuda.synchronize()
    assert np.array_equal(drv.cols().cpu().numpy(), cols)
    PT.check_outputs(o, O.col_attn(qf, kf, PT.oracle_inputs(v2)[0], blk, cols))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["stepdllm_8k", "stepdllm_8k_columns"])
def test_column_mask_8k_anchor(name):
    """An 8K workload's step-0 inputs at 90% (i.i.d., and with heavy key
    columns): every mass against the fp64 oracle, the lists against the
    oracle's (near-ties listed), and sampled rows of the attention."""
    w = WORKLOADS[name]
    s = w.sparsities[0]
    traj = Trajectory(w, DEV)
    q, k, v = traj.next()
    m = GpuCols(q, k, w.B, s)
    assert m.k_c == O.keep_count(w.L, s) == 820
    cols = m.cols()
    _check_cols_form(cols, m.k_c, w.L)
    assert np.array_equal(cols, O.col_select(m.scores(), m.k_c))
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    c64 = O.col_scores(qf, kf, w.B)
    _check_mass(m.scores(), c64)
    c_ref = c64.astype(np.float32)
    cols_ref = O.col_select(c_ref, m.k_c)
    listed = _compare_cols(cols, cols_ref, c_ref, m.k_c)
    print(f"8K column mask: k_c={m.k_c} near-ties={len(listed)} {listed[:6]}")
    assert len(listed) <= 8
    o = torch.empty_like(q)
    B.col_attn(m.dims, q, k, v, m.cols_t(), o)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(w.H * w.nb, size=96, replace=False).astype(np.int32)
    want = np.zeros((w.H, w.L, w.d), np.float64)
    PT.oracle_rows_parallel(O.col_attn, rows, q=qf, k=kf, v=vf, B=w.B, cols=cols, out=want)
    PT.check_outputs(o, want, PT.token_mask_for_rows(rows, w.H, w.nb, w.B))


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_column_recall_matches_oracle(shape):
    """Recall of column masks against the fp64 oracle; every column recalls 1,
    none 0; whole key blocks recall the GPU's block attention mass."""
    H, Hkv, L, d, blk, _ = shape
    q, k, _ = _qkv(shape, 616)
    dims = B.dims_of(q, k, blk)
    nb = L // blk
    rng = np.random.default_rng(L + 7)
    qf, kf = PT.oracle_inputs(q, k)
    rec = torch.empty(H * nb, dtype=torch.float32, device=DEV)
    for k_c in (1, 33, L // 4):
        cols = _random_cols(H, L, k_c, rng)
        B.col_recall(dims, q, k, torch.from_numpy(cols).to(DEV), rec)
        torch.cuda.synchronize()
        want = O.col_recall(qf, kf, blk, cols)
        assert np.max(np.abs(rec.cpu().numpy() - want)) < 1e-4, k_c
    allc = torch.arange(L, dtype=torch.int32, device=DEV).repeat(H, 1).contiguous()
    B.col_recall(dims, q, k, allc, rec)
    torch.cuda.synchronize()
    assert float((rec - 1.0).abs().max()) < 1e-4
    B.col_recall(dims, q, k, torch.empty((H, 0), dtype=torch.int32, device=DEV), rec, k_c=0)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(rec)) == 0
    blocks = [np.sort(rng.choice(nb, min(2, nb), replace=False)) for _ in range(H)]
    bcols = np.stack([np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in bl])
                      for bl in blocks]).astype(np.int32)
    mass = torch.empty(H * nb * nb, dtype=torch.float32, device=DEV)
    B.block_mass(dims, q, k, mass)
    B.col_recall(dims, q, k, torch.from_numpy(bcols).to(DEV), rec)
    torch.cuda.synchronize()
    A = mass.cpu().numpy().reshape(H, nb, nb)
    want = np.concatenate([A[h][:, blocks[h]].sum(axis=1) for h in range(H)])
    assert np.max(np.abs(rec.cpu().numpy() - want)) < 1e-5


@pytest.mark.timeout(600)
def test_column_recall_8k_sampled_rows():
    """The 8K anchor's column mask: recall of sampled rows against the oracle."""
    w = WORKLOADS["stepdllm_8k"]
    traj = Trajectory(w, DEV)
    q, k, _ = traj.next()
    m = GpuCols(q, k, w.B, w.sparsities[0])
    rec = torch.empty(w.H * w.nb, dtype=torch.float32, device=DEV)
    B.col_recall(m.dims, q, k, m.cols_t(), rec)
    torch.cuda.synchronize()
    got = rec.cpu().numpy()
    assert np.all((got > 0) & (got <= 1.0 + 1e-5))
    rows = np.random.default_rng(8).choice(w.H * w.nb, size=48, replace=False).astype(np.int32)
    qf, kf = PT.oracle_inputs(q, k)
    want = np.zeros(w.H * w.nb, np.float64)
    PT.oracle_rows_parallel(O.col_recall, rows, q=qf, k=kf, B=w.B, cols=m.cols(), out=want)
    assert np.max(np.abs(got[rows] - want[rows])) < 1e-4
