"""Mask quality on the GPU against the oracle, through the C ABI: the true
block attention mass of the full softmax map and the recall of a mask."""
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
    (8, 8, 16 * 64, 128, 64, 3.0),
]
SHAPE_IDS = [f"H{s[0]}kv{s[1]}L{s[2]}d{s[3]}B{s[4]}" for s in SHAPES]

# fp32 scores from exact bf16 products, fp32 exp2 and block sums: the mass is
# within 1e-4 relative (plus 1e-6 absolute) of the fp64 map.
MASS_REL, MASS_ABS = 1e-4, 1e-6


def _qkv(shape, seed):
    H, Hkv, L, d, blk, qs = shape
    return random_qkv(H, Hkv, L, d, seed, device=DEV, q_scale=qs, sinks=True)


def _mass(q, k, blk):
    dims = B.dims_of(q, k, blk)
    H, nb = q.shape[0], q.shape[1] // blk
    mass = torch.empty(H * nb * nb, dtype=torch.float32, device=DEV)
    B.block_mass(dims, q, k, mass)
    torch.cuda.synchronize()
    return dims, mass


def _check_mass(got, want):
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= MASS_ABS + MASS_REL * want), float(err.max())


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_block_mass_matches_oracle(shape):
    H, Hkv, L, d, blk, _ = shape
    q, k, _ = _qkv(shape, 414)
    dims, mass = _mass(q, k, blk)
    nb = L // blk
    got = mass.cpu().numpy().reshape(H, nb, nb)
    qf, kf = PT.oracle_inputs(q, k)
    want = O.block_mass(qf, kf, blk)
    _check_mass(got, want)
    assert np.max(np.abs(got.sum(axis=2) - 1.0)) < 1e-4
    # Deterministic: a second launch gives the same bits.
    _, mass2 = _mass(q, k, blk)
    assert torch.equal(mass, mass2)


def test_block_mass_closed_forms():
    """Q = 0: every block gets 1/nb.  The W1 concentrated head: 1/(1+3e^-50) on
    the diagonal and e^-50/(1+3e^-50) off it, to 1e-4 relative (the fp32
    exponent 50*log2(e) carries about 1e-5 of rounding)."""
    H, L, d, blk = 2, 512, 64, 64
    nb = L // blk
    q = torch.zeros(H, L, d, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(H, L, d, device=DEV).to(torch.bfloat16)
    _, mass = _mass(q, k, blk)
    assert torch.allclose(mass, torch.full_like(mass, 1.0 / nb), rtol=0, atol=2e-7)
    import oracle_pins as pins
    qw, kw, _, _ = pins.worked_example_w1()
    qg = torch.from_numpy(qw).to(DEV).to(torch.bfloat16)
    kg = torch.from_numpy(kw).to(DEV).to(torch.bfloat16)
    _, mw = _mass(qg, kg, 64)
    a0 = mw.cpu().numpy().reshape(2, 4, 4)[0].astype(np.float64)
    e = np.exp(-50.0)
    for i in range(4):
        for j in range(4):
            want = 1 / (1 + 3 * e) if i == j else e / (1 + 3 * e)
            assert abs(a0[i, j] - want) <= 1e-4 * want, (i, j, a0[i, j])


@pytest.mark.parametrize("s", [0.5, 0.9])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_mask_recall_matches_oracle(shape, s):
    H, Hkv, L, d, blk, _ = shape
    q, k, _ = _qkv(shape, 515)
    m = PT.GpuMask(q, k, blk, s)
    dims, mass = _mass(q, k, blk)
    rec = torch.empty(m.buf.rows, dtype=torch.float32, device=DEV)
    B.mask_recall(dims, mass, m.buf.row_ptr, m.buf.col_idx, rec, nnz=m.K)
    torch.cuda.synchronize()
    rp, ci = m.csr()
    got = rec.cpu().numpy()
    nb = L // blk
    # The oracle's recall of the same mask on the GPU's own mass: fp32 sums.
    own = O.mask_recall(mass.cpu().numpy().reshape(H, nb, nb), rp, ci)
    assert np.max(np.abs(got - own)) < 1e-5
    # ... and on the fp64 mass.
    qf, kf = PT.oracle_inputs(q, k)
    ref = O.mask_recall(O.block_mass(qf, kf, blk), rp, ci)
    assert np.max(np.abs(got - ref)) < 1e-4
    assert np.all(got[np.diff(rp) == 0] == 0)
    # A full mask recalls everything.
    full_rp = (np.arange(H * nb + 1) * nb).astype(np.int32)
    full_ci = np.tile(np.arange(nb, dtype=np.int32), H * nb)
    B.mask_recall(dims, mass, torch.from_numpy(full_rp).to(DEV), torch.from_numpy(full_ci).to(DEV),
                  rec)
    torch.cuda.synchronize()
    assert np.max(np.abs(rec.cpu().numpy() - 1.0)) < 1e-4


@pytest.mark.timeout(600)
def test_block_mass_8k_sampled_rows():
    """The 8K workload's step-0 inputs: the mass of sampled rows against the
    fp64 oracle, and every row summing to 1."""
    w = WORKLOADS["stepdllm_8k"]
    traj = Trajectory(w, DEV)
    q, k, _ = traj.next()
    dims, mass = _mass(q, k, w.B)
    got = mass.cpu().numpy().reshape(w.H, w.nb, w.nb)
    assert np.max(np.abs(got.sum(axis=2) - 1.0)) < 1e-3
    rows = np.array([0, 1, 127, 128 + 5, 17 * 128 + 64, 31 * 128 + 127, 9 * 128 + 3,
                     23 * 128 + 100], np.int32)
    qf, kf = PT.oracle_inputs(q, k)
    want = np.zeros((w.H, w.nb, w.nb), np.float64)
    PT.oracle_rows_parallel(O.block_mass, rows, q=qf, k=kf, B=w.B, out=want)
    for r in rows:
        _check_mass(got.reshape(-1, w.nb)[r], want.reshape(-1, w.nb)[r])
