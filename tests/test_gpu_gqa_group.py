"""GQA variant with group-shared K/V tiles (stepdllm_sparse_attn_group): each
head's output must equal the per-head sparse kernel's bit for bit (same
chunks, same order, same arithmetic), and the oracle's within the usual
tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import WORKLOADS, Trajectory, random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (H, Hkv, L, d): odd and even group sizes, one head per group, ragged blocks.
SHAPES = [(14, 2, 37 * 64, 128, ), (8, 4, 21 * 64, 128), (6, 6, 9 * 64, 64), (9, 3, 33 * 64, 64),
          (7, 1, 16 * 64, 128)]
IDS = ["H14G7", "H8G2", "H6G1_d64", "H9G3_d64", "H7G7"]


def _per_head(dims, q, k, v, rp, ci, nnz):
    buf = B.MaskBuffers(dims, 0.5, device=DEV)
    B.plan(dims, rp, ci, buf.ws, nnz=nnz)
    o = torch.full_like(q, float("nan"))
    B.sparse_attn(dims, q, k, v, ci, buf.ws, o, nnz=nnz)
    return o


def _group(dims, q, k, v, rp, ci, nnz):
    o = torch.full_like(q, float("nan"))
    B.sparse_attn_group(dims, q, k, v, rp, ci, o, nnz=nnz)
    return o


@pytest.mark.parametrize("s", [0.5, 0.9])
@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_group_equals_per_head_on_built_masks(shape, s):
    H, Hkv, L, d = shape
    q, k, v = random_qkv(H, Hkv, L, d, 1212, device=DEV, q_scale=2.0)
    dims = B.dims_of(q, k, 64)
    m = PT.GpuMask(q, k, 64, s)
    o_ref = _per_head(dims, q, k, v, m.buf.row_ptr, m.buf.col_idx, m.K)
    o = _group(dims, q, k, v, m.buf.row_ptr, m.buf.col_idx, m.K)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s", [0.5, 0.9])
def test_group_equals_per_head_at_the_largest_block_count(s):
    """nb = 1024 (L = 65536), the most the library takes: at s = 0.5 a head
    pair's union of lists fills most of the 1024 entries the workgroup holds
    in LDS; the output equals the per-head kernel's bit for bit."""
    H, Hkv, L, d = 4, 2, 65536, 128
    q, k, v = random_qkv(H, Hkv, L, d, 1313, device=DEV, q_scale=2.0)
    dims = B.dims_of(q, k, 64)
    m = PT.GpuMask(q, k, 64, s, scores_copy=False)
    rp = m.buf.row_ptr.cpu().numpy()
    assert m.nb == 1024 and int(np.diff(rp).max()) > 64
    o_ref = _per_head(dims, q, k, v, m.buf.row_ptr, m.buf.col_idx, m.K)
    o = _group(dims, q, k, v, m.buf.row_ptr, m.buf.col_idx, m.K)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_group_matches_oracle():
    H, Hkv, L, d = 14, 2, 37 * 64, 128
    q, k, v = random_qkv(H, Hkv, L, d, 1313, device=DEV, q_scale=2.0, sinks=True)
    qf, kf, vf = PT.oracle_inputs(q, k, v)
    ref = O.build_mask(qf, kf, 64, 0.8)
    dims = B.dims_of(q, k, 64)
    rp = torch.from_numpy(ref["row_ptr"]).to(DEV)
    ci = torch.from_numpy(np.concatenate([ref["col_idx"], [0]]).astype(np.int32)).to(DEV)
    o = _group(dims, q, k, v, rp, ci, ref["K"])
    torch.cuda.synchronize()
    PT.check_outputs(o, O.sparse_attn(qf, kf, vf, 64, ref["row_ptr"], ref["col_idx"]))


@pytest.mark.parametrize("shape", SHAPES[:2] + SHAPES[4:], ids=IDS[:2] + IDS[4:])
def test_group_with_empty_rows_and_lopsided_pairs(shape):
    """Injected masks: whole empty rows, pairs where one head keeps nothing for
    a query block, pairs with disjoint and with identical lists."""
    H, Hkv, L, d = shape
    nb = L // 64
    G = H // Hkv
    rng = np.random.default_rng(H * 100 + nb)
    keep = rng.random((H, nb, nb)) < 0.3
    keep[:, 0, :] = False                          # every head empty on block 0
    keep[0, 1, :] = False                          # head 0 empty on block 1, head 1 not
    keep[1, 1, :] = True
    if G > 1:
        keep[1, 2] = keep[0, 2]                    # identical lists
        keep[1, 3] = ~keep[0, 3]                   # disjoint lists
    rp_np, ci_np = O.csr(keep.astype(np.uint8))
    q, k, v = random_qkv(H, Hkv, L, d, 1414, device=DEV, q_scale=1.5)
    dims = B.dims_of(q, k, 64)
    rp = torch.from_numpy(rp_np).to(DEV)
    ci = torch.from_numpy(np.concatenate([ci_np, [0]]).astype(np.int32)).to(DEV)
    nnz = int(rp_np[-1])
    o_ref = _per_head(dims, q, k, v, rp, ci, nnz)
    o = _group(dims, q, k, v, rp, ci, nnz)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    rows = np.nonzero(np.diff(rp_np) == 0)[0]
    o_rows = o.view(H, nb, 64, d)
    for r in rows[:8]:
        assert torch.count_nonzero(o_rows[r // nb, r % nb].float()) == 0


def test_group_malformed_ids_are_clamped_like_the_per_head_kernel():
    H, Hkv, L, d = 8, 4, 12 * 64, 128
    nb = L // 64
    rng = np.random.default_rng(5)
    keep = rng.random((H, nb, nb)) < 0.4
    rp_np, ci_np = O.csr(keep.astype(np.uint8))
    ci_np = ci_np.astype(np.int64)
    ci_np[::7] += 3 * nb                           # out of range above
    ci_np[3::11] = -5                              # and below
    q, k, v = random_qkv(H, Hkv, L, d, 1515, device=DEV)
    dims = B.dims_of(q, k, 64)
    rp = torch.from_numpy(rp_np).to(DEV)
    ci = torch.from_numpy(ci_np.astype(np.int32)).to(DEV)
    o = _group(dims, q, k, v, rp, ci, int(rp_np[-1]))
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()


def test_group_rejects_block_128():
    q, k, v = random_qkv(4, 2, 4 * 128, 64, 1, device=DEV)
    dims = B.dims_of(q, k, 128)
    rp = torch.zeros(4 * 4 + 1, dtype=torch.int32, device=DEV)
    ci = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(B.StepDLLMError) as e:
        B.sparse_attn_group(dims, q, k, v, rp, ci, torch.empty_like(q), nnz=0)
    assert e.value.status == B.EUNSUPPORTED


@pytest.mark.parametrize("name,s", [("dream_gqa_8k", 0.7), ("dream_gqa_8k", 0.9),
                                    ("dream_gqa_8k_shared", 0.7), ("dream_gqa_8k_shared", 0.95)])
def test_group_equals_per_head_at_full_size(name, s):
    """The Dream-shaped GQA layer (H=28, Hkv=4, L=8192, d=128) at its anchor,
    with independent heads and with a KV group's heads keeping nearly the same
    blocks (long shared runs in every pair's union); on the shared inputs the
    group output is also checked against the oracle on sampled rows."""
    w = WORKLOADS[name]
    q, k, v = Trajectory(w, DEV).next()
    dims = B.make_dims(w.H, w.Hkv, w.L, w.d, w.B)
    buf = B.MaskBuffers(dims, s, device=DEV)
    B.build_mask(dims, s, q, k, buf.ws, buf.row_ptr, buf.col_idx)
    o_ref = torch.full_like(q, float("nan"))
    B.sparse_attn(dims, q, k, v, buf.col_idx, buf.ws, o_ref, nnz=buf.K)
    o = _group(dims, q, k, v, buf.row_ptr, buf.col_idx, buf.K)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    if w.shared:
        rp = buf.row_ptr.cpu().numpy()
        ci = buf.col_idx[:buf.K].cpu().numpy()
        rows = PT.sample_rows(rp, w.H, w.nb, heads=(0, 1), n_longest=32, n_random=32)
        qf, kf, vf = PT.oracle_inputs(q, k, v)
        out = np.zeros(qf.shape, np.float64)
        PT.oracle_rows_parallel(O.sparse_attn, rows, q=qf, k=kf, v=vf, B=w.B, row_ptr=rp,
                                col_idx=ci, out=out)
        stats = PT.check_outputs(o, out, PT.token_mask_for_rows(rows, w.H, w.nb, w.B))
        print(f"{name} s={s} group: {len(rows)} rows {stats}", flush=True)
