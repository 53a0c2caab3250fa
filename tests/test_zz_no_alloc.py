"""The allocation-free step (stepdllm_step_noalloc, workspace in the library's
static device array) against the step driver (stepdllm_step, caller-owned
workspace): the same kernels, so outputs and masks must be identical bit for
bit, on calls in a row whose later series use smaller inputs, and with the
array keeping the previous call's contents."""
import pytest
import torch

from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import random_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _series(shape, dense, every, s, steps, seed, per_head=False, columns=False):
    H, Hkv, L, d, blk = shape
    dims = B.make_dims(H, Hkv, L, d, blk)
    drv = B.Driver(dims, dense, every, s, device=DEV, per_head_budget=per_head,
                   column_sparse=columns)
    rp = None if columns else torch.full((H * (L // blk) + 1,), -1, dtype=torch.int32,
                                         device=DEV)
    ci = torch.full((max(drv.K, 1),), -1, dtype=torch.int32, device=DEV)
    for t in steps:
        print(f"no-alloc step: shape {shape} schedule ({dense}, {every}, {s}) "
              f"per_head={per_head} columns={columns} step {t}", flush=True)
        q, k, v = random_qkv(H, Hkv, L, d, seed + t, device=DEV, q_scale=2.0, sinks=True)
        o_ref = torch.empty_like(q)
        drv.step(t, q, k, v, o_ref)
        o = torch.full_like(q, float("nan"))
        st = B.step_noalloc(dims, dense, every, s, t, q, k, v, rp, ci, o,
                            per_head_budget=per_head, column_sparse=columns)
        torch.cuda.synchronize()
        assert st == B.OK, B.status_string(st)
        assert torch.equal(o, o_ref), (shape, t)
        if drv.step_kind(t) == 1:
            assert torch.equal(ci[:drv.K], drv.col_idx[:drv.K]), (shape, t)
            if not columns:
                assert torch.equal(rp, drv.row_ptr), (shape, t)
    drv.close()


def test_noalloc_step_matches_the_driver():
    # Dense warm-up step, anchors and reuse steps on a GQA shape ...
    _series((8, 4, 2048, 128, 64), 1, 2, 0.8, range(5), 100)
    # ... then a smaller shape: its anchor replaces the plan in the array.
    _series((4, 2, 512, 64, 64), 0, 3, 0.6, range(4), 200)
    # The uniform per-head budget and the column variant, smaller still.
    _series((2, 2, 256, 64, 64), 0, 2, 0.5, range(3), 300, per_head=True)
    _series((2, 1, 256, 64, 64), 0, 2, 0.75, range(3), 400, columns=True)
