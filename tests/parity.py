"""Helpers for GPU-vs-oracle comparisons (used by the gpu tests and smoke)."""
import numpy as np
import torch

import oracle as O
from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import to_host_f32

# Output gates (bf16 outputs against the fp64 oracle on the same bf16 inputs).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
ROW_REL_L2 = 2e-2
# Scores within this relative distance of the cut may fall either side of it.
NEAR_TIE_REL = 1e-5


def score_rel_bound(nb):
    """Largest relative difference between the GPU's and the oracle's
    row-softmaxed pooled scores P that fp32 rounding allows.  Both sides form
    the logits identically (fp32 block sums in ascending order, products and
    sums in ascending dimension order without fused multiply-adds, then the
    scale), take the same row maximum and subtract it exactly, so the logits
    agree bit for bit.  Then, with u = 2^-24:
      * exp: the device library's expf and glibc's are each within 1 ulp
        (at most 2u relative), so a numerator differs by at most 4u, and so
        does the exact sum of a row's terms;
      * row sums: the oracle adds the nb terms in order (error at most
        (nb - 1) u relative, all terms positive), the GPU adds ceil(nb/64)
        terms per lane and then 6 butterfly levels over the wave (at most
        (ceil(nb/64) + 5) u);
      * each side's division rounds once (u each).
    First-order total, with 1% for the second-order terms."""
    u = 2.0 ** -24
    return 1.01 * u * (4 + 4 + (nb - 1) + (-(-nb // 64) + 5) + 2)


def keep_from_csr(row_ptr, col_idx, H, nb):
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    keep = np.zeros((H * nb, nb), np.uint8)
    for r in range(H * nb):
        keep[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = 1
    return keep.reshape(H, nb, nb)


def check_csr_form(row_ptr, col_idx, K, nb):
    """row_ptr monotone from 0 to K; every list strictly ascending in [0, nb)."""
    row_ptr = np.asarray(row_ptr).astype(np.int64)
    col_idx = np.asarray(col_idx)
    assert row_ptr[0] == 0 and row_ptr[-1] == K, (row_ptr[0], row_ptr[-1], K)
    assert np.all(np.diff(row_ptr) >= 0)
    assert np.all((col_idx[:K] >= 0) & (col_idx[:K] < nb))
    for r in range(row_ptr.size - 1):
        seg = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(seg) > 0), r


def compare_masks(keep_gpu, keep_ref, P_ref, K):
    """Equal everywhere except at oracle scores within NEAR_TIE_REL of the cut.
    Returns the list of (flat index, oracle value, gpu kept) mismatches."""
    assert int(keep_gpu.sum()) == K and int(keep_ref.sum()) == K
    if K == 0:
        return []
    cut = O.cut_value(P_ref, K)
    diff = np.nonzero(keep_gpu.reshape(-1) != keep_ref.reshape(-1))[0]
    flat = P_ref.reshape(-1)
    listed = []
    for f in diff:
        v = float(flat[f])
        assert abs(v - cut) <= NEAR_TIE_REL * cut, (
            f"mask differs at flat {f}: score {v} vs cut {cut} (not a near-tie)")
        listed.append((int(f), v, int(keep_gpu.reshape(-1)[f])))
    return listed


def check_outputs(o_gpu, o_ref, empty_rows_mask=None):
    """o_gpu: bf16 tensor [H, L, d]; o_ref: fp64 [H, L, d] (only compared where
    sel is True, a boolean [H, L] token mask, or everywhere)."""
    g = o_gpu.detach().to("cpu").to(torch.float64).numpy()
    return check_outputs_np(g, o_ref, empty_rows_mask)


def check_outputs_np(g, o_ref, token_sel=None):
    if token_sel is not None:
        g = g[token_sel]
        r = o_ref[token_sel]
    else:
        g, r = g.reshape(-1, g.shape[-1]), o_ref.reshape(-1, o_ref.shape[-1])
    err = np.abs(g - r)
    stats = dict(max_abs=float(err.max(initial=0.0)), mean_abs=float(err.mean()) if err.size else 0.0)
    nr = np.linalg.norm(r, axis=-1)
    nd = np.linalg.norm(g - r, axis=-1)
    zero = nr == 0
    assert np.all(nd[zero] == 0), "a token the oracle leaves at zero is nonzero"
    rel = nd[~zero] / nr[~zero]
    stats["row_rel_l2"] = float(rel.max(initial=0.0))
    assert stats["max_abs"] <= MAX_ABS, stats
    assert stats["mean_abs"] <= MEAN_ABS, stats
    assert stats["row_rel_l2"] <= ROW_REL_L2, stats
    return stats


class GpuMask:
    """Run the library's anchor-step mask build and fetch every output."""

    def __init__(self, q, k, blk, sparsity, scores_copy=True, per_head=False):
        self.dims = B.dims_of(q, k, blk)
        self.buf = B.MaskBuffers(self.dims, sparsity, device=q.device, per_head=per_head)
        H, nb = q.shape[0], q.shape[1] // blk
        self.scores_out = (torch.empty(H * nb * nb, dtype=torch.float32, device=q.device)
                           if scores_copy else None)
        B.build_mask(self.dims, sparsity, q, k, self.buf.ws, self.buf.row_ptr,
                     self.buf.col_idx, self.scores_out, per_head=per_head)
        torch.cuda.synchronize()
        self.K = self.buf.K
        self.H, self.nb = H, nb

    def csr(self):
        return (self.buf.row_ptr.cpu().numpy(), self.buf.col_idx[: self.K].cpu().numpy())

    def keep(self):
        rp, ci = self.csr()
        return keep_from_csr(rp, ci, self.H, self.nb)

    def P(self):
        return self.scores_out.cpu().numpy().reshape(self.H, self.nb, self.nb)


def oracle_inputs(*tensors):
    return [to_host_f32(t) for t in tensors]


def token_mask_for_rows(rows, H, nb, blk):
    sel = np.zeros((H, nb * blk), bool)
    for r in rows:
        h, i = divmod(int(r), nb)
        sel[h, i * blk:(i + 1) * blk] = True
    return sel


def oracle_rows_parallel(fn, rows, threads=None, **kw):
    """Run an oracle attention function over `rows` split across host threads
    (ctypes releases the GIL); all calls write disjoint rows of one output."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    rows = np.asarray(rows, np.int32)
    threads = threads or max(1, min(16, len(os.sched_getaffinity(0))))
    out = kw.pop("out")
    parts = [p for p in np.array_split(rows, threads * 4) if p.size]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda p: fn(rows=p, out=out, **kw), parts))
    return out


def sample_rows(row_ptr, H, nb, heads=(0,), n_longest=64, n_random=64, seed=0):
    """All rows of the given heads, the longest lists, and seeded random rows."""
    lens = np.diff(np.asarray(row_ptr))
    rows = set()
    for h in heads:
        rows.update(range(h * nb, (h + 1) * nb))
    rows.update(np.argsort(-lens, kind="stable")[:n_longest].tolist())
    rng = np.random.default_rng(seed)
    rows.update(rng.choice(H * nb, size=min(n_random, H * nb), replace=False).tolist())
    return np.array(sorted(rows), np.int32)
