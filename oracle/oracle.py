"""ctypes wrapper over ``oracle.c`` -- TEST INFRASTRUCTURE ONLY.

Argument marshalling only: every step of the computation is in ``oracle.c``.
Arrays are numpy, host memory; float inputs are fp32 arrays that hold
bf16-rounded values; attention outputs are fp64.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

_lib = None


def build(out=_LIB, extra_flags=()):
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    cmd = ["gcc", *_CFLAGS, *extra_flags, _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
    ci, ci64, cd, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    sig = {
        "oracle_pool": (None, [f32p, ci, ci, ci, ci, f32p]),
        "oracle_scores": (None, [f32p, f32p, ci, ci, ci, ci, f32p]),
        "oracle_keep_count": (ci64, [ci64, cd]),
        "oracle_select": (None, [f32p, ci64, ci64, u8p]),
        "oracle_select_per_head": (None, [f32p, ci, ci, ci64, u8p]),
        "oracle_cut_value": (ctypes.c_float, [f32p, ci64, ci64]),
        "oracle_csr": (None, [u8p, ci, ci, i32p, i32p]),
        "oracle_build_mask": (ci64, [f32p, f32p, ci, ci, ci, ci, ci, cd, f32p, f32p, f32p, i32p, i32p]),
        "oracle_build_mask_per_head": (ci64, [f32p, f32p, ci, ci, ci, ci, ci, cd, f32p, f32p, f32p,
                                              i32p, i32p]),
        "oracle_plan": (ctypes.c_int32, [i32p, ci, ci, ci, i32p]),
        "oracle_sparse_attn": (None, [f32p, f32p, f32p, ci, ci, ci, ci, ci, i32p, i32p, vp, ci, f64p]),
        "oracle_dense_attn": (None, [f32p, f32p, f32p, ci, ci, ci, ci, ci, vp, ci, f64p]),
        "oracle_step_kind": (ci, [ci, ci, ci]),
        "oracle_block_mass": (None, [f32p, f32p, ci, ci, ci, ci, ci, vp, ci, f64p]),
        "oracle_mask_recall": (None, [f64p, ci, ci, i32p, i32p, f64p]),
        "oracle_bf16_round": (None, [f32p, ci64, f32p]),
        "oracle_col_scores": (None, [f32p, f32p, ci, ci, ci, ci, ci, f64p]),
        "oracle_col_select": (None, [f32p, ci, ci, ci64, i32p]),
        "oracle_build_col_mask": (ci64, [f32p, f32p, ci, ci, ci, ci, ci, cd, f32p, i32p]),
        "oracle_col_attn": (None, [f32p, f32p, f32p, ci, ci, ci, ci, ci, i32p, ci64, vp, ci, f64p]),
        "oracle_col_recall": (None, [f32p, f32p, ci, ci, ci, ci, ci, i32p, ci64, vp, ci, f64p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path=None):
    """Load the compiled oracle (building it first only if nothing is built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _rows_arg(rows):
    if rows is None:
        return None, 0, None
    r = np.ascontiguousarray(rows, dtype=np.int32)
    return r.ctypes.data_as(ctypes.c_void_p), int(r.size), r


def pool(x, B, lib=None):
    """x: [heads, L, d] -> block means [heads, L/B, d] (fp32)."""
    lib = lib or load()
    x = _f32(x)
    h, L, d = x.shape
    out = np.empty((h, L // B, d), np.float32)
    lib.oracle_pool(x, h, L, d, B, out)
    return out


def scores(qb, kb, lib=None):
    """Pooled scores softmaxed per (head, q-block) row: [H, nb, nb] (fp32)."""
    lib = lib or load()
    qb, kb = _f32(qb), _f32(kb)
    H, nb, d = qb.shape
    Hkv = kb.shape[0]
    out = np.empty((H, nb, nb), np.float32)
    lib.oracle_scores(qb, kb, H, Hkv, nb, d, out)
    return out


def keep_count(n, sparsity, lib=None):
    lib = lib or load()
    return int(lib.oracle_keep_count(int(n), float(sparsity)))


def select(P, K, lib=None):
    """Global top-K of P (value desc, flat index asc) -> uint8 keep mask, P's shape."""
    lib = lib or load()
    P = _f32(P)
    keep = np.empty(P.shape, np.uint8)
    lib.oracle_select(P.reshape(-1), P.size, int(K), keep.reshape(-1))
    return keep


def select_per_head(P, k_h, lib=None):
    """Uniform per-head budget: top-k_h of each head's slice P[h] -> uint8 keep mask."""
    lib = lib or load()
    P = _f32(P)
    H, nb, _ = P.shape
    keep = np.empty(P.shape, np.uint8)
    lib.oracle_select_per_head(P.reshape(-1), H, nb, int(k_h), keep.reshape(-1))
    return keep


def cut_value(P, K, lib=None):
    lib = lib or load()
    P = _f32(P)
    return float(lib.oracle_cut_value(P.reshape(-1), P.size, int(K)))


def csr(keep, lib=None):
    """keep [H, nb, nb] -> (row_ptr [H*nb+1], col_idx [nnz]) int32."""
    lib = lib or load()
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    H, nb, _ = keep.shape
    rows = H * nb
    row_ptr = np.empty(rows + 1, np.int32)
    col_idx = np.empty(max(int(keep.sum()), 1), np.int32)
    lib.oracle_csr(keep.reshape(-1), rows, nb, row_ptr, col_idx)
    return row_ptr, col_idx[: row_ptr[-1]].copy()


def build_mask(q, k, B, sparsity, lib=None, per_head=False):
    """Anchor-step mask build. Returns dict(qb, kb, P, K, row_ptr, col_idx).
    per_head: the uniform per-head budget instead of the global one."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    H, L, d = q.shape
    Hkv = k.shape[0]
    nb = L // B
    qb = np.empty((H, nb, d), np.float32)
    kb = np.empty((Hkv, nb, d), np.float32)
    P = np.empty((H, nb, nb), np.float32)
    row_ptr = np.empty(H * nb + 1, np.int32)
    col_idx = np.empty(H * nb * nb, np.int32)
    fn = lib.oracle_build_mask_per_head if per_head else lib.oracle_build_mask
    K = fn(q, k, H, Hkv, L, d, B, float(sparsity), qb, kb, P, row_ptr, col_idx)
    return dict(qb=qb, kb=kb, P=P, K=int(K), row_ptr=row_ptr, col_idx=col_idx[:K].copy())


DIES = 8


def plan(row_ptr, H, nb, B, lib=None):
    """-> (work [8 * cap] int32 with -1 padding, n_nonempty); cap =
    min(H, ceil(H/8) + 2) * nb; heads weigh (B/32)*kept + 4*nonempty rows."""
    lib = lib or load()
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    cap = min(H, -(-H // DIES) + 2) * nb
    work = np.empty(DIES * cap, np.int32)
    n = lib.oracle_plan(row_ptr, int(H), int(nb), int(B), work)
    return work, int(n)


def sparse_attn(q, k, v, B, row_ptr, col_idx, rows=None, lib=None, out=None):
    """fp64 block-sparse attention; only the listed rows of ``out`` are written."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, L, d = q.shape
    Hkv = k.shape[0]
    if out is None:
        out = np.zeros((H, L, d), np.float64)
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if ci.size == 0:
        ci = np.zeros(1, np.int32)
    rptr, nrows, _keep = _rows_arg(rows)
    lib.oracle_sparse_attn(q, k, v, H, Hkv, L, d, B, rp, ci, rptr, nrows, out)
    return out


def dense_attn(q, k, v, B, rows=None, lib=None, out=None):
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, L, d = q.shape
    Hkv = k.shape[0]
    if out is None:
        out = np.zeros((H, L, d), np.float64)
    rptr, nrows, _keep = _rows_arg(rows)
    lib.oracle_dense_attn(q, k, v, H, Hkv, L, d, B, rptr, nrows, out)
    return out


def step_kind(step, dense_steps, refresh_every, lib=None):
    lib = lib or load()
    return int(lib.oracle_step_kind(int(step), int(dense_steps), int(refresh_every)))


def block_mass(q, k, B, rows=None, lib=None, out=None):
    """True block attention mass A [H, nb, nb] (fp64): mean over each query
    block's tokens of the full softmax probability on each key block.  rows:
    optional row ids h*nb + i to compute (others stay as in `out`, else 0)."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    H, L, d = q.shape
    nb = L // B
    A = np.zeros((H, nb, nb), np.float64) if out is None else out
    rp, nr, keep = _rows_arg(rows)
    lib.oracle_block_mass(q, k, H, k.shape[0], L, d, B, rp, nr, A)
    return A


def mask_recall(A, row_ptr, col_idx, lib=None):
    """Per-row recall [H*nb] (fp64): the block mass on each row's kept blocks."""
    lib = lib or load()
    A = np.ascontiguousarray(A, dtype=np.float64)
    H, nb, _ = A.shape
    rec = np.empty(H * nb, np.float64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if ci.size == 0:
        ci = np.zeros(1, np.int32)
    lib.oracle_mask_recall(A, H * nb, nb, np.ascontiguousarray(row_ptr, dtype=np.int32), ci, rec)
    return rec


def bf16_round(x, lib=None):
    """Round fp32 values to the nearest bf16 (ties to even), as fp32."""
    lib = lib or load()
    x = _f32(x)
    y = np.empty_like(x)
    lib.oracle_bf16_round(x.reshape(-1), int(x.size), y.reshape(-1))
    return y


def col_scores(q, k, B, lib=None):
    """Column masses c [H, L] (fp64) of the column-sparse variant: the mean over
    each head's bf16-rounded pooled queries of the softmax over all key
    tokens."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    H, L, d = q.shape
    c = np.empty((H, L), np.float64)
    lib.oracle_col_scores(q, k, H, k.shape[0], L, d, B, c)
    return c


def col_select(c, k_c, lib=None):
    """Per head, the k_c largest fp32 column masses (ties to the lowest index),
    ascending: cols [H, k_c] int32."""
    lib = lib or load()
    c = _f32(c)
    H, L = c.shape
    cols = np.empty((H, max(int(k_c), 0)), np.int32)
    lib.oracle_col_select(c, H, L, int(k_c), cols if cols.size else np.zeros(1, np.int32))
    return cols


def build_col_mask(q, k, B, sparsity, lib=None):
    """-> (c fp32 [H, L], cols [H, k_c] int32, k_c) for the column-sparse variant."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    H, L, d = q.shape
    k_c = int(lib.oracle_keep_count(L, float(sparsity)))
    c = np.empty((H, L), np.float32)
    cols = np.empty((H, k_c), np.int32)
    got = lib.oracle_build_col_mask(q, k, H, k.shape[0], L, d, B, float(sparsity), c,
                                    cols if cols.size else np.zeros(1, np.int32))
    assert got == k_c
    return c, cols, k_c


def col_attn(q, k, v, B, cols, rows=None, lib=None, out=None):
    """fp64 column-sparse attention: every query of head h attends to the key
    tokens cols[h] (ascending); only the listed rows h*nb + i are written."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    H, L, d = q.shape
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    k_c = cols.shape[1] if cols.ndim == 2 else 0
    if out is None:
        out = np.zeros((H, L, d), np.float64)
    rptr, nrows, _keep = _rows_arg(rows)
    lib.oracle_col_attn(q, k, v, H, k.shape[0], L, d, B,
                        cols if cols.size else np.zeros(1, np.int32), int(k_c), rptr, nrows, out)
    return out


def col_recall(q, k, B, cols, rows=None, lib=None, out=None):
    """Recall of a column mask per row h*nb + i (fp64 [H*nb]): the mean over the
    block's query tokens of the full-softmax probability on the kept columns
    cols[h].  Only the listed rows are written."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    H, L, d = q.shape
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    k_c = cols.shape[1] if cols.ndim == 2 else 0
    if out is None:
        out = np.zeros(H * (L // B), np.float64)
    rptr, nrows, _keep = _rows_arg(rows)
    lib.oracle_col_recall(q, k, H, k.shape[0], L, d, B,
                          cols if cols.size else np.zeros(1, np.int32), int(k_c), rptr, nrows, out)
    return out


__all__ = ["build", "load", "pool", "scores", "keep_count", "select", "select_per_head",
           "cut_value", "csr",
           "build_mask", "plan", "sparse_attn", "dense_attn", "step_kind", "block_mass",
           "mask_recall", "bf16_round", "col_scores", "col_select", "build_col_mask",
           "col_attn", "col_recall"]
