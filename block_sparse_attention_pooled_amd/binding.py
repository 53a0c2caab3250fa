"""Thin Python binding over the C ABI (include/stepdllm.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory and the current HIP stream.  If the
built library is missing, every call raises instead of computing anything
another way.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstepdllm.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ESTATE, ENOMEM = 0, -1, -2, -3, -4, -5, -6


class Dims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32)]


class Schedule(ctypes.Structure):
    _fields_ = [("dense_steps", ctypes.c_int32), ("refresh_every", ctypes.c_int32),
                ("sparsity", ctypes.c_double), ("per_head_budget", ctypes.c_int32),
                ("column_sparse", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("pooled_q", "pooled_k", "scores", "select", "work", "work_meta",
                 "head_select", "col_scores", "col_stats", "work_rec", "total")]


class StepDLLMError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_lib = None
_vp = ctypes.c_void_p


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run block_sparse_attention_pooled_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    D = ctypes.POINTER(Dims)
    i32, i64, dbl, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    sig = {
        "stepdllm_keep_count": (i64, [D, dbl]),
        "stepdllm_keep_count_per_head": (i64, [D, dbl]),
        "stepdllm_workspace_bytes": (i64, [D]),
        "stepdllm_workspace_layout": (i32, [D, ctypes.POINTER(WsLayout)]),
        "stepdllm_build_mask": (i32, [D, dbl, _vp, _vp, _vp, sz, _vp, _vp, _vp, _vp]),
        "stepdllm_select_mask": (i32, [D, dbl, _vp, _vp, sz, _vp, _vp, _vp]),
        "stepdllm_build_mask_per_head": (i32, [D, dbl, _vp, _vp, _vp, sz, _vp, _vp, _vp, _vp]),
        "stepdllm_select_mask_per_head": (i32, [D, dbl, _vp, _vp, sz, _vp, _vp, _vp]),
        "stepdllm_plan": (i32, [D, _vp, _vp, i64, _vp, sz, _vp]),
        "stepdllm_sparse_attn": (i32, [D, _vp, _vp, _vp, _vp, i64, _vp, sz, _vp, _vp]),
        "stepdllm_dense_attn": (i32, [D, _vp, _vp, _vp, _vp, _vp]),
        "stepdllm_sparse_attn_group": (i32, [D, _vp, _vp, _vp, _vp, _vp, i64, _vp, _vp]),
        "stepdllm_block_mass": (i32, [D, _vp, _vp, _vp, _vp]),
        "stepdllm_mask_recall": (i32, [D, _vp, _vp, _vp, i64, _vp, _vp]),
        "stepdllm_keep_count_columns": (i64, [D, dbl]),
        "stepdllm_build_col_mask": (i32, [D, dbl, _vp, _vp, _vp, sz, _vp, _vp, _vp]),
        "stepdllm_select_col_mask": (i32, [D, dbl, _vp, _vp, sz, _vp, _vp]),
        "stepdllm_col_attn": (i32, [D, _vp, _vp, _vp, _vp, i64, _vp, _vp]),
        "stepdllm_col_recall": (i32, [D, _vp, _vp, _vp, i64, _vp, _vp]),
        "stepdllm_driver_create": (i32, [ctypes.POINTER(_vp), D, ctypes.POINTER(Schedule), _vp,
                                         sz, _vp, _vp]),
        "stepdllm_driver_step_kind": (i32, [_vp, ctypes.c_int32]),
        "stepdllm_step_noalloc": (i32, [D, ctypes.POINTER(Schedule), ctypes.c_int32, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp]),
        "stepdllm_step": (i32, [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]),
        "stepdllm_driver_destroy": (i32, [_vp]),
        "stepdllm_status_string": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


EXPORTS = ["stepdllm_keep_count", "stepdllm_workspace_bytes", "stepdllm_workspace_layout",
           "stepdllm_build_mask", "stepdllm_select_mask", "stepdllm_keep_count_per_head",
           "stepdllm_build_mask_per_head", "stepdllm_select_mask_per_head", "stepdllm_plan",
           "stepdllm_sparse_attn", "stepdllm_sparse_attn_group", "stepdllm_dense_attn",
           "stepdllm_block_mass",
           "stepdllm_mask_recall", "stepdllm_keep_count_columns", "stepdllm_build_col_mask",
           "stepdllm_select_col_mask", "stepdllm_col_attn", "stepdllm_col_recall",
           "stepdllm_driver_create",
           "stepdllm_driver_step_kind", "stepdllm_step", "stepdllm_driver_destroy",
           "stepdllm_step_noalloc",
           "stepdllm_status_string"]


def status_string(status):
    return load().stepdllm_status_string(int(status)).decode()


def _check(status, fn):
    if status != OK:
        raise StepDLLMError(status, fn)


def make_dims(H, Hkv, L, d, B):
    return Dims(int(H), int(Hkv), int(L), int(d), int(B))


def dims_of(q, k, B):
    H, L, d = q.shape
    return make_dims(H, k.shape[0], L, d, B)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def keep_count(dims, sparsity, per_head=False):
    """K of the global budget, or H * k_h of the uniform per-head one."""
    fn = "stepdllm_keep_count_per_head" if per_head else "stepdllm_keep_count"
    r = getattr(load(), fn)(ctypes.byref(dims), float(sparsity))
    if r < 0:
        raise StepDLLMError(int(r), fn)
    return int(r)


def workspace_bytes(dims):
    r = load().stepdllm_workspace_bytes(ctypes.byref(dims))
    if r < 0:
        raise StepDLLMError(int(r), "stepdllm_workspace_bytes")
    return int(r)


def workspace_layout(dims):
    out = WsLayout()
    _check(load().stepdllm_workspace_layout(ctypes.byref(dims), ctypes.byref(out)),
           "stepdllm_workspace_layout")
    return out


def build_mask(dims, sparsity, q, k, ws, row_ptr, col_idx, scores_out=None, stream=None,
               per_head=False):
    bf = torch.bfloat16
    fn = "stepdllm_build_mask_per_head" if per_head else "stepdllm_build_mask"
    _check(getattr(load(), fn)(
        ctypes.byref(dims), float(sparsity), _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _ptr(row_ptr, torch.int32, "row_ptr"),
        _ptr(col_idx, torch.int32, "col_idx"), _ptr(scores_out, torch.float32, "scores_out"),
        _stream(stream)), fn)


def select_mask(dims, sparsity, scores, ws, row_ptr, col_idx, stream=None, per_head=False):
    fn = "stepdllm_select_mask_per_head" if per_head else "stepdllm_select_mask"
    _check(getattr(load(), fn)(
        ctypes.byref(dims), float(sparsity), _ptr(scores, torch.float32, "scores"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _ptr(row_ptr, torch.int32, "row_ptr"),
        _ptr(col_idx, torch.int32, "col_idx"), _stream(stream)), fn)


def plan(dims, row_ptr, col_idx, ws, nnz=None, stream=None):
    """Work order and records of the mask row_ptr / col_idx; nnz defaults to
    col_idx.numel()."""
    nnz = col_idx.numel() if nnz is None else int(nnz)
    _check(load().stepdllm_plan(ctypes.byref(dims), _ptr(row_ptr, torch.int32, "row_ptr"),
                                _ptr(col_idx, torch.int32, "col_idx"), nnz,
                                _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "stepdllm_plan")


def sparse_attn(dims, q, k, v, col_idx, ws, o, nnz=None, stream=None):
    """Sparse attention on the mask whose plan is in ws (col_idx: its lists);
    nnz defaults to col_idx.numel()."""
    bf = torch.bfloat16
    nnz = col_idx.numel() if nnz is None else int(nnz)
    _check(load().stepdllm_sparse_attn(
        ctypes.byref(dims), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(col_idx, torch.int32, "col_idx"), nnz,
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _ptr(o, bf, "o"), _stream(stream)),
        "stepdllm_sparse_attn")


def sparse_attn_group(dims, q, k, v, row_ptr, col_idx, o, nnz=None, stream=None):
    """GQA variant with group-shared K/V tiles (no plan, no workspace); nnz
    defaults to col_idx.numel()."""
    bf = torch.bfloat16
    nnz = col_idx.numel() if nnz is None else int(nnz)
    _check(load().stepdllm_sparse_attn_group(
        ctypes.byref(dims), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"), nnz,
        _ptr(o, bf, "o"), _stream(stream)), "stepdllm_sparse_attn_group")


def dense_attn(dims, q, k, v, o, stream=None):
    bf = torch.bfloat16
    _check(load().stepdllm_dense_attn(
        ctypes.byref(dims), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(o, bf, "o"), _stream(stream)), "stepdllm_dense_attn")


def block_mass(dims, q, k, mass, stream=None):
    """True block attention mass, fp32 [H, nb, nb], into `mass`."""
    bf = torch.bfloat16
    _check(load().stepdllm_block_mass(ctypes.byref(dims), _ptr(q, bf, "q"), _ptr(k, bf, "k"),
                                      _ptr(mass, torch.float32, "mass"), _stream(stream)),
           "stepdllm_block_mass")


def mask_recall(dims, mass, row_ptr, col_idx, recall, nnz=None, stream=None):
    """Per-row recall [H*nb] of the mask (row_ptr, col_idx) against `mass`."""
    nnz = col_idx.numel() if nnz is None else int(nnz)
    _check(load().stepdllm_mask_recall(
        ctypes.byref(dims), _ptr(mass, torch.float32, "mass"),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"), nnz,
        _ptr(recall, torch.float32, "recall"), _stream(stream)), "stepdllm_mask_recall")


def keep_count_columns(dims, sparsity):
    """k_c: key columns kept per head by the column-sparse variant."""
    r = load().stepdllm_keep_count_columns(ctypes.byref(dims), float(sparsity))
    if r < 0:
        raise StepDLLMError(int(r), "stepdllm_keep_count_columns")
    return int(r)


def build_col_mask(dims, sparsity, q, k, ws, cols, scores_out=None, stream=None):
    """Column mask: per head the k_c kept key columns, ascending, into cols [H, k_c]."""
    bf = torch.bfloat16
    _check(load().stepdllm_build_col_mask(
        ctypes.byref(dims), float(sparsity), _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _ptr(cols, torch.int32, "cols"),
        _ptr(scores_out, torch.float32, "scores_out"), _stream(stream)),
        "stepdllm_build_col_mask")


def select_col_mask(dims, sparsity, scores, ws, cols, stream=None):
    _check(load().stepdllm_select_col_mask(
        ctypes.byref(dims), float(sparsity), _ptr(scores, torch.float32, "scores"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _ptr(cols, torch.int32, "cols"),
        _stream(stream)), "stepdllm_select_col_mask")


def col_attn(dims, q, k, v, cols, o, k_c=None, stream=None):
    """Every query of head h over the key tokens cols[h] ([H, k_c] int32)."""
    bf = torch.bfloat16
    k_c = (cols.shape[-1] if cols.dim() == 2 else 0) if k_c is None else int(k_c)
    _check(load().stepdllm_col_attn(
        ctypes.byref(dims), _ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
        _ptr(cols, torch.int32, "cols") if cols.numel() else None, k_c, _ptr(o, bf, "o"),
        _stream(stream)), "stepdllm_col_attn")


def col_recall(dims, q, k, cols, recall, k_c=None, stream=None):
    """Per-row recall [H*nb] of the column mask cols ([H, k_c] int32)."""
    bf = torch.bfloat16
    k_c = (cols.shape[-1] if cols.dim() == 2 else 0) if k_c is None else int(k_c)
    _check(load().stepdllm_col_recall(
        ctypes.byref(dims), _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        _ptr(cols, torch.int32, "cols") if cols.numel() else None, k_c,
        _ptr(recall, torch.float32, "recall"), _stream(stream)), "stepdllm_col_recall")


def step_noalloc(dims, dense_steps, refresh_every, sparsity, step, q, k, v, row_ptr, col_idx,
                 o, per_head_budget=False, column_sparse=False, stream=None):
    """One denoising step with the library's static workspace (no driver, no
    workspace argument); returns the status code (0 = ok) instead of raising,
    so callers can see a rejected shape."""
    bf = torch.bfloat16
    sched = Schedule(int(dense_steps), int(refresh_every), float(sparsity),
                     int(bool(per_head_budget)), int(bool(column_sparse)))
    return int(load().stepdllm_step_noalloc(
        ctypes.byref(dims), ctypes.byref(sched), int(step), _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        _ptr(v, bf, "v"), _ptr(row_ptr, torch.int32, "row_ptr"),
        _ptr(col_idx, torch.int32, "col_idx"), _ptr(o, bf, "o"), _stream(stream)))


class Driver:
    """Owns the C driver handle; buffers are torch device tensors kept alive here."""

    def __init__(self, dims, dense_steps, refresh_every, sparsity, device="cuda",
                 per_head_budget=False, column_sparse=False):
        self.dims = dims
        self.column_sparse = bool(column_sparse)
        if self.column_sparse:
            self.k_c = keep_count_columns(dims, sparsity)
            self.K = self.k_c * dims.n_q_heads
        else:
            self.K = keep_count(dims, sparsity, per_head_budget)
        rows = dims.n_q_heads * (dims.seq_len // dims.block)
        self.ws = torch.empty(workspace_bytes(dims), dtype=torch.uint8, device=device)
        self.row_ptr = None if self.column_sparse else torch.empty(rows + 1, dtype=torch.int32,
                                                                   device=device)
        self.col_idx = torch.empty(max(self.K, 1), dtype=torch.int32, device=device)
        self._h = _vp()
        sched = Schedule(int(dense_steps), int(refresh_every), float(sparsity),
                         int(bool(per_head_budget)), int(self.column_sparse))
        _check(load().stepdllm_driver_create(
            ctypes.byref(self._h), ctypes.byref(dims), ctypes.byref(sched), self.ws.data_ptr(),
            self.ws.numel(), None if self.row_ptr is None else self.row_ptr.data_ptr(),
            self.col_idx.data_ptr()), "stepdllm_driver_create")

    def cols(self):
        """Column mode: the kept columns [H, k_c] of the last anchor."""
        return self.col_idx[:self.K].view(self.dims.n_q_heads, self.k_c)

    def step_kind(self, step):
        r = load().stepdllm_driver_step_kind(self._h, int(step))
        if r < 0:
            raise StepDLLMError(r, "stepdllm_driver_step_kind")
        return r

    def step(self, step, q, k, v, o, stream=None):
        bf = torch.bfloat16
        _check(load().stepdllm_step(self._h, int(step), _ptr(q, bf, "q"), _ptr(k, bf, "k"),
                                    _ptr(v, bf, "v"), _ptr(o, bf, "o"), _stream(stream)),
               "stepdllm_step")

    def close(self):
        if self._h:
            load().stepdllm_driver_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MaskBuffers:
    """Workspace + CSR buffers for one shape and sparsity (torch device memory)."""

    def __init__(self, dims, sparsity, device="cuda", per_head=False):
        self.dims = dims
        self.sparsity = float(sparsity)
        self.K = keep_count(dims, sparsity, per_head)
        self.nb = dims.seq_len // dims.block
        self.rows = dims.n_q_heads * self.nb
        self.ws = torch.empty(workspace_bytes(dims), dtype=torch.uint8, device=device)
        self.row_ptr = torch.empty(self.rows + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(max(self.K, 1), dtype=torch.int32, device=device)
        self.layout = workspace_layout(dims)

    def view(self, offset, count, dtype):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.ws[offset:offset + nbytes].view(dtype)

    def scores(self):
        return self.view(self.layout.scores, self.rows * self.nb, torch.float32)

    def pooled(self):
        H, Hkv, d = self.dims.n_q_heads, self.dims.n_kv_heads, self.dims.head_dim
        return (self.view(self.layout.pooled_q, H * self.nb * d, torch.float32),
                self.view(self.layout.pooled_k, Hkv * self.nb * d, torch.float32))

    def select_state(self):
        return self.view(self.layout.select, 16, torch.int32)

    def work_cap(self):
        """Positions per die of the work order: min(H, ceil(H/8) + 2) * nb."""
        H = self.dims.n_q_heads
        return min(H, -(-H // 8) + 2) * self.nb

    def work(self):
        return self.view(self.layout.work, 8 * self.work_cap(), torch.int32)

    def work_meta(self):
        return self.view(self.layout.work_meta, 16, torch.int32)

    def plan_check(self):
        """The plan check word (work_meta[7]): 0 after a plan; bit 0 set by a
        sparse launch on another col_idx, nnz or shape than planned, bit 1 by
        one that found a row's first list entries changed.  Reads device
        memory (synchronises the device)."""
        return int(self.work_meta()[7].item())

    def work_rec(self):
        """[8 * cap, 4] int32: row, list begin, list end, first two block ids."""
        return self.view(self.layout.work_rec, 32 * self.work_cap(), torch.int32).view(-1, 4)

    def head_select(self):
        return self.view(self.layout.head_select, 8 * self.dims.n_q_heads, torch.int32)
