"""The C ABI on the host: the library loads, exports every declared entry point,
and validates arguments before anything reaches the GPU (no compute calls)."""
import ctypes
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

from block_sparse_attention_pooled_amd import binding as B
from block_sparse_attention_pooled_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stepdllm.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(stepdllm_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.load()
    names = declared_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def dims(H=32, Hkv=32, L=8192, d=128, blk=64):
    return B.make_dims(H, Hkv, L, d, blk)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_keep_count_matches_exact_rationals(name):
    w = WORKLOADS[name]
    for s in w.sparsities:
        want = math.ceil((1 - Fraction(str(s))) * w.H * w.nb * w.nb)
        assert B.keep_count(dims(w.H, w.Hkv, w.L, w.d, w.B), s) == want


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_per_head_keep_count_matches_exact_rationals(name, olib):
    import oracle as O
    w = WORKLOADS[name]
    for s in w.sparsities:
        k_h = math.ceil((1 - Fraction(str(s))) * w.nb * w.nb)
        assert O.keep_count(w.nb * w.nb, s, olib) == k_h
        assert B.keep_count(dims(w.H, w.Hkv, w.L, w.d, w.B), s, per_head=True) == w.H * k_h


def test_keep_count_edges():
    d = dims(2, 2, 256, 64, 64)                  # N = 32
    assert B.keep_count(d, 0.0) == 32
    assert B.keep_count(d, 0.5) == 16
    assert B.keep_count(d, 0.999999) == 1
    assert B.keep_count(d, 1 - 1e-12) == 1       # (1-s)*N = 3.2e-11 > 0
    assert B.keep_count(d, 1.0) == 0             # s = 1 drops every block
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(B.StepDLLMError) as e:
            B.keep_count(d, bad)
        assert e.value.status == B.EINVAL


@pytest.mark.parametrize("shape,s,want", [
    ((32, 32, 65536, 128, 64), 0.956, 1476396),   # N = 2^25: 0.044 N = 1476395.008
    ((100, 100, 6400, 128, 64), 0.999999, 1),     # N = 10^6: (1 - s) N is exactly 1
    ((10, 10, 64, 64, 64), 0.3, 7),               # N = 10: the double is below 0.3
    ((10, 10, 64, 64, 64), 0.1, 9),               # ... and above 0.1
    ((125, 125, 512, 64, 64), 0.999, 8),          # N = 8000
])
def test_keep_count_exact_on_the_decimal(shape, s, want, olib):
    """The library's budget is the exact ceiling on the decimal s, equal to
    the oracle's and to Python's rational arithmetic on repr(s)."""
    import oracle as O
    H, Hkv, L, d, blk = shape
    n = H * (L // blk) ** 2
    assert math.ceil((1 - Fraction(repr(s))) * n) == want
    assert B.keep_count(dims(*shape), s) == want == O.keep_count(n, s, olib)


def test_keep_count_random_decimals(olib):
    import oracle as O
    rng = np.random.default_rng(11)
    d = dims(32, 32, 65536, 128, 64)             # N = 2^25
    for u in rng.random(300):
        s = float(f"{u:.{1 + int(u * 1000) % 9}g}")
        want = math.ceil((1 - Fraction(repr(s))) * 2 ** 25)
        assert B.keep_count(d, s) == want == O.keep_count(2 ** 25, s, olib), s


@pytest.mark.parametrize("args,status", [
    ((0, 1, 256, 64, 64), B.EINVAL),
    ((4, 3, 256, 64, 64), B.EINVAL),         # H % Hkv != 0
    ((2, 2, 200, 64, 64), B.EINVAL),         # L % B != 0
    ((2, 2, 256, 96, 64), B.EUNSUPPORTED),   # head_dim
    ((2, 2, 256, 64, 32), B.EUNSUPPORTED),   # block
    ((2, 2, 64 * 1025, 64, 64), B.EUNSUPPORTED),   # nb > 1024
    ((2, 2, -64, 64, 64), B.EINVAL),
])
def test_dims_validation(args, status):
    with pytest.raises(B.StepDLLMError) as e:
        B.workspace_bytes(B.make_dims(*args))
    assert e.value.status == status


def test_workspace_layout():
    for w in WORKLOADS.values():
        d = dims(w.H, w.Hkv, w.L, w.d, w.B)
        lay = B.workspace_layout(d)
        offs = [lay.pooled_q, lay.pooled_k, lay.scores, lay.select, lay.work, lay.work_meta,
                lay.head_select]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert lay.total == B.workspace_bytes(d)
        assert lay.scores - lay.pooled_k >= w.Hkv * w.nb * w.d * 4
        assert lay.select - lay.scores >= w.H * w.nb * w.nb * 4
        assert lay.col_scores - lay.head_select >= w.H * 8 * 4
        assert lay.col_stats - lay.col_scores >= w.H * w.L * 4
        assert lay.total - lay.col_stats >= w.H * w.nb * 8
        assert lay.head_select < lay.col_scores < lay.col_stats < lay.work_rec < lay.total
        assert lay.col_scores % 256 == 0 and lay.col_stats % 256 == 0 and lay.work_rec % 256 == 0
        cap = min(w.H, -(-w.H // 8) + 2) * w.nb
        assert lay.total - lay.work_rec >= 8 * cap * 16


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_column_keep_count_matches_exact_rationals(name, olib):
    import oracle as O
    w = WORKLOADS[name]
    for s in w.sparsities:
        k_c = math.ceil((1 - Fraction(str(s))) * w.L)
        assert O.keep_count(w.L, s, olib) == k_c
        assert B.keep_count_columns(dims(w.H, w.Hkv, w.L, w.d, w.B), s) == k_c


def test_entry_points_reject_bad_arguments_before_launch():
    lib = B.load()
    d = dims(2, 2, 256, 64, 64)
    ws_need = B.workspace_bytes(d)
    r = ctypes.byref
    # null pointers
    assert lib.stepdllm_build_mask(r(d), 0.5, None, FAKE, FAKE, ws_need, FAKE, FAKE, None, None) == B.EINVAL
    assert lib.stepdllm_sparse_attn(r(d), FAKE, FAKE, None, FAKE, 16, FAKE, ws_need, FAKE, None) == B.EINVAL
    assert lib.stepdllm_sparse_attn(r(d), FAKE, FAKE, FAKE, None, 16, FAKE, ws_need, FAKE, None) == B.EINVAL
    assert lib.stepdllm_dense_attn(r(d), FAKE, FAKE, FAKE, None, None) == B.EINVAL
    assert lib.stepdllm_sparse_attn_group(r(d), FAKE, FAKE, FAKE, None, FAKE, 16, FAKE, None) == B.EINVAL
    assert lib.stepdllm_sparse_attn_group(r(d), FAKE, FAKE, FAKE, FAKE, FAKE, 33, FAKE, None) == B.EINVAL
    assert lib.stepdllm_sparse_attn_group(r(dims(2, 2, 256, 64, 128)), FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None) == B.EUNSUPPORTED
    assert lib.stepdllm_select_mask(r(d), 0.5, None, FAKE, ws_need, FAKE, FAKE, None) == B.EINVAL
    assert lib.stepdllm_plan(r(d), None, FAKE, 16, FAKE, ws_need, None) == B.EINVAL
    assert lib.stepdllm_plan(r(d), FAKE, None, 16, FAKE, ws_need, None) == B.EINVAL
    assert lib.stepdllm_plan(r(d), FAKE, FAKE, 33, FAKE, ws_need, None) == B.EINVAL
    assert lib.stepdllm_plan(r(d), FAKE, FAKE, -1, FAKE, ws_need, None) == B.EINVAL
    assert lib.stepdllm_build_mask_per_head(r(d), 0.5, None, FAKE, FAKE, ws_need, FAKE, FAKE, None, None) == B.EINVAL
    assert lib.stepdllm_select_mask_per_head(r(d), 0.5, FAKE, FAKE, ws_need - 1, FAKE, FAKE, None) == B.EWORKSPACE
    assert lib.stepdllm_keep_count_per_head(r(d), 1.0001) == B.EINVAL
    assert lib.stepdllm_keep_count_per_head(r(d), 1.0) == 0
    assert lib.stepdllm_block_mass(r(d), FAKE, None, FAKE, None) == B.EINVAL
    assert lib.stepdllm_block_mass(r(dims(2, 2, 256, 80, 64)), FAKE, FAKE, FAKE, None) == B.EUNSUPPORTED
    assert lib.stepdllm_mask_recall(r(d), FAKE, FAKE, FAKE, 33, FAKE, None) == B.EINVAL
    assert lib.stepdllm_mask_recall(r(d), FAKE, None, FAKE, 16, FAKE, None) == B.EINVAL
    # column-sparse entry points
    assert lib.stepdllm_keep_count_columns(r(d), 1.0001) == B.EINVAL
    assert lib.stepdllm_keep_count_columns(r(d), 1.0) == 0
    assert lib.stepdllm_keep_count_columns(r(d), 0.0) == 256
    assert lib.stepdllm_build_col_mask(r(d), 0.5, FAKE, None, FAKE, ws_need, FAKE, None, None) == B.EINVAL
    assert lib.stepdllm_build_col_mask(r(d), 0.5, FAKE, FAKE, FAKE, ws_need, None, None, None) == B.EINVAL
    assert lib.stepdllm_build_col_mask(r(d), 0.5, FAKE, FAKE, FAKE, ws_need - 1, FAKE, None, None) == B.EWORKSPACE
    assert lib.stepdllm_build_col_mask(r(d), 1.5, FAKE, FAKE, FAKE, ws_need, FAKE, None, None) == B.EINVAL
    assert lib.stepdllm_select_col_mask(r(d), 0.5, None, FAKE, ws_need, FAKE, None) == B.EINVAL
    assert lib.stepdllm_select_col_mask(r(d), 0.5, FAKE, FAKE, 8, FAKE, None) == B.EWORKSPACE
    assert lib.stepdllm_col_attn(r(d), FAKE, FAKE, FAKE, FAKE, 257, FAKE, None) == B.EINVAL
    assert lib.stepdllm_col_attn(r(d), FAKE, FAKE, FAKE, FAKE, -1, FAKE, None) == B.EINVAL
    assert lib.stepdllm_col_attn(r(d), FAKE, FAKE, FAKE, None, 4, FAKE, None) == B.EINVAL
    assert lib.stepdllm_col_attn(r(d), FAKE, FAKE, None, FAKE, 4, FAKE, None) == B.EINVAL
    assert lib.stepdllm_col_attn(r(dims(2, 2, 256, 80, 64)), FAKE, FAKE, FAKE, FAKE, 4, FAKE, None) == B.EUNSUPPORTED
    assert lib.stepdllm_col_recall(r(d), FAKE, FAKE, None, 4, FAKE, None) == B.EINVAL
    assert lib.stepdllm_col_recall(r(d), FAKE, FAKE, FAKE, 257, FAKE, None) == B.EINVAL
    assert lib.stepdllm_col_recall(r(d), FAKE, FAKE, FAKE, 4, None, None) == B.EINVAL
    # sparsity out of range
    for s in (-0.5, 1.0000001, float("nan")):
        assert lib.stepdllm_build_mask(r(d), s, FAKE, FAKE, FAKE, ws_need, FAKE, FAKE, None, None) == B.EINVAL
    # workspace too small
    assert lib.stepdllm_build_mask(r(d), 0.5, FAKE, FAKE, FAKE, ws_need - 1, FAKE, FAKE, None, None) == B.EWORKSPACE
    assert lib.stepdllm_sparse_attn(r(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 8, FAKE, None) == B.EWORKSPACE
    assert lib.stepdllm_plan(r(d), FAKE, FAKE, 16, FAKE, 0, None) == B.EWORKSPACE
    # nnz outside [0, H*nb*nb]
    assert lib.stepdllm_sparse_attn(r(d), FAKE, FAKE, FAKE, FAKE, 33, FAKE, ws_need, FAKE, None) == B.EINVAL
    assert lib.stepdllm_sparse_attn(r(d), FAKE, FAKE, FAKE, FAKE, -1, FAKE, ws_need, FAKE, None) == B.EINVAL
    # unsupported dims on a compute entry point
    bad = dims(2, 2, 256, 80, 64)
    assert lib.stepdllm_dense_attn(r(bad), FAKE, FAKE, FAKE, FAKE, None) == B.EUNSUPPORTED


def _driver(d, dense, every, s, ws_bytes=None, per_head=0, columns=0, row_ptr=FAKE):
    lib = B.load()
    h = ctypes.c_void_p()
    sched = B.Schedule(dense, every, s, per_head, columns)
    st = lib.stepdllm_driver_create(ctypes.byref(h), ctypes.byref(d), ctypes.byref(sched), FAKE,
                                    B.workspace_bytes(d) if ws_bytes is None else ws_bytes,
                                    row_ptr, FAKE)
    return st, h


def test_driver_schedule_matches_oracle(olib):
    import oracle as O
    lib = B.load()
    for name, w in WORKLOADS.items():
        d = dims(w.H, w.Hkv, w.L, w.d, w.B)
        st, h = _driver(d, w.dense_steps, w.refresh_every, w.sparsities[0])
        assert st == B.OK
        try:
            got = [lib.stepdllm_driver_step_kind(h, t) for t in range(w.steps)]
            want = [O.step_kind(t, w.dense_steps, w.refresh_every, olib) for t in range(w.steps)]
            assert got == want, name
        finally:
            lib.stepdllm_driver_destroy(h)


def test_driver_rejects_reuse_before_anchor_and_bad_schedules():
    lib = B.load()
    d = dims(2, 2, 256, 64, 64)
    st, h = _driver(d, 0, 4, 0.5)
    assert st == B.OK
    try:
        # Step 1 is a reuse step; no anchor ran, so nothing is launched.
        assert lib.stepdllm_step(h, 1, FAKE, FAKE, FAKE, FAKE, None) == B.ESTATE
        assert lib.stepdllm_step(h, -1, FAKE, FAKE, FAKE, FAKE, None) == B.EINVAL
        assert lib.stepdllm_step(h, 0, FAKE, None, FAKE, FAKE, None) == B.EINVAL
    finally:
        lib.stepdllm_driver_destroy(h)
    assert _driver(d, -1, 4, 0.5)[0] == B.EINVAL
    assert _driver(d, 0, -4, 0.5)[0] == B.EINVAL
    assert _driver(d, 0, 4, 1.5)[0] == B.EINVAL
    assert _driver(d, 0, 4, 0.5, ws_bytes=16)[0] == B.EWORKSPACE
    assert _driver(d, 0, 4, 0.5, per_head=2)[0] == B.EINVAL
    st, h = _driver(d, 0, 4, 0.5, per_head=1)
    assert st == B.OK
    lib.stepdllm_driver_destroy(h)
    # Column mode: no row_ptr needed; the per-head block budget does not apply.
    assert _driver(d, 0, 4, 0.5, columns=2)[0] == B.EINVAL
    assert _driver(d, 0, 4, 0.5, columns=1, per_head=1)[0] == B.EINVAL
    assert _driver(d, 0, 4, 0.5, row_ptr=None)[0] == B.EINVAL
    st, h = _driver(d, 0, 4, 0.5, columns=1, row_ptr=None)
    assert st == B.OK
    try:
        assert lib.stepdllm_step(h, 1, FAKE, FAKE, FAKE, FAKE, None) == B.ESTATE
    finally:
        lib.stepdllm_driver_destroy(h)


def test_status_strings():
    for st in (B.OK, B.EINVAL, B.EUNSUPPORTED, B.EWORKSPACE, B.EHIP, B.ESTATE):
        assert B.status_string(st) and B.status_string(st) != "unknown status"
    assert B.status_string(-99) == "unknown status"


def test_library_has_no_undefined_kernel_stubs():
    """Every kernel's host launch stub is defined (a host pass that drops a
    kernel leaves an undefined stub and the library fails to load on a GPU)."""
    import subprocess
    out = subprocess.run(["nm", "-D", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "__device_stub__" in l]
    assert not undefined, undefined


def test_step_noalloc_validates_before_touching_the_gpu():
    """The allocation-free step rejects bad arguments and shapes whose
    workspace exceeds its static array before any HIP call."""
    lib = B.load()
    r = ctypes.byref
    d = dims(2, 2, 256, 64, 64)
    sched = B.Schedule(0, 4, 0.5, 0, 0)
    f = lib.stepdllm_step_noalloc
    assert f(r(d), None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.EINVAL
    assert f(r(d), r(sched), -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.EINVAL
    assert f(r(d), r(sched), 0, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == B.EINVAL
    assert f(r(d), r(sched), 0, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == B.EINVAL
    assert f(r(d), r(B.Schedule(0, 4, 1.5, 0, 0)), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
             None) == B.EINVAL
    assert f(r(d), r(B.Schedule(0, 4, 0.5, 1, 1)), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
             None) == B.EINVAL
    assert f(r(dims(2, 2, 256, 80, 64)), r(sched), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
             None) == B.EUNSUPPORTED
    big = dims(64, 64, 65536, 128, 128)
    assert B.workspace_bytes(big) > 80 << 20
    assert f(r(big), r(sched), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.EWORKSPACE
    # Every workload of the benchmark fits the static array.
    for w in WORKLOADS.values():
        assert B.workspace_bytes(dims(w.H, w.Hkv, w.L, w.d, w.B)) <= 80 << 20, w.name
