"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with what the mathematics fixes:
closed forms, worked examples whose answer is derived by hand, invariants,
and brute force written in a different formulation (whole-matrix numpy fp64
instead of the oracle's per-row list loops).  The mutation tests run every
pin against deliberately broken copies of the oracle to show that the pins
can fail.
"""
import math
import os
from fractions import Fraction

import numpy as np

import oracle as O

RNG_SEEDS = (11, 12, 13)


def _bf16_round(x):
    """Round fp32 numpy values to bf16 (RNE), kept as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lists(name):
    """A hand-derived fixture under tests/golden/: '# ...' lines are its
    citation and derivation, every other line is 'key: id id ...'."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, ids = line.partition(":")
            out[int(key)] = [int(x) for x in ids.split()]
    return out


def _rand(shape, rng, scale=1.0):
    return _bf16_round(rng.standard_normal(shape).astype(np.float32) * scale)


def _expand_block_mask(keep, B):
    """[H, nb, nb] block mask -> [H, L, L] token mask."""
    return np.repeat(np.repeat(keep.astype(bool), B, axis=1), B, axis=2)


def brute_attention(q, k, v, token_mask):
    """Whole-matrix fp64 masked softmax attention; fully masked rows give 0."""
    H, L, d = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    out = np.zeros((H, L, d))
    for h in range(H):
        g = h // G
        s = q[h].astype(np.float64) @ k[g].astype(np.float64).T / math.sqrt(d)
        m = token_mask[h]
        s = np.where(m, s, -np.inf)
        rowmax = s.max(axis=1, keepdims=True)
        live = np.isfinite(rowmax[:, 0])
        e = np.zeros_like(s)
        e[live] = np.exp(s[live] - rowmax[live])
        den = e.sum(axis=1, keepdims=True)
        den[~live] = 1.0
        out[h] = (e / den) @ v[g].astype(np.float64)
    return out


# ------------------------------------------------------------------ budget --
def pin_keep_count(lib):
    """K = ceil((1-s)*N) in exact rational arithmetic on the decimal s the
    caller wrote (Python's repr: the shortest decimal that reads back as the
    same double), for every workload size and for cases where binary
    representation error or a relative guard would change the answer."""
    cases = [(32, "0.5"), (32768, "0.9"), (524288, "0.9"), (458752, "0.7"), (458752, "0.8"),
             (458752, "0.9"), (458752, "0.95"), (8388608, "0.95"), (64, "0.75"), (96, "0"),
             (100, "0.99"), (7, "0.5"), (1, "0.5"), (2 ** 25, "0.956"), (10, "0.3"),
             (10, "0.1"), (10 ** 6, "0.999999"), (8000, "0.999"), (2 ** 30, "0.123457"),
             (2 ** 20, "1e-07"), (32, "0.999999999999"), (5, "1"), (2 ** 30, "1e-300")]
    for n, s in cases:
        assert repr(float(s)) == s or float(s) in (0.0, 1.0), s
        want = math.ceil((1 - Fraction(s)) * n)
        got = O.keep_count(n, float(s), lib)
        assert got == want, (n, s, got, want)
    # Random decimals of 1 to 9 digits, and powers of two with their upper
    # neighbours (at a power of two the double's rounding interval is
    # lopsided, so repr may pick a decimal that is not the nearest one of its
    # length; s * N is then dyadic and the two decimals give the same K).
    rng = np.random.default_rng(7)
    for u in rng.random(400):
        s = float(f"{u:.{1 + int(u * 1000) % 9}g}")
        n = int(rng.integers(1, 2 ** 31))
        assert O.keep_count(n, s, lib) == math.ceil((1 - Fraction(repr(s))) * n), (n, s)
    for k in range(1, 60):
        for s in (2.0 ** -k, np.nextafter(2.0 ** -k, 1.0)):
            s = float(s)
            n = 2 ** 30 + 12345
            assert O.keep_count(n, s, lib) == math.ceil((1 - Fraction(repr(s))) * n), (n, s)
    # Values written out by hand.
    assert O.keep_count(524288, 0.9, lib) == 52429
    assert O.keep_count(8388608, 0.95, lib) == 419431
    assert O.keep_count(32, 0.5, lib) == 16
    assert O.keep_count(2 ** 25, 0.956, lib) == 1476396     # (0.044 * 2^25 = 1476395.008)
    assert O.keep_count(10, 0.3, lib) == 7                  # the double is below 0.3
    assert O.keep_count(10 ** 6, 0.999999, lib) == 1        # 1 - s carries 1e-11 relative error
    assert O.keep_count(32, 1.0, lib) == 0
    assert O.keep_count(32, 0.0, lib) == 32


# -------------------------------------------------------------------- pool --
def pin_pool(lib):
    # Closed form: a ramp x[h,t,c] = t + c/4 has block means i*B + (B-1)/2 + c/4.
    for B in (64, 128):
        H, L, d = 3, 4 * B, 64
        t = np.arange(L, dtype=np.float32)[None, :, None]
        c = np.arange(d, dtype=np.float32)[None, None, :] / 4
        x = np.broadcast_to(t + c + np.arange(H, dtype=np.float32)[:, None, None] * 1000,
                            (H, L, d)).astype(np.float32)
        got = O.pool(x, B, lib)
        i = np.arange(L // B, dtype=np.float64)[None, :, None]
        want = (i * B + (B - 1) / 2 + np.arange(d)[None, None, :] / 4
                + np.arange(H)[:, None, None] * 1000)
        assert np.array_equal(got.astype(np.float64), want), "ramp block mean"
    # Random data: within fp32 summation error of the fp64 mean.
    rng = np.random.default_rng(RNG_SEEDS[0])
    x = _rand((2, 256, 128), rng)
    got = O.pool(x, 64, lib).astype(np.float64)
    want = x.astype(np.float64).reshape(2, 4, 64, 128).mean(axis=2)
    assert np.max(np.abs(got - want)) <= 64 * 2 ** -24 * np.max(np.abs(x)), "random block mean"


# ---------------------------------------------------------- score/softmax --
def pin_scores(lib):
    rng = np.random.default_rng(RNG_SEEDS[1])
    # Q = 0: every pooled score is 0, so every softmax row is exactly 1/nb.
    qb = np.zeros((3, 8, 64), np.float32)
    kb = _rand((3, 8, 64), rng)
    P = O.scores(qb, kb, lib)
    assert np.all(P == np.float32(1 / 8)), "uniform rows"
    # fp64 definition with the GQA map g(h) = h // (H/Hkv), H=6, Hkv=2.
    for d in (64, 128):
        qb = _rand((6, 16, d), rng, 0.3)
        kb = _rand((2, 16, d), rng, 0.3)
        P = O.scores(qb, kb, lib).astype(np.float64)
        G = 3
        for h in range(6):
            s = qb[h].astype(np.float64) @ kb[h // G].astype(np.float64).T / math.sqrt(d)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            want = e / e.sum(axis=1, keepdims=True)
            rel = np.max(np.abs(P[h] - want) / want)
            assert rel < 2e-6, (d, h, rel)
        assert np.allclose(P.sum(axis=2), 1.0, atol=2e-6)


# ------------------------------------------------------------------ select --
def _brute_select(P, K):
    flat = P.reshape(-1).astype(np.float64)
    order = np.lexsort((np.arange(flat.size), -flat))   # value desc, then index asc
    keep = np.zeros(flat.size, np.uint8)
    keep[order[:K]] = 1
    return keep.reshape(P.shape)


def pin_select(lib):
    rng = np.random.default_rng(RNG_SEEDS[2])
    # Many exact ties: values drawn from 5 levels.
    for n_levels, shape in ((5, (2, 8, 8)), (3, (4, 4, 4)), (50, (3, 16, 16))):
        levels = np.sort(rng.random(n_levels)).astype(np.float32)
        P = levels[rng.integers(0, n_levels, size=shape)]
        N = P.size
        for K in (0, 1, N // 3, N // 2, N - 1, N):
            got = O.select(P, K, lib)
            assert np.array_equal(got, _brute_select(P, K)), (shape, K)
            assert int(got.sum()) == K
    # All equal: the first K flat indices.
    P = np.full((2, 4, 4), 0.25, np.float32)
    for K in (0, 5, 16, 31, 32):
        got = O.select(P, K, lib).reshape(-1)
        assert np.array_equal(got, (np.arange(32) < K).astype(np.uint8)), K
    # The cut value is the K-th largest.
    P = rng.random((2, 8, 8)).astype(np.float32)
    assert O.cut_value(P, 10, lib) == np.sort(P.reshape(-1))[::-1][9]


def _check_top_k(vals, keep, k):
    """keep (bool, flat order) holds exactly the k largest of vals, ties at the
    cut going to the lowest indices: the properties that fix a top-k uniquely."""
    kept, dropped = np.nonzero(keep)[0], np.nonzero(~keep)[0]
    assert kept.size == k
    if kept.size == 0 or dropped.size == 0:
        return
    lo, hi = vals[kept].min(), vals[dropped].max()
    assert lo >= hi, (lo, hi)
    if lo == hi:
        assert kept[vals[kept] == lo].max() < dropped[vals[dropped] == hi].min()


def pin_select_per_head(lib):
    rng = np.random.default_rng(RNG_SEEDS[2] + 11)
    for n_levels, shape in ((4, (3, 8, 8)), (40, (2, 16, 16)), (2, (5, 4, 4))):
        levels = np.sort(rng.random(n_levels)).astype(np.float32)
        P = levels[rng.integers(0, n_levels, size=shape)]
        per = shape[1] * shape[2]
        for k in (0, 1, per // 3, per // 2, per - 1, per):
            keep = O.select_per_head(P, k, lib).astype(bool)
            for h in range(shape[0]):
                _check_top_k(P[h].reshape(-1), keep[h].reshape(-1), k)
            # One head alone is the global select.
            assert np.array_equal(O.select_per_head(P[:1], k, lib), O.select(P[:1], k, lib))
        # A head's choice does not depend on the other heads' scores.
        k = per // 2
        base = O.select_per_head(P, k, lib)
        P2 = P.copy()
        P2[1:] = rng.random(P2[1:].shape).astype(np.float32)
        assert np.array_equal(O.select_per_head(P2, k, lib)[0], base[0])


def pin_csr(lib):
    rng = np.random.default_rng(RNG_SEEDS[0] + 7)
    keep = (rng.random((3, 8, 8)) < 0.3).astype(np.uint8)
    keep[1, 2, :] = 0            # one empty row
    row_ptr, col_idx = O.csr(keep, lib)
    flat = keep.reshape(24, 8)
    assert row_ptr[0] == 0 and np.array_equal(np.diff(row_ptr), flat.sum(axis=1))
    for r in range(24):
        assert np.array_equal(col_idx[row_ptr[r]:row_ptr[r + 1]], np.nonzero(flat[r])[0])


def _die_lists(lens, H, nb, B):
    """The die lists of the work-order spec written out in Python: heads by
    weight (B/32)*kept + 4*nonempty rows (descending, then id) to the
    least-loaded die with room for min(H, ceil(H/8) + 2) heads; each die lists
    the non-empty rows of its heads in that order (rows by length desc, ties by
    row id), then the empty rows of its heads in that order (ascending)."""
    cap_h = min(H, -(-H // 8) + 2)
    weight = [(B // 32) * int(sum(lens[h * nb:(h + 1) * nb]))
              + 4 * int(sum(1 for r in range(h * nb, (h + 1) * nb) if lens[r] > 0))
              for h in range(H)]
    dies = [[] for _ in range(8)]
    load = [0] * 8
    for h in sorted(range(H), key=lambda h: (-weight[h], h)):
        x = min((x for x in range(8) if len(dies[x]) < cap_h), key=lambda x: (load[x], x))
        dies[x].append(h)
        load[x] += weight[h]
    out = []
    for x in range(8):
        full = [r for h in dies[x] for r in sorted(range(h * nb, (h + 1) * nb),
                                                   key=lambda r: (-lens[r], r)) if lens[r] > 0]
        empty = [r for h in dies[x] for r in range(h * nb, (h + 1) * nb) if lens[r] <= 0]
        out.append(full + empty)
    return out


def pin_plan(lib):
    # Hand-derived: H=3, nb=4, B=64 (2 steps of 32 keys per block), one head
    # per die.  Kept blocks per head 5, 9, 5 over 2, 3, 4 non-empty rows, so
    # the weights are 2*5 + 4*2 = 18, 2*9 + 4*3 = 30, 2*5 + 4*4 = 26: head 1 ->
    # die 0, head 2 -> die 1, head 0 -> die 2 (by kept blocks alone, heads 0
    # and 2 would tie and head 0 would come first); dies 3..7 stay empty.  A
    # die may hold min(3, 1 + 2) = 3 heads, so 12 positions per die.
    lens = np.array([2, 0, 3, 0,   4, 1, 4, 0,   1, 1, 1, 2])
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, n = O.plan(row_ptr, 3, 4, 64, lib)
    pad = [-1] * 8
    want = [4, 6, 5, 7] + pad + [11, 8, 9, 10] + pad + [2, 0, 1, 3] + pad + [-1] * 60
    assert list(work) == want and n == 9
    # The same mask with B=128 (4 steps per block): weights 28, 48, 36, same
    # order.
    work, n = O.plan(row_ptr, 3, 4, 128, lib)
    assert list(work) == want and n == 9
    # Block size decides: head 0 keeps two rows of 1 block, head 1 one row of
    # 4.  B=64: weights 2*2 + 8 = 12 and 2*4 + 4 = 12 tie, head 0 -> die 0.
    # B=128: 4*2 + 8 = 16 against 4*4 + 4 = 20, head 1 -> die 0.
    lens = np.array([1, 1, 4, 0])
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, n = O.plan(row_ptr, 2, 2, 64, lib)
    assert list(work) == [0, 1, -1, -1, 2, 3, -1, -1] + [-1] * 24 and n == 3
    work, n = O.plan(row_ptr, 2, 2, 128, lib)
    assert list(work) == [2, 3, -1, -1, 0, 1, -1, -1] + [-1] * 24 and n == 3
    # Hand-derived die choice: H=9, nb=4, B=64, 4 positions per head, a die
    # may hold min(9, 2 + 2) = 4 heads (16 positions).  Head 0 keeps one row of
    # 3 blocks (weight 6 + 4 = 10), head 1 three rows of 1 block (6 + 12 =
    # 18), heads 2..7 one row of 4 blocks (8 + 4 = 12), head 8 one row of 1
    # block (2 + 4 = 6).  Order: head 1, heads 2..7, head 0, head 8; heads
    # 1..7 take dies 0..6, head 0 die 7 (load 10) and head 8 the least-loaded
    # die, die 7.  (By kept blocks alone, head 8 would join head 0 on die 6.)
    # Die 7 lists the two heads' non-empty rows, 0 and 32, before their empty
    # rows 1, 2, 3 and 33, 34, 35.
    lens = np.zeros(9 * 4, np.int64)
    lens[0] = 3
    lens[4:7] = 1
    for h in range(2, 8):
        lens[4 * h] = 4
    lens[32] = 1
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, n = O.plan(row_ptr, 9, 4, 64, lib)
    assert n == 11 and len(work) == 8 * 16
    assert list(work[:16]) == [4, 5, 6, 7] + [-1] * 12
    for x in range(1, 7):
        assert list(work[16 * x:16 * (x + 1)]) == [4 * (x + 1) + c for c in range(4)] + [-1] * 12, x
    assert list(work[112:]) == [0, 32, 1, 2, 3, 33, 34, 35] + [-1] * 8
    # Head cap slack: 12 heads of kept 30, 1, 1, ..., 1 with 8 dies (weights
    # 2*30 + 4*2 = 68 and 2 + 4 = 6): each die may hold min(12, 2 + 2) = 4
    # heads.  Head 0 -> die 0; heads 1..7 -> dies 1..7; heads 8..11 go to the
    # lightest dies, 1..4, never to die 0.  Within a die, heads in assignment
    # order, non-empty rows first: die x in 1..4 lists 2x, 2(x+7), then the
    # empty rows 2x+1, 2(x+7)+1.
    lens = np.zeros(12 * 2, np.int64)
    lens[0], lens[1] = 20, 10
    for h in range(1, 12):
        lens[2 * h] = 1
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, n = O.plan(row_ptr, 12, 2, 64, lib)
    cap = 8
    assert len(work) == 8 * cap and n == 13
    assert list(work[:cap]) == [0, 1] + [-1] * 6
    for x in range(1, 5):
        assert list(work[x * cap:(x + 1) * cap]) == [2 * x, 2 * (x + 7), 2 * x + 1,
                                                     2 * (x + 7) + 1] + [-1] * 4, x
    for x in range(5, 8):
        assert list(work[x * cap:(x + 1) * cap]) == [2 * x, 2 * x + 1] + [-1] * 6, x
    # Hand-derived row order: one head of 5 rows with lengths 2, 4, 1, 3, 2:
    # longest first, the two of length 2 by row id.
    lens = np.array([2, 4, 1, 3, 2])
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, n = O.plan(row_ptr, 1, 5, 64, lib)
    assert list(work[:5]) == [1, 3, 0, 4, 2] and all(w == -1 for w in work[5:])
    assert len(work) == 8 * 5 and n == 5
    # Random shapes (several heads per die) against the spec written out.
    rng = np.random.default_rng(RNG_SEEDS[1] + 7)
    for H, nb, B in ((20, 6, 64), (28, 9, 128), (8, 5, 64), (33, 3, 64), (17, 12, 128)):
        lens = rng.integers(0, nb + 1, size=H * nb) * (rng.random(H * nb) < 0.7)
        lens[: nb] = 0                                  # one head keeps nothing
        row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        work, n = O.plan(row_ptr, H, nb, B, lib)
        cap = min(H, -(-H // 8) + 2) * nb
        want = []
        for lst in _die_lists(lens, H, nb, B):
            want += lst + [-1] * (cap - len(lst))
        assert list(work) == want
        assert n == int((lens > 0).sum())


# --------------------------------------------------------------- attention --
def _random_mask(H, nb, rng, frac):
    keep = (rng.random((H, nb, nb)) < frac).astype(np.uint8)
    return keep


def pin_attention_brute(lib):
    rng = np.random.default_rng(RNG_SEEDS[2] + 7)
    for (H, Hkv, nb, d, B) in ((2, 2, 4, 64, 64), (4, 2, 3, 128, 64), (3, 1, 2, 64, 128)):
        L = nb * B
        q, k, v = _rand((H, L, d), rng), _rand((Hkv, L, d), rng), _rand((Hkv, L, d), rng)
        keep = _random_mask(H, nb, rng, 0.5)
        keep[0, 0, :] = 0                      # an empty row
        row_ptr, col_idx = O.csr(keep, lib)
        got = O.sparse_attn(q, k, v, B, row_ptr, col_idx, lib=lib)
        want = brute_attention(q, k, v, _expand_block_mask(keep, B))
        assert np.max(np.abs(got - want)) < 1e-12, ("sparse", H, Hkv, nb, d, B)
        assert np.all(got[0, :B] == 0.0), "empty row is zero"
        gd = O.dense_attn(q, k, v, B, lib=lib)
        wd = brute_attention(q, k, v, np.ones((H, L, L), bool))
        assert np.max(np.abs(gd - wd)) < 1e-12, ("dense", H, Hkv, nb, d, B)
        # A row subset writes exactly those rows.
        rows = np.array([H * nb - 1, 1], np.int32)
        part = O.sparse_attn(q, k, v, B, row_ptr, col_idx, rows=rows, lib=lib)
        for r in rows:
            h, i = divmod(int(r), nb)
            assert np.array_equal(part[h, i * B:(i + 1) * B], got[h, i * B:(i + 1) * B])


def pin_attention_closed_forms(lib):
    rng = np.random.default_rng(RNG_SEEDS[0] + 17)
    H, Hkv, nb, d, B = 4, 2, 4, 64, 64
    L = nb * B
    q, k = _rand((H, L, d), rng), _rand((Hkv, L, d), rng)
    keep = _random_mask(H, nb, rng, 0.4)
    keep[1, 3, :] = 0
    keep[2, 0, :] = 1
    row_ptr, col_idx = O.csr(keep, lib)
    rows_nonempty = keep.reshape(H * nb, nb).any(axis=1)
    # Constant V = c gives O = c on every non-empty row.
    c = np.float32(-1.5)
    v = np.full((Hkv, L, d), c, np.float32)
    o = O.sparse_attn(q, k, v, B, row_ptr, col_idx, lib=lib).reshape(H * nb, B, d)
    assert np.all(np.abs(o[rows_nonempty] - c) < 1e-12) and np.all(o[~rows_nonempty] == 0)
    # Q = 0 gives the mean of V over the kept blocks' tokens.
    v = _rand((Hkv, L, d), rng)
    o = O.sparse_attn(np.zeros_like(q), k, v, B, row_ptr, col_idx, lib=lib)
    for h in range(H):
        for i in range(nb):
            kept = np.nonzero(keep[h, i])[0]
            want = (v[h // 2].astype(np.float64).reshape(nb, B, d)[kept].reshape(-1, d).mean(axis=0)
                    if kept.size else np.zeros(d))
            assert np.max(np.abs(o[h, i * B:(i + 1) * B] - want)) < 1e-12, (h, i)
    # s = 0 keeps everything: sparse equals dense.
    full = np.ones((H, nb, nb), np.uint8)
    rp, ci = O.csr(full, lib)
    a = O.sparse_attn(q, k, v, B, rp, ci, lib=lib)
    b = O.dense_attn(q, k, v, B, lib=lib)
    assert np.max(np.abs(a - b)) < 1e-12
    # GQA: H=4 over Hkv=2 equals H=4 over Hkv=4 with each key head duplicated.
    k4, v4 = np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0)
    a = O.sparse_attn(q, k, v, B, row_ptr, col_idx, lib=lib)
    b = O.sparse_attn(q, k4, v4, B, row_ptr, col_idx, lib=lib)
    assert np.array_equal(a, b)


# ------------------------------------------------------- worked examples --
def worked_example_w1():
    """H=Hkv=2, d=64, L=256, B=64 (nb=4), s=0.5 -> K=16.

    Head 0: every query token of block i is 20*e_i and every key token of
    block j is 20*e_j, so S_ij = 400/8 * [i == j] = 50 [i == j]; each row's
    softmax is 1 on the diagonal and e^-50 / (1 + 3 e^-50) elsewhere.
    Head 1: Q = 0, so every score is exactly 1/4.
    The 16 largest: head 0's four diagonal ones (value 1), then twelve 0.25s
    of head 1 in lowest flat order -- rows 0, 1, 2 of head 1 complete, row 3
    of head 1 empty.  The concentrated head keeps one block per row.
    """
    rng = np.random.default_rng(5)
    H, d, B, nb = 2, 64, 64, 4
    L = nb * B
    q = np.zeros((H, L, d), np.float32)
    k = _rand((H, L, d), rng)
    for i in range(nb):
        q[0, i * B:(i + 1) * B, i] = 20.0
        k[0, i * B:(i + 1) * B, :] = 0.0
        k[0, i * B:(i + 1) * B, i] = 20.0
    v = _rand((H, L, d), rng)
    keep = np.zeros((H, nb, nb), np.uint8)
    for i in range(nb):
        keep[0, i, i] = 1
    keep[1, 0:3, :] = 1
    return q, k, v, keep


def pin_worked_w1(lib):
    q, k, v, keep_want = worked_example_w1()
    B = 64
    m = O.build_mask(q, k, B, 0.5, lib)
    P = m["P"]
    assert m["K"] == 16
    for i in range(4):
        assert P[0, i, i] == np.float32(1.0)
        for j in range(4):
            if j != i:
                assert abs(P[0, i, j] / math.exp(-50) - 1) < 1e-6
    assert np.all(P[1] == np.float32(0.25))
    keep = np.zeros(P.shape, np.uint8)
    for r in range(8):
        keep.reshape(8, 4)[r, m["col_idx"][m["row_ptr"][r]:m["row_ptr"][r + 1]]] = 1
    assert np.array_equal(keep, keep_want)
    want = golden_lists("w1_global_mask.txt")
    assert sorted(want) == list(range(8))
    for r, cols in want.items():
        assert list(m["col_idx"][m["row_ptr"][r]:m["row_ptr"][r + 1]]) == cols, r
    o = O.sparse_attn(q, k, v, B, m["row_ptr"], m["col_idx"], lib=lib)
    for i in range(4):
        want = v[0, i * B:(i + 1) * B].astype(np.float64).mean(axis=0)
        assert np.max(np.abs(o[0, i * B:(i + 1) * B] - want)) < 1e-12
    want1 = v[1].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(o[1, :3 * B] - want1)) < 1e-12
    assert np.all(o[1, 3 * B:] == 0)


def pin_worked_w1_per_head(lib):
    """W1 under the uniform per-head budget: each head keeps k_h = 8 of 16.
    Head 0 keeps its diagonal (value 1) and the four lowest-index blocks among
    its equal off-diagonal scores, (0,1), (0,2), (0,3), (1,0); head 1 keeps its
    first 8 flat positions, rows 0 and 1 whole, rows 2 and 3 empty."""
    q, k, v, _ = worked_example_w1()
    B = 64
    m = O.build_mask(q, k, B, 0.5, lib, per_head=True)
    assert m["K"] == 16
    want = golden_lists("w1_per_head_mask.txt")
    assert sorted(want) == list(range(8))
    rp, ci = m["row_ptr"], m["col_idx"]
    for r, cols in want.items():
        assert list(ci[rp[r]:rp[r + 1]]) == cols, (r, list(ci[rp[r]:rp[r + 1]]))
    o = O.sparse_attn(q, k, v, B, rp, ci, lib=lib)
    # Head 0: the own block outweighs the others by e^50.
    for i in range(4):
        want0 = v[0, i * B:(i + 1) * B].astype(np.float64).mean(axis=0)
        assert np.max(np.abs(o[0, i * B:(i + 1) * B] - want0)) < 1e-12
    want1 = v[1].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(o[1, :2 * B] - want1)) < 1e-12
    assert np.all(o[1, 2 * B:] == 0)


def pin_block_mass(lib):
    """A[h,i,j]: whole-matrix fp64 softmax (numpy matmul, a different
    formulation) summed over blocks; rows sum to 1; Q = 0 gives 1/nb; the W1
    concentrated head in closed form; a row subset equals the full map."""
    rng = np.random.default_rng(RNG_SEEDS[1] + 21)
    H, Hkv, L, d, B = 4, 2, 256, 64, 64
    nb = L // B
    q = _rand((H, L, d), rng) * 2.0
    k = _rand((Hkv, L, d), rng)
    A = O.block_mass(q, k, B, lib=lib)
    want = np.zeros_like(A)
    for h in range(H):
        S = q[h].astype(np.float64) @ k[h // (H // Hkv)].astype(np.float64).T / math.sqrt(d)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        want[h] = P.reshape(nb, B, nb, B).sum(axis=(1, 3)) / B
    assert np.max(np.abs(A - want)) < 1e-12
    assert np.max(np.abs(A.sum(axis=2) - 1.0)) < 1e-12
    rows = [1, 6, 13]
    part = O.block_mass(q, k, B, rows=rows, lib=lib)
    for r in range(H * nb):
        got = part.reshape(H * nb, nb)[r]
        assert np.array_equal(got, A.reshape(H * nb, nb)[r]) if r in rows else not got.any()
    assert np.max(np.abs(O.block_mass(np.zeros_like(q), k, B, lib=lib) - 1.0 / nb)) < 1e-15
    qw, kw, _, _ = worked_example_w1()
    Aw = O.block_mass(qw, kw, 64, lib=lib)
    e = math.exp(-50)
    for i in range(4):
        for j in range(4):
            w = 1 / (1 + 3 * e) if i == j else e / (1 + 3 * e)
            assert abs(Aw[0, i, j] / w - 1) < 1e-12, (i, j)


def pin_mask_recall(lib):
    rng = np.random.default_rng(RNG_SEEDS[1] + 22)
    A = rng.random((3, 5, 5))
    A /= A.sum(axis=2, keepdims=True)
    keep = (rng.random((3, 5, 5)) < 0.4).astype(np.uint8)
    keep[0, 1, :] = 0        # an empty row recalls nothing
    keep[2, 3, :] = 1        # a full row recalls everything
    rp, ci = O.csr(keep, lib)
    rec = O.mask_recall(A, rp, ci, lib)
    assert np.allclose(rec, (A * keep).sum(axis=2).reshape(-1), rtol=0, atol=1e-15)
    assert rec[1] == 0.0 and abs(rec[2 * 5 + 3] - 1.0) < 1e-15


def pin_worked_w2(lib):
    """Q = 0 for every head: every score is 1/nb and the mask is the first K
    flat indices, whatever the sparsity."""
    rng = np.random.default_rng(6)
    H, Hkv, nb, d, B = 4, 2, 8, 128, 64
    L = nb * B
    q = np.zeros((H, L, d), np.float32)
    k = _rand((Hkv, L, d), rng)
    for s in (0.0, 0.3, 0.5, 0.9, 0.97):
        m = O.build_mask(q, k, B, s, lib)
        K = math.ceil((1 - Fraction(str(s))) * H * nb * nb)
        assert m["K"] == K
        flat = np.zeros(H * nb * nb, np.uint8)
        for r in range(H * nb):
            flat[r * nb + m["col_idx"][m["row_ptr"][r]:m["row_ptr"][r + 1]]] = 1
        assert np.array_equal(flat, (np.arange(H * nb * nb) < K).astype(np.uint8)), s


def pin_build_mask_brute(lib):
    """The mask of build_mask equals a brute-force sort of fp64-recomputed
    scores wherever the fp64 value is not within 1e-5 of the cut."""
    rng = np.random.default_rng(7)
    H, Hkv, nb, d, B = 4, 2, 8, 64, 64
    L = nb * B
    q = _rand((H, L, d), rng) * np.array([0.5, 1, 2, 4], np.float32)[:, None, None]
    q = _bf16_round(q)
    k = _rand((Hkv, L, d), rng)
    m = O.build_mask(q, k, B, 0.8, lib)
    qb = q.astype(np.float64).reshape(H, nb, B, d).mean(axis=2)
    kb = k.astype(np.float64).reshape(Hkv, nb, B, d).mean(axis=2)
    P64 = np.empty((H, nb, nb))
    for h in range(H):
        s = qb[h] @ kb[h // 2].T / math.sqrt(d)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        P64[h] = e / e.sum(axis=1, keepdims=True)
    assert np.max(np.abs(m["P"] - P64) / P64) < 2e-6
    K = m["K"]
    want = _brute_select(P64, K).reshape(-1)
    got = np.zeros(H * nb * nb, np.uint8)
    for r in range(H * nb):
        got[r * nb + m["col_idx"][m["row_ptr"][r]:m["row_ptr"][r + 1]]] = 1
    cut = np.sort(P64.reshape(-1))[::-1][K - 1]
    near = np.abs(P64.reshape(-1) - cut) <= 1e-5 * cut
    assert np.array_equal(got[~near], want[~near])
    assert int(got.sum()) == K


# ------------------------------------------------------------------ driver --
def pin_step_kind(lib):
    # Anchor every 32 steps over 256 steps: anchors 0, 32, ..., 224.
    kinds = [O.step_kind(t, 0, 32, lib) for t in range(256)]
    assert [t for t, x in enumerate(kinds) if x == 1] == list(range(0, 256, 32))
    assert all(x in (1, 2) for x in kinds)
    # Built once at step 0, reused for 7.
    assert [O.step_kind(t, 0, 0, lib) for t in range(8)] == [1] + [2] * 7
    # Dense warm-up for 26 of 128 steps, then one mask reused to the end.
    kinds = [O.step_kind(t, 26, 0, lib) for t in range(128)]
    assert kinds == [0] * 26 + [1] + [2] * 101
    # Dense warm-up followed by periodic refresh.
    kinds = [O.step_kind(t, 3, 4, lib) for t in range(12)]
    assert kinds == [0, 0, 0, 1, 2, 2, 2, 1, 2, 2, 2, 1]


# ----------------------------------------------------------- column-sparse --
def _torch_bf16(x):
    """bf16 rounding by torch (an independent implementation), as fp32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(
        torch.float32).numpy()


def pin_bf16_round(lib):
    rng = np.random.default_rng(RNG_SEEDS[0] + 11)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 4000),
                        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -8 + 2 ** -16,
                                    0.0, -0.0, 65504.0, 1e-30])]).astype(np.float32)
    got = O.bf16_round(x, lib)
    assert np.array_equal(got.view(np.uint32), _torch_bf16(x).view(np.uint32))
    # Ties to even, by hand: 1 + 2^-8 is halfway between 1 and 1 + 2^-7.
    assert got[4000] == 1.0 and got[4001] == np.float32(1 + 2 ** -6)


def _pooled_bf16(q, B, lib):
    return _torch_bf16(O.pool(q, B, lib))


def _softmax_rows(z):
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def worked_example_w3():
    """One head, L = 128, B = 64, d = 64: every query is 2*e0; key 5 is 3*e0,
    key 70 is 2*e0, every other key is 0.  Scores q.k/8 are 0.75 (key 5), 0.5
    (key 70) and 0 elsewhere, so with D = e^0.75 + e^0.5 + 126 the column
    masses are e^0.75/D, e^0.5/D and 1/D."""
    L, d = 128, 64
    q = np.zeros((1, L, d), np.float32)
    q[0, :, 0] = 2.0
    k = np.zeros((1, L, d), np.float32)
    k[0, 5, 0], k[0, 70, 0] = 3.0, 2.0
    v = np.zeros((1, L, d), np.float32)
    v[0, :, 1] = np.arange(L, dtype=np.float32) / 64.0
    v[0, :, 2] = 1.0
    return q, k, v


def pin_col_scores(lib):
    # Q = 0: every column gets 1/L.
    rng = np.random.default_rng(RNG_SEEDS[1] + 11)
    k = _rand((2, 256, 64), rng)
    c = O.col_scores(np.zeros((4, 256, 64), np.float32), k, 64, lib)
    assert np.max(np.abs(c - 1.0 / 256)) < 1e-15
    # Whole-matrix numpy fp64 on torch-rounded pooled queries, with GQA and
    # head temperatures; each head's masses sum to 1.
    for (H, Hkv, L, d, B, qs) in ((4, 2, 320, 64, 64, 2.0), (3, 1, 256, 128, 128, 0.5),
                                  (2, 2, 192, 64, 64, 4.0)):
        q, k = _rand((H, L, d), rng, qs), _rand((Hkv, L, d), rng)
        got = O.col_scores(q, k, B, lib)
        qb = _pooled_bf16(q, B, lib).astype(np.float64)
        for h in range(H):
            z = qb[h] @ k[h // (H // Hkv)].astype(np.float64).T / math.sqrt(d)
            want = _softmax_rows(z).mean(axis=0)
            assert np.max(np.abs(got[h] - want) / want) < 1e-12, (H, Hkv, L, d, B, h)
        assert np.max(np.abs(got.sum(axis=1) - 1.0)) < 1e-12
    # W3 in closed form.
    q, k, _ = worked_example_w3()
    c = O.col_scores(q, k, 64, lib)[0]
    D = math.exp(0.75) + math.exp(0.5) + 126
    want = np.full(128, 1 / D)
    want[5], want[70] = math.exp(0.75) / D, math.exp(0.5) / D
    assert np.max(np.abs(c - want)) < 1e-15


def pin_col_select(lib):
    rng = np.random.default_rng(RNG_SEEDS[2] + 11)
    H, L = 3, 200
    vals = rng.integers(0, 6, size=(H, L)).astype(np.float32) / 8.0   # heavy ties
    vals[1] = rng.random(L).astype(np.float32)
    for k_c in (0, 1, 7, 64, 199, 200):
        got = O.col_select(vals, k_c, lib)
        assert got.shape == (H, k_c)
        for h in range(H):
            order = np.lexsort((np.arange(L), -vals[h].astype(np.float64)))
            assert np.array_equal(got[h], np.sort(order[:k_c])), (k_c, h)
    # W3: k_c = 2 keeps keys 5 and 70; k_c = 3 adds the lowest-index tie, 0.
    q, k, _ = worked_example_w3()
    gold = golden_lists("w3_columns.txt")
    for s, want in ((1 - 2 / 128, gold[2]), (1 - 3 / 128, gold[3]), (0.0, list(range(128)))):
        c, cols, k_c = O.build_col_mask(q, k, 64, s, lib)
        assert k_c == len(want) and list(cols[0]) == want, (s, list(cols[0]))


def pin_col_attention(lib):
    rng = np.random.default_rng(RNG_SEEDS[0] + 12)
    for (H, Hkv, L, d, B, k_c) in ((4, 2, 256, 64, 64, 37), (3, 1, 256, 128, 128, 5),
                                   (2, 2, 192, 64, 64, 1)):
        q, k, v = _rand((H, L, d), rng), _rand((Hkv, L, d), rng), _rand((Hkv, L, d), rng)
        cols = np.stack([np.sort(rng.choice(L, k_c, replace=False)) for _ in range(H)]).astype(np.int32)
        mask = np.zeros((H, L, L), bool)
        for h in range(H):
            mask[h][:, cols[h]] = True
        got = O.col_attn(q, k, v, B, cols, lib=lib)
        want = brute_attention(q, k, v, mask)
        assert np.max(np.abs(got - want)) < 1e-12, (H, Hkv, L, d, B, k_c)
        # A subset of rows writes only those rows.
        rows = np.array([1, L // B + 2], np.int32) % (H * (L // B))
        part = O.col_attn(q, k, v, B, cols, rows=rows, lib=lib)
        for r in rows:
            h, i = divmod(int(r), L // B)
            assert np.array_equal(part[h, i * B:(i + 1) * B], got[h, i * B:(i + 1) * B])
    # Every column kept is dense attention.
    q, k, v = _rand((2, 128, 64), rng), _rand((2, 128, 64), rng), _rand((2, 128, 64), rng)
    allc = np.tile(np.arange(128, dtype=np.int32), (2, 1))
    assert np.max(np.abs(O.col_attn(q, k, v, 64, allc, lib=lib) - O.dense_attn(q, k, v, 64, lib=lib))) < 1e-13
    # W3: columns 5 and 70 with weights e^0.75 : e^0.5 for every query.
    q, k, v = worked_example_w3()
    o = O.col_attn(q, k, v, 64, np.array([[5, 70]], np.int32), lib=lib)[0]
    w5 = math.exp(0.75) / (math.exp(0.75) + math.exp(0.5))
    assert np.max(np.abs(o[:, 1] - (w5 * 5 + (1 - w5) * 70) / 64)) < 1e-15
    assert np.max(np.abs(o[:, 2] - 1.0)) < 1e-15 and np.all(o[:, 0] == 0) and np.all(o[:, 3:] == 0)


def pin_col_recall(lib):
    rng = np.random.default_rng(RNG_SEEDS[1] + 12)
    for (H, Hkv, L, d, B, qs) in ((4, 2, 256, 64, 64, 2.0), (3, 1, 256, 128, 128, 1.0)):
        nb = L // B
        q, k = _rand((H, L, d), rng, qs), _rand((Hkv, L, d), rng)
        allc = np.tile(np.arange(L, dtype=np.int32), (H, 1))
        assert np.max(np.abs(O.col_recall(q, k, B, allc, lib=lib) - 1.0)) < 1e-12
        assert np.all(O.col_recall(q, k, B, np.zeros((H, 0), np.int32), lib=lib) == 0)
        # Whole-matrix numpy fp64: softmax rows, summed over the kept columns,
        # averaged over each query block.
        k_c = 37
        cols = np.stack([np.sort(rng.choice(L, k_c, replace=False)) for _ in range(H)]).astype(np.int32)
        got = O.col_recall(q, k, B, cols, lib=lib)
        for h in range(H):
            p = _softmax_rows(q[h].astype(np.float64) @ k[h // (H // Hkv)].astype(np.float64).T
                              / math.sqrt(d))
            want = p[:, cols[h]].sum(axis=1).reshape(nb, B).mean(axis=1)
            assert np.max(np.abs(got[h * nb:(h + 1) * nb] - want)) < 1e-12, (H, h)
        # Keeping whole key blocks (the same blocks for every row of a head)
        # recalls the block attention mass of those blocks.
        blocks = [np.sort(rng.choice(nb, 2, replace=False)) for _ in range(H)]
        bcols = np.stack([np.concatenate([np.arange(j * B, (j + 1) * B) for j in bl])
                          for bl in blocks]).astype(np.int32)
        A = O.block_mass(q, k, B, lib=lib)
        want = np.concatenate([A[h][:, blocks[h]].sum(axis=1) for h in range(H)])
        assert np.max(np.abs(O.col_recall(q, k, B, bcols, lib=lib) - want)) < 1e-12
        # A row subset writes only those rows.
        part = O.col_recall(q, k, B, cols, rows=[1, H * nb - 1], lib=lib)
        assert part[1] == got[1] and part[-1] == got[-1] and part[0] == 0


ALL_PINS = [pin_keep_count, pin_pool, pin_scores, pin_select, pin_select_per_head, pin_csr,
            pin_plan, pin_worked_w1_per_head,
            pin_attention_brute, pin_attention_closed_forms, pin_worked_w1, pin_worked_w2,
            pin_build_mask_brute, pin_step_kind, pin_block_mass, pin_mask_recall,
            pin_bf16_round, pin_col_scores, pin_col_select, pin_col_attention, pin_col_recall]
