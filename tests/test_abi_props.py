"""Properties of the host-side planner and refusals over random arguments (no GPU).

The rules are restated here from the header's documentation, independently of the
library's C++: the wave rule of the page ("Kernel contract": 8 waves from 8192 output
columns, else 4), passes of 16 rows, the row-capacity buckets, the column-split
threshold, the LDS figures, the stream size, and which argument each refusal names.
"""

import ctypes

from hypothesis import given, settings
from hypothesis import strategies as st

import trellis_quantized_linear_tf_amd as tq
from trellis_quantized_linear_tf_amd import _lib

WIDTHS = (2, 3, 4, 5, 6, 8)
dims = st.integers(min_value=1, max_value=600).map(lambda m: 128 * m)
bad_dims = st.integers(min_value=-300, max_value=80000).filter(lambda d: d < 128 or d % 128 != 0)


def bucket(r):
    return next(c for c in (1, 2, 4, 8, 12, 16) if r <= c)


def expected_plan(bits, rows, k, n, waves):
    w = (8 if n >= 8192 else 4) if waves == 0 else waves
    passes = -(-rows // 16)
    cap = bucket(min(rows, 16)) if rows else 0
    first = rows // 16 if rows >= 16 else 1
    split = int(rows > 0 and (n // 128) * first * w < 2048)
    fr = min(cap, 16)
    if rows == 0:
        lds = 0
    elif split:
        lds = w * fr * 512 + 2 * w * 2 * cap * 16
    else:
        lds = w * fr * 512 + (w * 2 * cap * 16 if cap > 4 else 0)
    return {
        "width_index": WIDTHS.index(bits),
        "waves": w,
        "threads": (128 if split else 64) * w,
        "grid_x": n // 128,
        "passes": passes,
        "rows_last_pass": rows - (passes - 1) * 16 if rows else 0,
        "rows_kernel": cap,
        "lds_bytes": lds,
        "column_split": split,
    }


def stream_fits(bits, k, n):
    return k * n * bits // 8 < 2**32


@settings(max_examples=400, deadline=None)
@given(st.sampled_from(WIDTHS), st.integers(0, 300), dims, dims, st.sampled_from([0, 4, 8]))
def test_plan_matches_the_stated_rules(bits, rows, k, n, waves):
    if not stream_fits(bits, k, n):
        return
    assert tq.linear_plan(bits, rows, k, n, waves) == expected_plan(bits, rows, k, n, waves)


@settings(max_examples=300, deadline=None)
@given(st.sampled_from(WIDTHS), dims, dims)
def test_trellis_bytes(bits, k, n):
    want = k * n * bits // 8 if stream_fits(bits, k, n) else 0
    assert tq.trellis_bytes(bits, k, n) == want


@settings(max_examples=300, deadline=None)
@given(st.integers(-4, 12).filter(lambda b: b not in WIDTHS), st.integers(0, 20), dims, dims,
       st.sampled_from([0, 4, 8]))
def test_bad_width_is_refused_first(bits, rows, k, n, waves):
    p = _lib.Plan()
    assert _lib.load().tf_exl3_linear_plan(bits, rows, k, n, waves, ctypes.byref(p)) == -1


@settings(max_examples=300, deadline=None)
@given(st.sampled_from(WIDTHS), st.integers(0, 20), bad_dims, dims, st.booleans())
def test_bad_shape_is_refused(bits, rows, bad, good, bad_is_k):
    k, n = (bad, good) if bad_is_k else (good, bad)
    p = _lib.Plan()
    assert _lib.load().tf_exl3_linear_plan(bits, rows, k, n, 0, ctypes.byref(p)) == -2


@settings(max_examples=200, deadline=None)
@given(st.sampled_from(WIDTHS), st.integers(-1000, -1), dims, dims)
def test_negative_rows_are_refused(bits, rows, k, n):
    if not stream_fits(bits, k, n):
        return
    p = _lib.Plan()
    assert _lib.load().tf_exl3_linear_plan(bits, rows, k, n, 0, ctypes.byref(p)) == -3


@settings(max_examples=200, deadline=None)
@given(st.sampled_from(WIDTHS), st.integers(0, 20), dims, dims, st.integers(-3, 12).filter(lambda w: w not in (0, 4, 8)))
def test_bad_waves_are_refused(bits, rows, k, n, waves):
    if not stream_fits(bits, k, n):
        return
    p = _lib.Plan()
    assert _lib.load().tf_exl3_linear_plan(bits, rows, k, n, waves, ctypes.byref(p)) == -8


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 200), dims, dims, st.sampled_from([0, 4, 8]))
def test_project_pass_rows_fit_the_lds_budget(rows, k, n, waves):
    """A pass holds its rows' z (fp16) and the waves' partial sums in at most 48 KiB,
    takes a power of two rows, never more than 16 or than the rows asked for, and is
    the largest such power of two when rows allow it."""
    if not stream_fits(4, k, n):
        return
    w = (8 if n >= 8192 else 4) if waves == 0 else waves
    lds = lambda r: r * k * 2 + w * r * 512
    r = _lib.load().tf_exl3_project_pass_rows(rows, k, n, waves)
    if lds(1) > 48 * 1024:
        assert r == -2
        return
    assert r in (1, 2, 4, 8, 16) and lds(r) <= 48 * 1024
    cap = max(c for c in (1, 2, 4, 8, 16) if lds(c) <= 48 * 1024)
    assert r == min(cap, next(c for c in (1, 2, 4, 8, 16) if min(rows, 16) <= c))
