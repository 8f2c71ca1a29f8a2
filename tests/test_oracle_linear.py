"""Pins for oracle/linear.py: the float64 projection, the fp32 finish and the gate.

Independent checks: dense brute force with explicit rotation matrices (no
butterflies), the whole projection composed from x against rot_in followed by
the linear, the page's exactness gate for the linear (all-ones states, inputs
of 4096, k = 6144: every sum is an integer below 2^24) worked out in closed
form, and planted mistakes (inputs read one row late, the wrong width) that
must blow through the 2e-3 gate.
"""

import numpy as np
import pytest

import synth
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import rotation as rot
from oracle import trellis as tr


def case(bits, k, n, rows, seed):
    stream = synth.trellis_words(seed, bits, k, n)
    x = synth.rows(seed + 1, rows, k, "f16")
    suh = synth.signs(seed + 2, k)
    svh = synth.signs(seed + 3, n)
    return stream, x, suh, svh


@pytest.mark.parametrize("bits", tr.WIDTHS)
def test_linear_f64_matches_dense_brute_force(bits):
    for k, n, rows in ((128, 256, 3), (256, 128, 1), (256, 256, 4)):
        stream, x, suh, svh = case(bits, k, n, rows, 10 * bits + k)
        z = rot.rot_in(x, "f16", suh)
        y = lin.linear_f64(z, stream, bits, k, n, svh)
        w = tr.unpack(stream, bits, k, n)
        ref = lin.dense_from_z(z, w, svh)
        assert np.max(np.abs(y - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_strip_subset_equals_full():
    stream, x, suh, svh = case(4, 256, 512, 2, 5)
    z = rot.rot_in(x, "f16", suh)
    full = lin.linear_f64(z, stream, 4, 256, 512, svh)
    sub = lin.linear_f64(z, stream, 4, 256, 512, svh, strips=[3, 1])
    assert np.array_equal(sub, full[:, np.r_[384:512, 128:256]])


def test_projection_composes_from_x():
    """rot_in then the linear equals x . diag(suh) H W H diag(svh), up to z's fp16 rounding."""
    for bits in (2, 5, 8):
        stream, x, suh, svh = case(bits, 256, 256, 4, 50 + bits)
        z = rot.rot_in(x, "f16", suh)
        y = lin.linear_f64(z, stream, bits, 256, 256, svh)
        ref = lin.dense_from_x(x, "f16", suh, tr.unpack(stream, bits, 256, 256), svh)
        rel = np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2))
        assert rel < 1e-2


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_gate_closed_form(bits):
    k, n = 6144, 128
    stream = synth.constant_trellis(bits, k, n, ones=True)
    z = np.full((1, k), 0x6C00, dtype=np.uint16)  # fp16 4096
    assert nf.f16_bits_to_f64(np.uint16(0x6C00)) == 4096.0
    w1 = nf.f16_bits_to_f64(tr.decode_states(np.array([0xFFFF]))[0])
    prod = 4096 * w1
    assert prod == int(prod) and 6144 * int(prod) < 2 ** 24 and 6144 * int(prod) > 65504
    acc = lin.accumulate_f64(z, tr.unpack(stream, bits, k, n))
    assert np.all(acc == 6144 * int(prod))
    svh = synth.signs(9, n)
    y = lin.finish_f32(acc.astype(np.float32), svh, "f32")[0]
    head = np.float32(np.float32(6144 * int(prod) * 128) * rot.SCALE_F32)
    sgn = np.where(svh == synth.F16_ONE, np.float32(1), np.float32(-1))
    want = np.concatenate([[head * sgn[0]], np.float32(0.0) * sgn[1:]]).astype(np.float32)
    assert np.array_equal(nf.f32_bits(y), nf.f32_bits(want))
    assert int(nf.f32_bits(head)) == 0x4D31CB0C


def test_finish_f32_close_to_f64():
    acc = synth.normals(3, 4 * 384).reshape(4, 384) * 100
    svh = synth.signs(4, 384)
    y32 = lin.finish_f32(acc.astype(np.float32), svh, "f32").astype(np.float64)
    y64 = lin.finish_f64(acc.astype(np.float32).astype(np.float64), svh)
    assert np.max(np.abs(y32 - y64)) <= 1e-6 * np.sqrt(np.mean(y64 ** 2))


def test_finish_outputs_are_casts_of_fp32():
    acc = (synth.normals(5, 2 * 256).reshape(2, 256) * 3e4).astype(np.float32)
    svh = synth.signs(6, 256)
    y32 = lin.finish_f32(acc, svh, "f32")
    assert np.array_equal(lin.finish_f32(acc, svh, "f16"), nf.f64_to_f16_bits(y32.astype(np.float64)))
    assert np.array_equal(lin.finish_f32(acc, svh, "bf16"), nf.f64_to_bf16_bits(y32.astype(np.float64)))


def test_gate_metric():
    y64 = synth.normals(7, 1000)
    assert lin.gate_error(y64.astype(np.float32), "f32", y64) < 1e-6
    bumped = y64.copy()
    bumped[17] += 3e-3 * np.sqrt(np.mean(y64 ** 2))
    assert lin.gate_error(bumped.astype(np.float32), "f32", y64) > 2e-3
    assert lin.gate_error(nf.f64_to_f16_bits(y64), "f16", y64) == 0.0
    assert lin.gate_error(nf.f64_to_bf16_bits(y64), "bf16", y64) == 0.0
    odd = y64.copy()
    odd[3] = np.inf
    assert lin.gate_error(odd.astype(np.float32), "f32", y64) == float("inf")
    assert lin.gate_error(odd.astype(np.float32), "f32", odd) < 1e-6


def test_planted_inputs_one_row_late_fail_the_gate():
    bits, k, n, rows = 4, 128, 512, 16
    stream, x, suh, svh = case(bits, k, n, rows + 1, 77)
    z = rot.rot_in(x, "f16", suh)
    y64 = lin.linear_f64(z[:rows], stream, bits, k, n, svh)
    late = lin.linear_f64(z[1 : rows + 1], stream, bits, k, n, svh)
    assert lin.gate_error(late.astype(np.float32), "f32", y64) > 100 * lin.GATE


def test_planted_wrong_width_fails_the_gate():
    k, n = 256, 256
    stream, x, suh, svh = case(4, k, n, 2, 78)
    z = rot.rot_in(x, "f16", suh)
    y64 = lin.linear_f64(z, stream, 4, k, n, svh)
    as3 = lin.linear_f64(z, stream[: k * n * 3 // 32], 3, k, n, svh)
    assert lin.gate_error(as3.astype(np.float32), "f32", y64) > 100 * lin.GATE


def test_nonfinite_classes_propagate():
    k, n = 128, 256
    stream, x, suh, svh = case(4, k, n, 3, 79)
    z = rot.rot_in(x, "f16", suh)
    z[0, 5] = 0x7C00  # +inf
    z[1, 9] = 0x7E00  # NaN
    y = lin.linear_f64(z, stream, 4, k, n, svh)
    assert np.all(np.isnan(y[1]))  # a NaN input reaches every output through the rotation
    assert not np.isfinite(y[0]).any()
    assert np.all(np.isfinite(y[2]))


def test_float64_reference_does_not_depend_on_threads_chunks_or_rows():
    """The page's threaded float64 reference is bit-identical to one thread ("Checks on
    this head"); here: one BLAS thread against the default, strips in chunks of 3
    against 32, and each row alone against all rows at once, bit for bit."""
    from threadpoolctl import threadpool_limits

    bits, k, n, rows = 4, 1024, 1280, 5
    stream = synth.trellis_words(71, bits, k, n)
    z = synth.rows(72, rows, k, "f16", 1.0)
    svh = synth.signs(73, n)
    a = lin.linear_f64(z, stream, bits, k, n, svh)
    with threadpool_limits(1):
        b = lin.linear_f64(z, stream, bits, k, n, svh)
    c = lin.linear_f64(z, stream, bits, k, n, svh, strip_chunk=3)
    d = np.concatenate([lin.linear_f64(z[i : i + 1], stream, bits, k, n, svh) for i in range(rows)])
    assert np.array_equal(a, b) and np.array_equal(a, c) and np.array_equal(a, d)
    # The threaded reference: strip chunks spread over pools of several widths.
    for threads, chunk in ((2, 1), (3, 2), (lin.reference_threads(), 4)):
        e = lin.linear_f64(z, stream, bits, k, n, svh, strip_chunk=chunk, threads=threads)
        assert np.array_equal(a, e), (threads, chunk)


def test_threaded_reference_keeps_strip_order():
    """A strip list out of order (and with repeats) gives each strip's block where the
    list puts it, threaded or not: the pool writes every chunk to its own columns."""
    bits, k, n = 3, 256, 1024
    stream = synth.trellis_words(74, bits, k, n)
    z = synth.rows(75, 2, k, "f16", 1.0)
    svh = synth.signs(76, n)
    full = lin.linear_f64(z, stream, bits, k, n, svh)
    order = [7, 0, 3, 3, 5, 1]
    y = lin.linear_f64(z, stream, bits, k, n, svh, strips=order, strip_chunk=1, threads=4)
    assert np.array_equal(y, full[:, lin.strip_columns(order)])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_ulp_is_the_rounding_bound_exactly(dtype):
    """half_ulp(v) is the largest error of rounding v to the output type: midpoints
    between neighbouring values reach it (so a full-ulp allowance would be caught),
    and no value exceeds it. The rounding comes from numpy (fp16) and torch (bf16),
    not from the oracle."""
    import torch

    rng = np.random.default_rng(5)
    if dtype == "f16":
        lo = rng.integers(0x0400, 0x7BFF, 4000).astype(np.uint16)  # normal, below the largest
        a = lo.view(np.float16).astype(np.float64)
        b = (lo + 1).astype(np.uint16).view(np.float16).astype(np.float64)
        rnd = lambda v: v.astype(np.float16).astype(np.float64)
    else:
        lo = rng.integers(0x0080, 0x7F7F, 4000).astype(np.uint32)
        a = (lo << 16).view(np.float32).astype(np.float64)
        b = ((lo + 1) << 16).view(np.float32).astype(np.float64)
        rnd = lambda v: torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    for sign in (1.0, -1.0):
        mid = sign * (a + b) / 2  # exact in float64
        assert np.array_equal(lin.half_ulp(mid, dtype), np.abs(rnd(mid) - mid))
        off = sign * (a + 0.3 * (b - a))
        assert np.all(np.abs(rnd(off) - off) <= lin.half_ulp(off, dtype))


def test_gate_charges_a_one_ulp_miss_half_an_ulp():
    """An fp16 output one ulp from y64 = 1 is charged exactly half an ulp (2^-11):
    the allowance is half an ulp, not a whole one."""
    y64 = np.array([1.0, -1.0])
    y = np.array([0x3C01, 0xBC00], dtype=np.uint16)  # 1 + 2^-10, -1
    assert lin.gate_error(y, "f16", y64) == 2.0 ** -11
    yb = np.array([0x3F81, 0xBF80], dtype=np.uint16)  # bf16 1 + 2^-7, -1
    assert lin.gate_error(yb, "bf16", y64) == 2.0 ** -8
