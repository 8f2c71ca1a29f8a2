"""Pins for oracle/rotation.py: the 128-point transform and rot_in's fp32 steps.

Independent checks: an explicit Sylvester matrix built by the recursive block
construction; the transform being its own inverse up to 128; Parseval; a
scalar pure-Python pass in the stated stage order; the scale constant bracketed
with exact rationals; integer inputs on which every fp32 step is exact (the
page's exactness gate for rot_in: only fp16's rounding can show); one-hot and
constant blocks. Planted mistakes in copies of the oracle's steps (divide by
sqrt(128), one fused rounding, fp16 products, the next block's suh) must each
change outputs, which is what lets the GPU's bit-exact comparison catch them.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import numfmt as nf
from oracle import rotation as rot


def sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_fwht_equals_explicit_matrix():
    v = (synth.splitmix64(1, 3 * 256) % np.uint64(201)).astype(np.int64).reshape(3, 256) - 100
    got = rot.fwht128(v.astype(np.float64))
    h = sylvester(128)
    want = np.concatenate([v[:, :128] @ h.T, v[:, 128:] @ h.T], axis=1)
    assert np.array_equal(got, want.astype(np.float64))
    assert np.array_equal(rot.hadamard_matrix(128), h)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_fwht_is_its_own_inverse_up_to_128(dtype):
    v = ((synth.splitmix64(2, 512) % np.uint64(41)).astype(np.int64) - 20).astype(dtype).reshape(2, 256)
    assert np.array_equal(rot.fwht128(rot.fwht128(v)), 128 * v)


def test_parseval():
    v = synth.normals(3, 4 * 384).reshape(4, 384)
    f = rot.fwht128(v)
    assert np.allclose((f * f).sum(axis=1), 128 * (v * v).sum(axis=1), rtol=1e-12)


def test_fp32_stage_order_against_scalar_loops():
    v = synth.store_f32(synth.normals(4, 128))
    a = [np.float32(t) for t in v]
    h = 1
    while h < 128:
        for i in range(128):
            if i & h == 0:
                x, y = a[i], a[i + h]
                a[i], a[i + h] = np.float32(x + y), np.float32(x - y)
        h *= 2
    assert np.array_equal(rot.fwht128(v), np.array(a, dtype=np.float32))


def test_scale_is_nearest_fp32_to_inv_sqrt128():
    s = Fraction(float(rot.SCALE_F32))
    half_ulp = Fraction(1, 2 ** 28)  # s in [2^-4, 2^-3): spacing 2^-27
    assert (s - half_ulp) ** 2 < Fraction(1, 128) < (s + half_ulp) ** 2
    assert int(nf.f32_bits(rot.SCALE_F32)) == 0x3DB504F3


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_integer_inputs_exact_gate(x_dtype):
    rows, k = 6, 512
    xi = (synth.splitmix64(5, rows * k) % np.uint64(129)).astype(np.int64).reshape(rows, k) - 64
    x = synth.store(xi.astype(np.float64), x_dtype)
    suh = synth.signs(6, k)
    sgn = np.where(suh == synth.F16_ONE, 1, -1)
    h = sylvester(128)
    p = xi * sgn
    exact = np.concatenate([p[:, b : b + 128] @ h.T for b in range(0, k, 128)], axis=1)  # Python-exact ints
    want = (exact.astype(np.float32) * rot.SCALE_F32).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(rot.rot_in(x, x_dtype, suh), want)


def test_one_hot_gives_scaled_sign_pattern():
    suh = synth.signs(8, 128)
    for i in (0, 1, 77, 127):
        x = np.zeros((1, 128), dtype=np.float32)
        x[0, i] = 1.0
        z = rot.rot_in(x, "f32", suh)[0]
        row = sylvester(128)[i] * (1 if suh[i] == synth.F16_ONE else -1)
        assert np.array_equal(z, np.where(row > 0, 0x2DA8, 0xADA8).astype(np.uint16))


def test_constant_block():
    for c in (1.0, -3.0, 0.25):
        x = np.full((1, 128), c, dtype=np.float32)
        z = rot.rot_in(x, "f32", np.full(128, synth.F16_ONE, dtype=np.uint16))[0]
        head = np.float32(np.float32(128 * c) * rot.SCALE_F32)
        assert z[0] == np.array([head], dtype=np.float32).astype(np.float16).view(np.uint16)[0]
        assert np.all(z[1:] == 0)  # +0: a - a is +0 under round to nearest


# ---------------------------------------------------------------------------
# The 391,680-rounding set (1020 blocks per input type) and planted mistakes.


def stress_rows(dtype, seed):
    """1020 blocks of 128: 4 x 6144 + 16 x 5120 + 32 x 512 + 60 x 128."""
    out = []
    for i, (r, k) in enumerate([(4, 6144), (16, 5120), (32, 512), (60, 128)]):
        if dtype == "f32":
            x = synth.heavy_rows(seed + i, r, k)
        else:
            x = synth.rows(seed + i, r, k, dtype)
        suh = synth.signs(seed + 10 + i, k)
        out.append((x, suh))
    return out


def test_stress_set_size():
    n = sum(x.size for x, _ in stress_rows("f16", 1))
    assert 3 * n == 391_680


def _f32_bound(x, x_dtype, suh):
    """|z - z64| <= half an fp16 ulp plus the fp32 error of depth 8 (product + 7 stages)."""
    p = np.abs(nf.input_to_f32(x, x_dtype).astype(np.float64) * nf.f16_bits_to_f64(suh))
    tot = p.reshape(p.shape[0], -1, 128).sum(axis=2, keepdims=True)
    return np.repeat(tot, 128, axis=2).reshape(p.shape) * rot.SCALE_F64 * 9 * 2.0 ** -24


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_rot_in_within_float64_bound(x_dtype):
    for x, suh in stress_rows(x_dtype, 40):
        z = nf.f16_bits_to_f64(rot.rot_in(x, x_dtype, suh))
        z64 = rot.rot_in_f64(x, x_dtype, suh)
        ulp = np.ldexp(1.0, np.maximum(np.frexp(np.abs(z64))[1] - 1, -14) - 10)
        assert np.all(np.abs(z - z64) <= ulp / 2 + _f32_bound(x, x_dtype, suh))


def _planted(x, x_dtype, suh, plant):
    x32 = nf.input_to_f32(x, x_dtype)
    s32 = nf.f16_bits_to_f32(suh)
    if plant == "next_block_suh":
        s32 = np.roll(s32, -128)
    p = (x32 * s32).astype(np.float32)
    if plant == "fp16_products":
        p = nf.f16_bits_to_f32(nf.f64_to_f16_bits(p.astype(np.float64)))
    v = rot.fwht128(p)
    if plant == "divide":
        v = (v / np.float32(np.sqrt(128.0))).astype(np.float32)
        return nf.f64_to_f16_bits(v.astype(np.float64))
    if plant == "one_rounding":
        return nf.f64_to_f16_bits(v.astype(np.float64) * float(rot.SCALE_F32))
    v = (v * rot.SCALE_F32).astype(np.float32)
    return nf.f64_to_f16_bits(v.astype(np.float64))


@pytest.mark.parametrize("plant", ["divide", "one_rounding", "fp16_products", "next_block_suh"])
def test_planted_mistakes_move_outputs(plant):
    moved = 0
    total = 0
    for x_dtype in ("f32", "f16", "bf16"):
        for x, suh in stress_rows(x_dtype, 70):
            if plant == "fp16_products":
                suh = synth.scales(71, suh.size)  # non +-1 suh, so fp16 products round
            good = rot.rot_in(x, x_dtype, suh)
            bad = _planted(x, x_dtype, suh, plant)
            moved += int(np.count_nonzero(good != bad))
            total += good.size
    assert total == 391_680
    assert moved >= 1, plant
