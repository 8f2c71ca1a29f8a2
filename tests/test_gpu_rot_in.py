"""rot_in on the GPU against the oracle's fp32 steps, bit for bit.

The 391,680-rounding set (1020 blocks of 128 per input type: fp32 heavy-tailed
rows, fp16 and bf16 normal rows; the page's "Checks on this head" test),
non +-1 suh so the products round, integer inputs on which fp32 is exact,
non-finite inputs, ragged and empty row counts, and the page's planted control
(reading the next block's suh) launched from the host on the real kernel.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import numfmt as nf
from oracle import rotation as rot
from tests.gpu_util import down, rot_in, same_bits, say, up
from tests.test_oracle_rotation import stress_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_stress_set_bit_exact(gpu, x_dtype):
    n = 0
    for x, suh in stress_rows(x_dtype, 40):
        say(f"rot_in {x_dtype} rows={x.shape[0]} k={x.shape[1]}")
        got = rot_in(x, x_dtype, suh)
        want = rot.rot_in(x, x_dtype, suh)
        assert np.array_equal(got, want), np.argwhere(got != want)[:5]
        n += got.size
    assert 3 * n == 391_680


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_rounding_products(gpu, x_dtype):
    """suh of arbitrary magnitude: the fp32 product rounds before the butterflies."""
    x = synth.heavy_rows(91, 8, 1024) if x_dtype == "f32" else synth.rows(91, 8, 1024, x_dtype, 3.0)
    suh = synth.scales(92, 1024, 0.1, 30.0)
    say(f"rot_in {x_dtype} with non +-1 suh")
    assert np.array_equal(rot_in(x, x_dtype, suh), rot.rot_in(x, x_dtype, suh))


@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
def test_integer_inputs(gpu, x_dtype):
    xi = (synth.splitmix64(5, 6 * 512) % np.uint64(129)).astype(np.float64).reshape(6, 512) - 64
    x = synth.store(xi, x_dtype)
    suh = synth.signs(6, 512)
    say(f"rot_in integer inputs {x_dtype}")
    assert np.array_equal(rot_in(x, x_dtype, suh), rot.rot_in(x, x_dtype, suh))


def test_nonfinite_inputs(gpu):
    x = synth.heavy_rows(93, 32, 512)
    x[0, 3] = np.inf
    x[1, 200] = -np.inf
    x[2, 5] = np.nan
    x[3, :] = np.float32(3e38)  # products and sums overflow to inf
    x[4, 7] = np.inf
    x[4, 8] = -np.inf  # inf - inf = NaN inside the butterflies
    x[5, 0] = np.float32(1e-42)  # fp32 subnormal
    suh = synth.signs(94, 512)
    say("rot_in non-finite inputs")
    got = rot_in(x, "f32", suh)
    want = rot.rot_in(x, "f32", suh)
    assert same_bits(got, want)
    nonfinite = int(np.count_nonzero((want & 0x7C00) == 0x7C00))
    assert nonfinite >= 4 * 128


@pytest.mark.parametrize("rows", [0, 1, 3, 17, 64])
def test_row_counts(gpu, rows):
    x = synth.rows(95, rows, 384, "f16")
    suh = synth.signs(96, 384)
    say(f"rot_in rows={rows}")
    got = rot_in(x, "f16", suh)
    assert got.shape == (rows, 384)
    assert np.array_equal(got, rot.rot_in(x, "f16", suh))


def test_determinism(gpu):
    x, suh = stress_rows("bf16", 40)[0]
    say("rot_in five runs")
    runs = [rot_in(x, "bf16", suh) for _ in range(5)]
    assert all(np.array_equal(runs[0], r) for r in runs[1:])


def test_planted_control_next_block_suh(gpu):
    """The real kernel told to read suh one block late (in bounds: suh padded by a block)."""
    rows, k = 64, 512
    x = synth.rows(97, rows, k, "bf16")
    suh = synth.signs(98, k + 128)
    say("rot_in planted control: suh + 128")
    xt = up(x, "bf16")
    suh_t = up(suh)
    z = tq.rot_in(xt, suh_t[128:])
    torch.cuda.synchronize()
    got = nf.f16_bits_to_f64(down(z))
    z64 = rot.rot_in_f64(x, "bf16", suh[:k])
    ulp = np.ldexp(1.0, np.maximum(np.frexp(np.abs(z64))[1] - 1, -14) - 10)
    p = np.abs(nf.input_to_f32(x, "bf16").astype(np.float64))
    bound = ulp / 2 + np.repeat(p.reshape(rows, -1, 128).sum(2, keepdims=True), 128, 2).reshape(rows, k) \
        * rot.SCALE_F64 * 9 * 2.0 ** -24
    worst = float(np.max(np.abs(got - z64) / bound))
    say(f"planted control worst ratio to bound: {worst:.1f}")
    assert worst > 100
