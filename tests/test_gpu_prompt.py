"""The prompt path (tf_exl3_linear_prompt) on the GPU.

Its rows must be bit-identical to the decode linear's (the page's "Known limits":
the prompt path that follows must reproduce the decode linear's bits), for every width, both
wave counts, the three output types and row counts on both sides of the 32-row
pass (a remainder that runs as decode passes). The oracle's gate is checked on
one case directly, and on sampled strips at the LM-head shape.
"""

import numpy as np
import pytest

import synth
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import trellis as tr
from tests.gpu_util import linear, same_bits, say, up

pytestmark = pytest.mark.gpu


def make(bits, k, n, rows, seed):
    stream = synth.trellis_words(seed, bits, k, n)
    z = synth.rows(seed + 1, rows, k, "f16", 1.0)
    svh = synth.signs(seed + 2, n)
    return stream, z, svh


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("rows", [32, 45, 64, 97])
def test_bit_equal_to_the_decode_linear(gpu, bits, waves, rows):
    k, n = 512, 640
    stream, z, svh = make(bits, k, n, rows, 900 + 10 * bits + rows)
    say(f"prompt bits={bits} waves={waves} rows={rows}")
    tt = up(stream)
    a = linear(z, None, svh, bits, n, "f32", waves, stream_t=tt, engine="prompt")
    b = linear(z, None, svh, bits, n, "f32", waves, stream_t=tt, engine="dot2")
    assert same_bits(a, b), np.argwhere(nf.f32_bits(a) != nf.f32_bits(b))[:5]


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_output_types(gpu, out):
    bits, k, n, rows = 3, 256, 384, 40
    stream, z, svh = make(bits, k, n, rows, 950)
    say(f"prompt out={out}")
    tt = up(stream)
    a = linear(z, None, svh, bits, n, out, stream_t=tt, engine="prompt")
    b = linear(z, None, svh, bits, n, out, stream_t=tt, engine="dot2")
    assert same_bits(a, b, out)


def test_gate_against_the_oracle(gpu):
    bits, k, n, rows = 4, 256, 384, 70
    stream, z, svh = make(bits, k, n, rows, 960)
    say("prompt gate")
    y = linear(z, stream, svh, bits, n, "f32", engine="prompt")
    assert lin.gate_error(y, "f32", lin.linear_f64(z, stream, bits, k, n, svh)) <= lin.GATE


def test_lm_head_rows(gpu):
    """64 fp16 rows ~N(0, 0.5) at 5120 -> 129280, 4-bit: bit-equal to the decode linear
    on every row, and within the gate of float64 on three sampled strips."""
    k, n, rows, bits = 5120, 129280, 64, 4
    stream = synth.trellis_words(970, bits, k, n)
    z = synth.rows(971, rows, k, "f16", 0.5)
    svh = synth.signs(972, n)
    say("prompt LM head 64 rows")
    tt = up(stream)
    a = linear(z, None, svh, bits, n, "f32", stream_t=tt, engine="prompt")
    b = linear(z, None, svh, bits, n, "f32", stream_t=tt, engine="dot2")
    assert same_bits(a, b)
    strips = [0, 517, 1009]
    y64 = lin.linear_f64(z[:4], stream, bits, k, n, svh, strips=strips)
    assert lin.gate_error(a[:4][:, lin.strip_columns(strips)], "f32", y64) <= lin.GATE


def test_zero_rows(gpu):
    stream, z, svh = make(4, 128, 128, 0, 980)
    say("prompt zero rows")
    assert linear(z, stream, svh, 4, 128, engine="prompt").shape == (0, 128)


def test_nonfinite_rows(gpu):
    """inf and NaN in some rows of a 40-row prompt: the same bits as the decode linear
    (NaNs equal to NaNs), row by row."""
    bits, k, n, rows = 4, 512, 384, 40
    stream, z, svh = make(bits, k, n, rows, 990)
    z[0, 3], z[17, 100], z[33, 7] = 0x7C00, 0xFC00, 0x7E00
    say("prompt non-finite")
    tt = up(stream)
    a = linear(z, None, svh, bits, n, "f32", stream_t=tt, engine="prompt")
    b = linear(z, None, svh, bits, n, "f32", stream_t=tt, engine="dot2")
    assert same_bits(a, b)
    assert np.count_nonzero(lin.classes(a)) >= 3 * 128
