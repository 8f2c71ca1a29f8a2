"""The column-split variant of the linear (narrow matrices: twice the waves, one column
per lane) against the regular kernels, bit for bit on the same inputs: every width,
both wave counts, row counts across the pass and bucket sizes, three output types.
Shapes that fill the GPU take the regular kernels and narrow ones the split kernels
through tf_exl3_linear; tf_exl3_debug_linear_split forces either."""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import trellis as tr
from tests.gpu_util import TORCH_DT, down, same_bits, say, up

pytestmark = pytest.mark.gpu


def run(z, tt, svh, bits, n, split, out="f32", waves=0):
    y = tq.debug_linear_split(up(z), tt, up(svh), bits, n, split, out_dtype=TORCH_DT[out], waves=waves)
    torch.cuda.synchronize()
    return down(y)


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("rows", [1, 2, 3, 8, 13, 16, 21, 40])
def test_split_is_bit_equal(gpu, bits, waves, rows):
    k, n = 1024, 640
    stream = synth.trellis_words(5000 + bits, bits, k, n)
    z = synth.rows(5001 + rows, rows, k, "f16", 1.0)
    svh = synth.signs(5002, n)
    say(f"column split bits={bits} waves={waves} rows={rows}")
    tt = up(stream)
    a = run(z, tt, svh, bits, n, 1, waves=waves)
    b = run(z, tt, svh, bits, n, 0, waves=waves)
    assert same_bits(a, b), np.argwhere(nf.f32_bits(a) != nf.f32_bits(b))[:5]


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_split_output_types(gpu, out):
    bits, k, n, rows = 5, 512, 384, 6
    stream = synth.trellis_words(5100, bits, k, n)
    z = synth.rows(5101, rows, k, "f16", 1.0)
    svh = synth.signs(5102, n)
    say(f"column split out={out}")
    tt = up(stream)
    assert same_bits(run(z, tt, svh, bits, n, 1, out), run(z, tt, svh, bits, n, 0, out), out)


def test_split_gate_and_engram_shape(gpu):
    """Engram's 6144 -> 25600 at 3 bits and 4 waves (a column-split launch through the
    plain entry point): equal to the forced regular kernels and within the gate."""
    bits, k, n, rows = 3, 6144, 25600, 2
    assert tq.linear_plan(bits, rows, k, n, waves=4)["column_split"] == 1
    stream = synth.trellis_words(5200, bits, k, n)
    z = synth.rows(5201, rows, k, "f16", 1.0)
    svh = synth.signs(5202, n)
    say("column split Engram shape")
    tt = up(stream)
    y = tq.linear(up(z), tt, up(svh), bits, n, waves=4)
    torch.cuda.synchronize()
    y = down(y)
    assert same_bits(y, run(z, tt, svh, bits, n, 0, waves=4))
    strips = [0, 99, 199]
    y64 = lin.linear_f64(z, stream, bits, k, n, svh, strips=strips)
    assert lin.gate_error(y[:, lin.strip_columns(strips)], "f32", y64) <= lin.GATE


def test_split_refuses_other_values(gpu):
    with pytest.raises(Exception):
        run(np.zeros((1, 128), np.uint16), up(np.zeros(128 * 128 // 8, np.uint32)), np.zeros(128, np.uint16),
            4, 128, 2)
