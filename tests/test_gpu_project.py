"""The fused projection (rot_in and the linear in one launch) against the two-launch
path: the same bits for every width, wave count, input and output type, ragged row
counts spanning several passes, and the full LM head; and against the oracle."""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import rotation as rot
from oracle import trellis as tr
from tests.gpu_util import TORCH_DT, down, same_bits, say, up

pytestmark = pytest.mark.gpu


def two_launch(xt, suh_t, st, svh_t, bits, n, out, waves):
    z = tq.rot_in(xt, suh_t)
    return tq.linear(z, st, svh_t, bits, n, out_dtype=TORCH_DT[out], waves=waves)


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("x_dtype,rows", [("f32", 1), ("f16", 2), ("bf16", 3), ("f16", 5), ("bf16", 17)])
def test_equals_rot_in_then_linear(gpu, bits, waves, x_dtype, rows):
    k, n = 1024, 512
    stream = synth.trellis_words(900 + bits, bits, k, n)
    x = synth.heavy_rows(901, rows, k) if x_dtype == "f32" else synth.rows(901, rows, k, x_dtype)
    suh = synth.scales(902, k)
    svh = synth.signs(903, n)
    say(f"project bits={bits} waves={waves} {x_dtype} rows={rows} pass={tq.project_pass_rows(rows, k, n, waves)}")
    xt, suh_t, st, svh_t = up(x, x_dtype), up(suh), up(stream), up(svh)
    a = tq.project(xt, suh_t, st, svh_t, bits, n, waves=waves)
    b = two_launch(xt, suh_t, st, svh_t, bits, n, "f32", waves)
    torch.cuda.synchronize()
    assert same_bits(down(a), down(b))


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_output_types(gpu, out):
    bits, k, n, rows = 4, 2048, 1024, 2
    stream = synth.trellis_words(904, bits, k, n)
    x = synth.rows(905, rows, k, "bf16")
    suh = synth.signs(906, k)
    svh = synth.signs(907, n)
    say(f"project out={out}")
    xt, suh_t, st, svh_t = up(x, "bf16"), up(suh), up(stream), up(svh)
    a = tq.project(xt, suh_t, st, svh_t, bits, n, out_dtype=TORCH_DT[out])
    b = two_launch(xt, suh_t, st, svh_t, bits, n, out, 0)
    torch.cuda.synchronize()
    assert same_bits(down(a), down(b), out)


@pytest.mark.parametrize("rows", [1, 2])
def test_lm_head(gpu, rows):
    bits, k, n = 4, 5120, 129280
    stream = synth.trellis_words(3000, bits, k, n)
    x = synth.rows(3001, rows, k, "f16", 0.5)
    suh = synth.signs(3002, k)
    svh = synth.signs(3003, n)
    say(f"project lm head rows={rows}")
    xt, suh_t, st, svh_t = up(x, "f16"), up(suh), up(stream), up(svh)
    a = tq.project(xt, suh_t, st, svh_t, bits, n)
    b = two_launch(xt, suh_t, st, svh_t, bits, n, "f32", 0)
    torch.cuda.synchronize()
    ya = down(a)
    assert same_bits(ya, down(b))
    strips = [0, 505, 1009]
    y64 = lin.linear_f64(rot.rot_in(x, "f16", suh), stream, bits, k, n, svh, strips=strips)
    assert lin.gate_error(ya[:, lin.strip_columns(strips)], "f32", y64) <= lin.GATE


def test_zero_rows_and_refusal(gpu):
    x = torch.empty((0, 256), dtype=torch.float16, device=gpu)
    suh = up(synth.signs(908, 256))
    st = up(synth.trellis_words(909, 4, 256, 128))
    svh = up(synth.signs(910, 128))
    say("project zero rows")
    assert tq.project(x, suh, st, svh, 4, 128).shape == (0, 128)
    with pytest.raises(tq.Exl3Error):
        tq.project_pass_rows(1, 32768, 128)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_nonfinite_inputs(gpu, x_dtype):
    """inf and NaN in x go through the rotation into z and the linear exactly as the
    two-call path takes them: the same bits (NaNs equal to NaNs) and float64's classes."""
    bits, k, n, rows = 4, 512, 384, 3
    stream = synth.trellis_words(7100, bits, k, n)
    x = synth.rows(7101, rows, k, x_dtype, 1.0)
    suh = synth.signs(7102, k)
    svh = synth.signs(7103, n)
    if x_dtype == "f32":
        x[0, 5], x[1, 200], x[2, 7] = np.inf, -np.inf, np.nan
    else:
        x[0, 5], x[1, 200], x[2, 7] = 0x7F80, 0xFF80, 0x7FC0
    say(f"project non-finite x={x_dtype}")
    xt, st, tt, vt = up(x, x_dtype), up(suh), up(stream), up(svh)
    y = down(tq.project(xt, st, tt, vt, bits, n))
    z = tq.rot_in(xt, st)
    y_ref = down(tq.linear(z, tt, vt, bits, n))
    assert same_bits(y, y_ref)
    z_oracle = rot.rot_in(x, x_dtype, suh)
    y64 = lin.linear_f64(z_oracle, stream, bits, k, n, svh)
    assert np.array_equal(lin.classes(y), lin.classes(y64))
    assert np.count_nonzero(lin.classes(y)) >= 3 * 128
