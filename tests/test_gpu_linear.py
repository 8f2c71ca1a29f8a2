"""The trellis linear on the GPU against the oracle.

Element-by-element on shapes the oracle finishes in seconds (several strips,
ragged row counts across passes, both wave counts, all widths, three output
types), the page's identity test (outputs are weight rows through the fp32
output rotation, bit for bit), its exactness gate (all-ones states, k = 6144,
inputs 4096: bit for bit), batch invariance across windows and passes,
five-run byte identity (batch invariance is in test_gpu_windows.py), non-finite classes, and the two planted controls
(inputs one row late, the wrong width) launched on the real kernel.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import rotation as rot
from oracle import trellis as tr
from tests.gpu_util import down, linear, same_bits, say, up

pytestmark = pytest.mark.gpu
ENGINES = pytest.mark.parametrize("engine", ["dot2", "mfma"])


def make(bits, k, n, rows, seed, sigma=1.0):
    stream = synth.trellis_words(seed, bits, k, n)
    z = synth.rows(seed + 1, rows, k, "f16", sigma)
    svh = synth.signs(seed + 2, n)
    return stream, z, svh


@ENGINES
@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("k,n,rows", [(128, 128, 1), (256, 384, 3), (384, 256, 5), (640, 128, 2), (512, 1024, 17),
                                       (1024, 256, 33)])
def test_small_shapes_gate(gpu, engine, bits, waves, k, n, rows):
    stream, z, svh = make(bits, k, n, rows, 1000 * bits + k + rows)
    say(f"linear {engine} bits={bits} waves={waves} k={k} n={n} rows={rows}")
    y = linear(z, stream, svh, bits, n, "f32", waves, engine=engine)
    y64 = lin.linear_f64(z, stream, bits, k, n, svh)
    err = lin.gate_error(y, "f32", y64)
    assert err <= lin.GATE, err


@ENGINES
@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_low_precision_outputs_are_casts(gpu, engine, out, bits):
    k, n, rows = 512, 768, 5
    stream, z, svh = make(bits, k, n, rows, 77 + bits)
    say(f"linear {engine} bits={bits} out={out}")
    y32 = linear(z, stream, svh, bits, n, "f32", engine=engine)
    yt = linear(z, stream, svh, bits, n, out, engine=engine)
    assert same_bits(yt, nf.f32_to_output(y32, out), out)
    assert lin.gate_error(yt, out, lin.linear_f64(z, stream, bits, k, n, svh)) <= lin.GATE


@ENGINES
@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
def test_identity_rows_give_rotated_weight_rows(gpu, engine, bits, waves):
    k, n = 256, 384
    stream = synth.trellis_words(600 + bits, bits, k, n)
    svh = synth.signs(601, n)
    eye = np.where(np.eye(k, dtype=bool), np.uint16(0x3C00), np.uint16(0)).astype(np.uint16)
    say(f"identity {engine} bits={bits} waves={waves}")
    y = linear(eye, stream, svh, bits, n, "f32", waves, engine=engine)
    w = nf.f16_bits_to_f32(tr.unpack(stream, bits, k, n))
    want = lin.finish_f32(w, svh, "f32")
    assert same_bits(y, want), np.argwhere(nf.f32_bits(y) != nf.f32_bits(want))[:5]


@ENGINES
@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
def test_exact_gate(gpu, engine, bits, waves):
    k, n = 6144, 128
    stream = synth.constant_trellis(bits, k, n, ones=True)
    z = np.full((1, k), 0x6C00, dtype=np.uint16)
    svh = synth.signs(602, n)
    say(f"exact gate {engine} bits={bits} waves={waves}")
    y = linear(z, stream, svh, bits, n, "f32", waves, engine=engine)[0]
    acc = np.full((1, n), 6144 * 2682, dtype=np.float32)
    want = lin.finish_f32(acc, svh, "f32")[0]
    assert same_bits(y, want)
    assert abs(int(nf.f32_bits(y[0])) & 0x7FFFFFFF) == 0x4D31CB0C


@ENGINES
def test_five_runs_byte_identical(gpu, engine):
    stream, z, svh = make(4, 2048, 8192, 16, 800)
    say(f"five runs {engine}")
    tt = up(stream)
    runs = [linear(z, None, svh, 4, 8192, "f32", 0, stream_t=tt, engine=engine) for _ in range(5)]
    assert all(np.array_equal(nf.f32_bits(runs[0]), nf.f32_bits(r)) for r in runs[1:])


@ENGINES
def test_nonfinite_classes(gpu, engine):
    k, n, rows = 512, 512, 4
    stream, z, svh = make(4, k, n, rows, 801)
    z[0, 3] = 0x7C00  # +inf
    z[1, 100] = 0xFC00  # -inf
    z[2, 7] = 0x7E00  # NaN
    say(f"non-finite inputs {engine}")
    y = linear(z, stream, svh, 4, n, "f32", engine=engine)
    y64 = lin.linear_f64(z, stream, 4, k, n, svh)
    assert np.array_equal(lin.classes(y), lin.classes(y64))
    assert lin.gate_error(y, "f32", y64) <= lin.GATE
    assert np.count_nonzero(lin.classes(y)) >= 3 * n


@ENGINES
def test_planted_control_rows_one_late(gpu, engine):
    bits, k, n, rows = 4, 128, 512, 16
    stream, z, svh = make(bits, k, n, rows + 1, 802)
    say("planted control: z + in_dim")
    zt = up(z)
    y = tq.linear(zt[1:], up(stream), up(svh), bits, n, engine=engine)
    torch.cuda.synchronize()
    y64 = lin.linear_f64(z[:rows], stream, bits, k, n, svh)
    err = lin.gate_error(down(y), "f32", y64)
    say(f"planted control error / gate = {err / lin.GATE:.0f}")
    assert err > 100 * lin.GATE


@ENGINES
def test_planted_control_wrong_width(gpu, engine):
    k, n, rows = 256, 512, 2
    stream, z, svh = make(4, k, n, rows, 803)
    say("planted control: 4-bit stream read as 3-bit")
    y = linear(z, stream[: k * n * 3 // 32], svh, 3, n, engine=engine)  # the 3-bit size: in bounds
    y64 = lin.linear_f64(z, stream, 4, k, n, svh)
    assert lin.gate_error(y, "f32", y64) > 100 * lin.GATE


@ENGINES
def test_zero_rows(gpu, engine):
    stream, z, svh = make(4, 128, 128, 0, 804)
    say(f"zero rows {engine}")
    y = linear(z, stream, svh, 4, 128, engine=engine)
    assert y.shape == (0, 128)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_engines_agree(gpu, bits):
    """Both engines sit within the gate of float64, hence of each other (not bit for bit:
    their k orders differ)."""
    k, n, rows = 1024, 2048, 16
    stream, z, svh = make(bits, k, n, rows, 805 + bits)
    say(f"engines agree bits={bits}")
    a = linear(z, stream, svh, bits, n, engine="dot2")
    b = linear(z, stream, svh, bits, n, engine="mfma")
    y64 = lin.linear_f64(z, stream, bits, k, n, svh)
    assert lin.gate_error(a, "f32", y64) <= lin.GATE and lin.gate_error(b, "f32", y64) <= lin.GATE


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("k,rows", [(256, 5), (384, 17)])
def test_mfma_column_split_same_bits(gpu, bits, k, rows):
    """At 4 waves the matrix-core linear splits each strip's columns over twice the
    waves when fewer than 256 strips would leave SIMDs idle; each column keeps its
    MFMAs and cross-wave order. A narrow matrix made of the first 8 strips of a wide
    one (which runs the unsplit form) gives the wide run's bits for those columns."""
    n_wide, n_narrow = 32768, 1024
    wide = synth.trellis_words(900 + bits + k, bits, k, n_wide)
    narrow = np.ascontiguousarray(tr.tile_grid(wide, bits, k, n_wide)[:, : n_narrow // 16]).reshape(-1)
    z = synth.rows(901 + bits, rows, k, "f16")
    svh = synth.signs(902 + bits, n_wide)
    say(f"mfma column split bits={bits} k={k} rows={rows}")
    yw = linear(z, wide, svh, bits, n_wide, "f32", 4, engine="mfma")
    yn = linear(z, narrow, svh[:n_narrow], bits, n_narrow, "f32", 4, engine="mfma")
    assert same_bits(yn, yw[:, :n_narrow])
    y64 = lin.linear_f64(z, narrow, bits, k, n_narrow, svh[:n_narrow])
    assert lin.gate_error(yn, "f32", y64) <= lin.GATE


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("k,n,rows", [(384, 1024, 3), (640, 256, 17), (6144, 1280, 16)])
def test_mfma_forms_same_bits(gpu, bits, k, n, rows):
    """The matrix-core linear's two forms at 4 waves (each strip's 8 column tiles on
    every wave, or in halves over twice the waves) run the same MFMAs per column in
    the same order: bit-identical outputs, within the gate."""
    stream, z, svh = make(bits, k, n, rows, 930 + bits + k)
    say(f"mfma forms bits={bits} k={k} n={n} rows={rows}")
    zt, tt, vt = up(z), up(stream), up(svh)
    ys = [down(tq.debug_linear_mfma_split(zt, tt, vt, bits, n, split, waves=4)) for split in (0, 1)]
    torch.cuda.synchronize()
    assert same_bits(ys[1], ys[0])
    assert same_bits(linear(z, None, svh, bits, n, "f32", 4, stream_t=tt, engine="mfma"), ys[1])
    y64 = lin.linear_f64(z, stream, bits, k, n, svh)
    assert lin.gate_error(ys[1], "f32", y64) <= lin.GATE
