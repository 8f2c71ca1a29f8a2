"""The strips layout on the GPU: the repacker against the oracle's layout, bit for bit,
and tf_exl3_linear_strips against tf_exl3_linear on the same tiles, bit for bit (same
waves, same order), including the page's identity check run at 8 waves on the strips
layout ("Checks on this head") and the LM-head shape."""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import trellis as tr
from tests.gpu_util import linear, same_bits, say, up

pytestmark = pytest.mark.gpu


def repack(stream, bits, k, n):
    t = tq.repack_strips(up(stream), bits, k, n)
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("k,n", [(128, 128), (256, 384), (1024, 640), (6144, 256)])
def test_repack_matches_the_oracle(gpu, bits, k, n):
    stream = synth.trellis_words(4000 + bits + k, bits, k, n)
    say(f"repack bits={bits} k={k} n={n}")
    got = repack(stream, bits, k, n).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, tr.tiles_to_strips(stream, bits, k, n))


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("rows", [1, 3, 17, 40])
def test_strips_linear_is_bit_equal_to_tiles(gpu, bits, waves, rows):
    k, n = 512, 1024
    stream = synth.trellis_words(4100 + bits, bits, k, n)
    z = synth.rows(4101 + rows, rows, k, "f16", 1.0)
    svh = synth.signs(4102, n)
    say(f"strips linear bits={bits} waves={waves} rows={rows}")
    tt = up(stream)
    st = repack(stream, bits, k, n)
    a = linear(z, None, svh, bits, n, "f32", waves, stream_t=st, engine="strips")
    b = linear(z, None, svh, bits, n, "f32", waves, stream_t=tt, engine="dot2")
    assert same_bits(a, b), np.argwhere(nf.f32_bits(a) != nf.f32_bits(b))[:5]


@pytest.mark.parametrize("bits", tr.WIDTHS)
def test_identity_at_8_waves_on_strips(gpu, bits):
    """The page's check: identity rows give the weight rows through the fp32 output
    rotation, bit for bit, here with the strips stream built by the oracle."""
    k, n = 256, 384
    stream = synth.trellis_words(4200 + bits, bits, k, n)
    svh = synth.signs(4201, n)
    strips = tr.tiles_to_strips(stream, bits, k, n)
    eye = np.where(np.eye(k, dtype=bool), np.uint16(0x3C00), np.uint16(0)).astype(np.uint16)
    say(f"identity on strips bits={bits}")
    y = linear(eye, strips, svh, bits, n, "f32", 8, engine="strips")
    w = nf.f16_bits_to_f32(tr.unpack(tr.strips_to_tiles(strips, bits, k, n), bits, k, n))
    assert same_bits(y, lin.finish_f32(w, svh, "f32"))


def test_gate_on_strips(gpu):
    bits, k, n, rows = 3, 768, 512, 5
    stream = synth.trellis_words(4300, bits, k, n)
    z = synth.rows(4301, rows, k, "f16", 1.0)
    svh = synth.signs(4302, n)
    say("strips gate")
    y = linear(z, tr.tiles_to_strips(stream, bits, k, n), svh, bits, n, "f32", engine="strips")
    assert lin.gate_error(y, "f32", lin.linear_f64(z, stream, bits, k, n, svh)) <= lin.GATE


@pytest.mark.parametrize("rows", [1, 16])
def test_lm_head_strips(gpu, rows):
    """5120 -> 129280, 4-bit: the repack of the whole stream equals the oracle's, and
    the strips linear equals the tile linear bit for bit."""
    k, n, bits = 5120, 129280, 4
    stream = synth.trellis_words(4400, bits, k, n)
    z = synth.rows(4401, rows, k, "f16", 0.5)
    svh = synth.signs(4402, n)
    say(f"LM head strips rows={rows}")
    tt = up(stream)
    st = tq.repack_strips(tt, bits, k, n)
    torch.cuda.synchronize()
    if rows == 1:
        got = st.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, tr.tiles_to_strips(stream, bits, k, n))
    a = linear(z, None, svh, bits, n, "f32", stream_t=st, engine="strips")
    b = linear(z, None, svh, bits, n, "f32", stream_t=tt, engine="dot2")
    assert same_bits(a, b)


def test_nonfinite_on_strips(gpu):
    bits, k, n, rows = 5, 256, 640, 3
    stream = synth.trellis_words(4500, bits, k, n)
    z = synth.rows(4501, rows, k, "f16", 1.0)
    z[0, 9], z[1, 77], z[2, 200] = 0x7C00, 0xFC00, 0x7E00
    svh = synth.signs(4502, n)
    say("strips non-finite")
    tt = up(stream)
    a = linear(z, None, svh, bits, n, "f32", stream_t=repack(stream, bits, k, n), engine="strips")
    b = linear(z, None, svh, bits, n, "f32", stream_t=tt, engine="dot2")
    assert same_bits(a, b)
    assert np.array_equal(lin.classes(a), lin.classes(lin.linear_f64(z, stream, bits, k, n, svh)))
