"""Trellis decode on the GPU against the oracle, bit for bit.

The debug entry points run the linear's own device decode: every one of the
65,536 states through the codebook, and whole tile-layout streams through the
linear's share load, window extraction and codebook, at all six widths.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import trellis as tr
from tests.gpu_util import down, say, up

pytestmark = pytest.mark.gpu


def test_every_state(gpu):
    say("decode all 65536 states")
    states = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = down(tq.debug_decode_states(torch.from_numpy(states.view(np.int16)).to(gpu)))
    torch.cuda.synchronize()
    assert np.array_equal(w, tr.decode_states(states))


@pytest.mark.parametrize("bits", tr.WIDTHS)
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (1024, 2048)])
def test_random_streams(gpu, bits, shape):
    k, n = shape
    say(f"decode tiles bits={bits} k={k} n={n}")
    stream = synth.trellis_words(500 + bits, bits, k, n)
    w = down(tq.debug_decode_tiles(up(stream), bits, k, n))
    assert np.array_equal(w, tr.unpack(stream, bits, k, n))


@pytest.mark.parametrize("bits", tr.WIDTHS)
def test_constant_streams(gpu, bits):
    say(f"decode constant streams bits={bits}")
    for ones in (True, False):
        stream = synth.constant_trellis(bits, 128, 256, ones)
        w = down(tq.debug_decode_tiles(up(stream), bits, 128, 256))
        want = tr.decode_states(np.array([0xFFFF if ones else 0]))[0]
        assert np.all(w == want)


def test_lm_head_shape_sampled(gpu):
    """The head's full 5120 x 129280 stream at 4 bits; a few strips checked against the oracle."""
    bits, k, n = 4, 5120, 129280
    say(f"decode tiles bits={bits} k={k} n={n} (sampled strips)")
    stream = synth.trellis_words(501, bits, k, n)
    w = tq.debug_decode_tiles(up(stream), bits, k, n)
    torch.cuda.synchronize()
    for s in (0, 1, 517, 1009):
        got = down(w[:, 128 * s : 128 * s + 128].contiguous())
        assert np.array_equal(got, tr.unpack_columns(stream, bits, k, n, tr.strip_tile_cols([s]))), s
