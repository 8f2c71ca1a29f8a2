"""The calibration kernels do what their measurements assume: the copy copies
every byte and the read stream reads every byte (its XOR words cover all input)."""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 4096 * 4 + 12, 1 << 22])
def test_copy(gpu, n_words):
    say(f"calib copy {n_words} words")
    src = torch.from_numpy(synth.uniform_words(5, n_words).view(np.int32)).to(gpu)
    dst = torch.zeros_like(src)
    tq.calib_copy(src, dst, blocks=64)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("n_words", [4, 4096 * 4 + 12, 1 << 22])
def test_stream_read_xor(gpu, n_words):
    say(f"calib stream read {n_words} words")
    host = synth.uniform_words(6, n_words)
    src = torch.from_numpy(host.view(np.int32)).to(gpu)
    out = torch.empty(64 * 256, dtype=torch.int32, device=gpu)
    tq.calib_stream_read(src, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
