"""A stream past 2 GiB: 8-bit, 16384 -> 163840 (2.68 GB). Every path on it, checked on
64 strips spread evenly from the first to the last (in the tile layout every strip's
tile rows from 820 on lie past the 2 GiB mark) against the oracle's threaded float64
result, and the bit-equal paths against the decode linear on every output."""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import rotation as rot
from tests.gpu_util import down, same_bits, say, up

pytestmark = pytest.mark.gpu

BITS, K, N = 8, 16384, 163840
STRIPS = [int(v) for v in np.linspace(0, N // 128 - 1, 64).round()]


@pytest.fixture(scope="module")
def large():
    assert tq.trellis_bytes(BITS, K, N) == K * N > 2**31
    say("large stream: generating 2.68 GB")
    stream = synth.trellis_words(6000, BITS, K, N)
    tt = up(stream)
    svh = synth.signs(6002, N)
    yield stream, tt, svh
    del tt
    torch.cuda.empty_cache()


def check_strips(y, z, stream, svh):
    y64 = lin.linear_f64(z, stream, BITS, K, N, svh, strips=STRIPS, threads=lin.reference_threads())
    err = lin.gate_error(y[:, lin.strip_columns(STRIPS)], "f32", y64)
    assert err <= lin.GATE, err


def test_large_dot2_strips_prompt(gpu, large):
    stream, tt, svh = large
    z = synth.rows(6001, 33, K, "f16", 1.0)
    zt, st = up(z), up(svh)
    say("large: dot2, strips, prompt")
    y = down(tq.linear(zt, tt, st, BITS, N))
    check_strips(y[:2], z[:2], stream, svh)
    y_prompt = down(tq.linear(zt, tt, st, BITS, N, engine="prompt"))
    assert same_bits(y_prompt, y)
    strips = tq.repack_strips(tt, BITS, K, N)
    y_strips = down(tq.linear(zt, strips, st, BITS, N, engine="strips"))
    del strips
    torch.cuda.empty_cache()
    assert same_bits(y_strips, y)


def test_large_mfma(gpu, large):
    stream, tt, svh = large
    z = synth.rows(6003, 17, K, "f16", 1.0)
    say("large: mfma at 2 and 17 rows")
    for rows in (2, 17):
        y = down(tq.linear(up(z[:rows]), tt, up(svh), BITS, N, engine="mfma"))
        check_strips(y[:2], z[:2], stream, svh)


def test_large_fused(gpu, large):
    stream, tt, svh = large
    x = synth.rows(6004, 2, K, "bf16", 1.0)
    suh = synth.signs(6005, K)
    say("large: fused projection")
    xt = up(x, "bf16")
    y = down(tq.project(xt, up(suh), tt, up(svh), BITS, N))
    z = rot.rot_in(x, "bf16", suh)
    y_ref = down(tq.linear(up(z), tt, up(svh), BITS, N))
    assert same_bits(y, y_ref)
    check_strips(y, z, stream, svh)
