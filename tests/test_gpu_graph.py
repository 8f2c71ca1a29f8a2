"""The entry points captured in a HIP graph (through torch.cuda.graph): every replay
gives the eager launches' bits.

A caller that replays a decode step as a graph captures rot_in and the linear (or the
single launch) once and changes only the contents of its input buffers. The library
launches kernels only (no memset, no allocation), so capture records just those.
Each graph is replayed three times; before each replay the program writes new rows
into the captured input buffer eagerly and synchronizes, and the replay's outputs
must equal an eager run on the same rows, bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from tests.gpu_util import say, up

pytestmark = pytest.mark.gpu

CASES = [  # (label, bits, in_dim, out_dim, rows, engine, waves)
    ("wide dot2", 4, 1024, 8192, 1, "dot2", 0),
    ("wide mfma 16 rows", 4, 1024, 8192, 16, "mfma", 0),
    ("narrow column split", 3, 6144, 1024, 2, "dot2", 4),
    ("narrow mfma split", 3, 6144, 1024, 2, "mfma", 4),
    ("single launch", 4, 2048, 4096, 1, "fused", 0),
]


def step(engine, x, suh, z, t, svh, y, bits, n, waves):
    if engine == "fused":
        tq.project(x, suh, t, svh, bits, n, y=y, waves=waves)
    else:
        tq.rot_in(x, suh, z)
        tq.linear(z, t, svh, bits, n, y=y, waves=waves, engine=engine)


@pytest.mark.parametrize("label,bits,k,n,rows,engine,waves", CASES)
def test_graph_replays_equal_eager(gpu, label, bits, k, n, rows, engine, waves):
    seed = 1200 + bits + k // 128 + rows
    t = up(synth.trellis_words(seed, bits, k, n))
    suh, svh = up(synth.signs(seed + 1, k)), up(synth.signs(seed + 2, n))
    xs = [up(synth.rows(seed + 3 + i, rows, k, "bf16"), "bf16") for i in range(4)]
    x = xs[0].clone()
    z = torch.empty((rows, k), dtype=torch.float16, device=gpu)
    y = torch.empty((rows, n), dtype=torch.float32, device=gpu)
    say(f"graph {label}: bits={bits} {k}->{n} rows={rows}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture, as torch asks
        step(engine, x, suh, z, t, svh, y, bits, n, waves)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(engine, x, suh, z, t, svh, y, bits, n, waves)
    torch.cuda.synchronize()

    for i in (1, 2, 3):
        x.copy_(xs[i])  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ze = torch.empty_like(z)
        ye = torch.empty_like(y)
        step(engine, xs[i], suh, ze, t, svh, ye, bits, n, waves)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ye.view(torch.int32)), (label, i)
        if engine != "fused":
            assert torch.equal(z.view(torch.int16), ze.view(torch.int16)), (label, i)
