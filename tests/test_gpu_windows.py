"""Batch invariance on the GPU: a row's output bits are the same alone, in a window
of 2 to 24 rows starting at any first row, and in one 64-row launch (four passes of
16), on 6144 -> 25600 (the width sweep's shape) at every width, on both wave counts
and both engines. Source: the TensorFold pull request "hip exl3: the input rotation
and trellis linear for decode rows", "Checks on this head" (the window test).

At 4 waves this shape puts fewer waves in flight than the chip has SIMDs, so the
planner runs the column-split forms for one pass and the regular ones for the
64-row launch: the comparison crosses forms. The single rows are also run with each
form forced (debug entry points), so every form is compared rows-alone against the
batch. Comparisons stay on the device (bit patterns as int32); the oracle checks the
batch on sampled strips.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import trellis as tr
from tests.gpu_util import down, say, up

pytestmark = pytest.mark.gpu

K, N, ROWS = 6144, 25600, 64


def run(engine, zt, tt, vt, bits, waves, split=None):
    if split is None:
        y = tq.linear(zt, tt, vt, bits, N, waves=waves, engine=engine)
    elif engine == "dot2":
        y = tq.debug_linear_split(zt, tt, vt, bits, N, split, waves=waves)
    else:
        y = tq.debug_linear_mfma_split(zt, tt, vt, bits, N, split, waves=waves)
    return y.view(torch.int32)


@pytest.mark.parametrize("engine", ["dot2", "mfma"])
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("bits", tr.WIDTHS)
def test_rows_alone_windows_and_passes(gpu, engine, waves, bits):
    stream = synth.trellis_words(700 + bits, bits, K, N)
    z = synth.rows(701 + bits, ROWS, K, "f16")
    svh = synth.signs(702 + bits, N)
    say(f"windows {engine} waves={waves} bits={bits}: every first row, sizes 2..24, rows alone, 64 rows")
    tt, zt, vt = up(stream), up(z), up(svh)
    full = run(engine, zt, tt, vt, bits, waves)
    # Each row alone: the planner's form, then each form forced where the engine has two.
    forms = [None] + ([0, 1] if (engine == "dot2" or waves == 4) else [0])
    bad = []
    for split in forms:
        flags = torch.stack([(run(engine, zt[r : r + 1], tt, vt, bits, waves, split)[0] != full[r]).any()
                             for r in range(ROWS)])
        bad += [("alone", split, int(r)) for r in torch.nonzero(flags).flatten().tolist()]
    # Every window of 2..24 rows from every first row.
    cases, flags = [], []
    for size in range(2, 25):
        for first in range(0, ROWS - size + 1):
            w = run(engine, zt[first : first + size], tt, vt, bits, waves)
            flags.append((w != full[first : first + size]).any())
            cases.append((size, first))
    hit = torch.nonzero(torch.stack(flags)).flatten().tolist()
    bad += [("window",) + cases[i] for i in hit]
    say(f"  {len(cases)} windows, {ROWS * len(forms)} single rows: {len(bad)} differ")
    assert not bad, bad[:10]
    strips = [0, 77, 199]
    y64 = lin.linear_f64(z, stream, bits, K, N, svh, strips=strips)
    y = down(full.view(torch.float32))[:, lin.strip_columns(strips)]
    assert lin.gate_error(y, "f32", y64) <= lin.GATE


@pytest.mark.parametrize("engine", ["dot2", "mfma"])
@pytest.mark.parametrize("bits", [3, 4])
def test_engram_prefixes_are_bit_equal(gpu, engine, bits):
    """Engram's row counts (1, 2, 8, 16 bf16 rows, fp16 out, 4 waves): the first r rows
    of the 16-row run, bit for bit, for each r."""
    k, n = 6144, 25600
    stream = synth.trellis_words(synth.seed_for(2, synth.STREAM_TRELLIS) + 10 * bits, bits, k, n)
    x = synth.rows(synth.seed_for(2, synth.STREAM_ROWS), 16, k, "bf16")
    suh = synth.signs(synth.seed_for(2, synth.STREAM_SUH), k)
    svh = synth.signs(synth.seed_for(2, synth.STREAM_SVH), n)
    say(f"engram prefixes {engine} bits={bits}")
    tt, vt = up(stream), up(svh)
    z = tq.rot_in(up(x, "bf16"), up(suh))
    y16 = tq.linear(z, tt, vt, bits, n, out_dtype=torch.float16, waves=4, engine=engine).view(torch.int16)
    for r in (1, 2, 8):
        yr = tq.linear(z[:r].contiguous(), tt, vt, bits, n, out_dtype=torch.float16, waves=4,
                       engine=engine).view(torch.int16)
        assert torch.equal(yr, y16[:r]), r
