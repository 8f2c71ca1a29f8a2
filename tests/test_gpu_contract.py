"""The page's contract registrations on the GPU, against the float64 oracle.

Source: the TensorFold pull request "hip exl3: the input rotation and trellis linear
for decode rows", "Kernel contract". The linear is registered at each of the six
widths with fp32 outputs, and at 4 bits with bf16 outputs, on these shapes (the page
writes them as N x K, output columns by input width; here K -> N):
  - the indexer's wk (512 -> 128) at one row and in windows of 16 and 64 rows, 4 waves;
  - Engram's wkv (6144 -> 25600) at 4 rows, 8 waves;
  - the plan's 8-wave edge, 1024 -> 8192 at 4 and 16 rows, and the shape below it,
    1024 -> 8064 (which the planner runs on 4 waves);
  - the exact gate's shape with random inputs, 6144 -> 128 at one row, 4 waves;
  - the edges at 1, 15, 16, 17 and 64 rows, each with K and N of 128, 256 and the
    largest served (K 6144, Engram's; N 129280, the head's);
  - at 8 bits, also the head (5120 -> 129280) at one row, 8 waves.
Every registration runs five times and the five outputs are byte-identical. Both
engines run every registration. The oracle evaluates every output, except for the
6144 -> 129280 edges, where it evaluates 64 of the 1010 strips (first, last and
seeded picks): all five row counts come from one 64-row oracle run, since a row's
float64 result does not depend on the rows beside it.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import trellis as tr
from tests.gpu_util import TORCH_DT, down, say, up

pytestmark = pytest.mark.gpu
ROW_EDGES = (1, 15, 16, 17, 64)
DIM_EDGES = (128, 256)
K_MAX, N_MAX = 6144, 129280


def registrations(bits):
    """(label, K, N, row counts, waves) of one width's registration."""
    regs = [
        ("indexer wk", 512, 128, (1, 16, 64), 4),
        ("Engram wkv", 6144, 25600, (4,), 8),
        ("8-wave edge", 1024, 8192, (4, 16), 0),
        ("below the edge", 1024, 8064, (4, 16), 0),
        ("exact gate shape", 6144, 128, (1,), 4),
    ]
    for k in DIM_EDGES + (K_MAX,):
        for n in DIM_EDGES + (N_MAX,):
            regs.append((f"edges {k}->{n}", k, n, ROW_EDGES, 0))
    if bits == 8:
        regs.append(("LM head", 5120, 129280, (1,), 8))
    return regs


def oracle_strips(n, seed, count=64):
    """Every strip for narrow outputs; else `count` strips: the first two, the middle
    one and the last two, and seeded picks for the rest."""
    m = n // 128
    if m <= 256:
        return None  # every strip
    picks = [0, 1, m // 2, m - 2, m - 1]
    for v in synth.splitmix64(seed, 4 * count) % np.uint64(m):
        if len(picks) == count:
            break
        if int(v) not in picks:
            picks.append(int(v))
    return sorted(picks)


def five_runs(engine, zt, tt, vt, bits, n, waves, out):
    ys = [tq.linear(zt, tt, vt, bits, n, out_dtype=TORCH_DT[out], waves=waves, engine=engine) for _ in range(5)]
    bits_view = [y.view(torch.int16 if out != "f32" else torch.int32) for y in ys]
    same = all(torch.equal(bits_view[0], b) for b in bits_view[1:])
    return ys[0], same


@pytest.mark.parametrize("bits", tr.WIDTHS)
def test_registrations(gpu, bits):
    outs = ["f32", "bf16"] if bits == 4 else ["f32"]
    for i, (label, k, n, row_counts, waves) in enumerate(registrations(bits)):
        seed = 5000 + 100 * bits + i
        stream = synth.trellis_words(seed, bits, k, n)
        z = synth.rows(seed + 1, max(row_counts), k, "f16")
        svh = synth.signs(seed + 2, n)
        strips = oracle_strips(n, seed + 3)
        y64_all = lin.linear_f64(z, stream, bits, k, n, svh, strips=strips, threads=lin.reference_threads())
        cols = None if strips is None else torch.as_tensor(lin.strip_columns(strips), device=gpu)
        tt, zt, vt = up(stream), up(z), up(svh)
        plan_w = tq.linear_plan(bits, 1, k, n, waves)["waves"]
        for engine in ("dot2", "mfma"):
            for rows in row_counts:
                for out in outs:
                    say(f"[{engine}] {bits}-bit {label} {k}->{n}, {rows} rows, {out} out, waves {plan_w}")
                    y, same = five_runs(engine, zt[:rows], tt, vt, bits, n, waves, out)
                    assert same, "five runs differ"
                    ys = y if cols is None else y[:, cols].contiguous()
                    err = lin.gate_error(down(ys), out, y64_all[:rows])
                    assert err <= lin.GATE, (engine, label, rows, out, err)
                    if out != "f32":
                        y32 = tq.linear(zt[:rows], tt, vt, bits, n, waves=waves, engine=engine)
                        assert np.array_equal(down(y), nf.f32_to_output(down(y32), out))
        del tt, zt


def test_registered_wave_counts(gpu):
    """The planner's waves on the registered shapes (the page's plan: 8 waves from
    8192 output columns)."""
    assert tq.linear_plan(4, 4, 1024, 8192)["waves"] == 8
    assert tq.linear_plan(4, 4, 1024, 8064)["waves"] == 4
    assert tq.linear_plan(8, 1, 5120, 129280)["waves"] == 8
    assert tq.linear_plan(4, 1, 512, 128)["waves"] == 4
