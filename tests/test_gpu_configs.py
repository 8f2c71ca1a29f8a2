"""The five workloads at their full sizes, through rot_in and the linear as the
bench launches them, against the oracle on every output.

rot_in's fp16 rows are compared whole (bit for bit); the linear's outputs are
compared whole within the 2e-3 float64 gate, every strip of every row, with the
oracle's float64 linear threaded over strips (bit-identical to one thread). The
oracle runs once per workload input and is shared by both engines and by the
row-count prefixes (a row's float64 result does not depend on the rows beside it).
fp16 outputs must also equal the rounding of an fp32-output run.
Seeds: 1000 * workload + stream (0 trellis, 1 rows, 2 suh, 3 svh, 4 extra rows).
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import numfmt as nf
from oracle import rotation as rot
from tests.gpu_util import TORCH_DT, down, same_bits, say, up

pytestmark = pytest.mark.gpu
ENGINES = pytest.mark.parametrize("engine", ["dot2", "mfma"])


def inputs(workload, bits, k, n, rows, x_dtype, sigma=1.0):
    s = lambda stream: synth.seed_for(workload, stream)
    stream = synth.trellis_words(s(synth.STREAM_TRELLIS) + 10 * bits, bits, k, n)
    x = synth.rows(s(synth.STREAM_ROWS), rows, k, x_dtype, sigma)
    suh = synth.signs(s(synth.STREAM_SUH), k)
    svh = synth.signs(s(synth.STREAM_SVH), n)
    return stream, x, suh, svh


def run_path(stream_t, x, x_dtype, suh, svh, bits, n, out, waves, engine="dot2"):
    z = tq.rot_in(up(x, x_dtype), up(suh))
    y = tq.linear(z, stream_t, up(svh), bits, n, out_dtype=TORCH_DT[out], waves=waves, engine=engine)
    torch.cuda.synchronize()
    return down(z), y


_Y64 = {}


def oracle_y64(key, stream, x, x_dtype, suh, svh, bits, k, n):
    """y64 of every output for rot_in(x) (cached under `key` for the other engine and
    for row prefixes of the same x)."""
    if key not in _Y64:
        while len(_Y64) >= 8:  # a few workload inputs at a time
            _Y64.pop(next(iter(_Y64)))
        z_ref = rot.rot_in(x, x_dtype, suh)
        _Y64[key] = lin.linear_f64(z_ref, stream, bits, k, n, svh, threads=lin.reference_threads())
    return _Y64[key]


def check(z_gpu, y_gpu, stream, x, x_dtype, suh, svh, bits, k, n, out, key, rows=None):
    """rot_in bit for bit, then every output of the linear within the gate; `key` names
    the oracle run over x (whose first `rows` rows were launched)."""
    rows = x.shape[0] if rows is None else rows
    z_ref = rot.rot_in(x[:rows], x_dtype, suh)
    assert np.array_equal(z_gpu, z_ref), np.argwhere(z_gpu != z_ref)[:5]
    y64 = oracle_y64(key, stream, x, x_dtype, suh, svh, bits, k, n)[:rows]
    err = lin.gate_error(down(y_gpu), out, y64)
    say(f"  all {n // 128} strips x {rows} rows: max|y-y64|/rms = {err:.3g}")
    assert err <= lin.GATE, err
    return err


@ENGINES
def test_indexer_wk(gpu, engine):
    bits, k, n = 4, 512, 128
    stream, x, suh, svh = inputs(1, bits, k, n, 1, "f16")
    say("indexer wk 512->128 4-bit, 1 fp16 row, fp32 out, auto waves")
    z, y = run_path(up(stream), x, "f16", suh, svh, bits, n, "f32", 0, engine)
    assert tq.linear_plan(bits, 1, k, n)["waves"] == 4
    check(z, y, stream, x, "f16", suh, svh, bits, k, n, "f32", ("indexer",))


@ENGINES
@pytest.mark.parametrize("bits", [3, 4])
def test_engram_wkv(gpu, engine, bits):
    k, n = 6144, 25600
    stream, x, suh, svh = inputs(2, bits, k, n, 16, "bf16")
    st = up(stream)
    for rows in (1, 2, 8, 16):
        say(f"[{engine}] engram wkv 6144->25600 {bits}-bit, {rows} bf16 rows, fp16 out, 4 waves")
        z, y16 = run_path(st, x[:rows], "bf16", suh, svh, bits, n, "f16", 4, engine)
        check(z, y16, stream, x, "bf16", suh, svh, bits, k, n, "f16", ("engram", bits), rows)
        y32 = tq.linear(up(z), st, up(svh), bits, n, out_dtype=torch.float32, waves=4, engine=engine)
        torch.cuda.synchronize()
        assert same_bits(down(y16), nf.f32_to_output(down(y32), "f16"), "f16")


@pytest.mark.parametrize("rows", [1, 16])
@ENGINES
def test_lm_head(gpu, engine, rows):
    bits, k, n = 4, 5120, 129280
    stream, x, suh, svh = inputs(3, bits, k, n, 16, "f16", 0.5)
    say(f"[{engine}] lm head 5120->129280 4-bit, {rows} fp16 rows ~N(0,0.5), fp32 out, auto waves")
    z, y = run_path(up(stream), x[:rows], "f16", suh, svh, bits, n, "f32", 0, engine)
    assert tq.linear_plan(bits, rows, k, n)["waves"] == 8
    check(z, y, stream, x, "f16", suh, svh, bits, k, n, "f32", ("head",), rows)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@ENGINES
def test_width_sweep(gpu, engine, bits):
    k, n, rows = 6144, 25600, 64
    stream, x, suh, svh = inputs(4, bits, k, n, rows, "f16")
    say(f"[{engine}] width sweep 6144->25600 {bits}-bit, 64 fp16 rows (4 passes), fp32 out, 8 waves")
    z, y = run_path(up(stream), x, "f16", suh, svh, bits, n, "f32", 8, engine)
    check(z, y, stream, x, "f16", suh, svh, bits, k, n, "f32", ("sweep", bits))


@ENGINES
def test_stress_linear_8bit(gpu, engine):
    bits, k, n = 8, 5120, 129280
    stream, xb, suh, svh = inputs(5, bits, k, n, 64, "bf16")
    xf = synth.heavy_rows(synth.seed_for(5, synth.STREAM_EXTRA), 64, k)
    st = up(stream)
    for x, x_dtype in ((xb, "bf16"), (xf, "f32")):
        say(f"[{engine}] stress lm head 8-bit, 64 {x_dtype} rows, fp32 out, auto waves")
        z, y = run_path(st, x, x_dtype, suh, svh, bits, n, "f32", 0, engine)
        check(z, y, stream, x, x_dtype, suh, svh, bits, k, n, "f32", ("stress", x_dtype))


def test_whole_projection_from_x(gpu):
    """rot_in then the linear against x . diag(suh) H W H diag(svh) in float64 (no z rounding):
    the difference is z's fp16 rounding, well inside 1e-2 of the rms."""
    bits, k, n = 4, 1024, 2048
    stream, x, suh, svh = inputs(6, bits, k, n, 5, "f32")
    say("whole projection from x, 1024->2048")
    _, y = run_path(up(stream), x, "f32", suh, svh, bits, n, "f32", 0)
    from oracle import trellis as tr

    ref = lin.dense_from_x(x, "f32", suh, tr.unpack(stream, bits, k, n), svh)
    assert np.max(np.abs(down(y) - ref)) / np.sqrt(np.mean(ref ** 2)) < 1e-2


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_width_sweep_bit_equal_paths(gpu, bits):
    """The width sweep's 64 rows through the prompt path, the strips layout and the
    single launch: bit for bit the decode linear's outputs, at full size."""
    k, n, rows = 6144, 25600, 64
    stream, x, suh, svh = inputs(4, bits, k, n, rows, "f16")
    say(f"width sweep {bits}-bit: prompt, strips and single launch against the linear")
    tt, xt, st, vt = up(stream), up(x), up(suh), up(svh)
    z = tq.rot_in(xt, st)
    y = down(tq.linear(z, tt, vt, bits, n, waves=8))
    assert same_bits(down(tq.linear(z, tt, vt, bits, n, waves=8, engine="prompt")), y)
    strips = tq.repack_strips(tt, bits, k, n)
    assert same_bits(down(tq.linear(z, strips, vt, bits, n, waves=8, engine="strips")), y)
    del strips
    assert same_bits(down(tq.project(xt, st, tt, vt, bits, n, waves=8)), y)


def test_stress_bit_equal_paths(gpu):
    """The stress workload's heavy-tailed fp32 rows (8-bit LM head) through the prompt
    path and the single launch: bit for bit the decode linear's outputs."""
    bits, k, n = 8, 5120, 129280
    stream, _, suh, svh = inputs(5, bits, k, n, 64, "bf16")
    xf = synth.heavy_rows(synth.seed_for(5, synth.STREAM_EXTRA), 64, k)
    say("stress 8-bit heavy fp32 rows: prompt and single launch against the linear")
    tt, xt, st, vt = up(stream), up(xf), up(suh), up(svh)
    z = tq.rot_in(xt, st)
    y = down(tq.linear(z, tt, vt, bits, n))
    assert same_bits(down(tq.linear(z, tt, vt, bits, n, engine="prompt")), y)
    assert same_bits(down(tq.project(xt, st, tt, vt, bits, n)), y)
