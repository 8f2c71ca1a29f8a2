"""The largest launch the planner accepts: 1,048,560 rows (65,535 passes of 16, the
grid's second dimension at its limit) on a 128 -> 128 layer, through rot_in, the
decode linear, the prompt path (32-row passes) and the matrix cores.

rot_in's rows are checked bit for bit and the linear's within the float64 gate on
sampled rows (the first and last 20 and 64 seeded picks; a row's result does not
depend on its neighbours), and each engine's sampled rows, launched alone, must give
the big launch's bits. One row more is refused on the host.
"""

import numpy as np
import pytest
import torch

import synth
import trellis_quantized_linear_tf_amd as tq
from oracle import linear as lin
from oracle import rotation as rot
from tests.gpu_util import down, say, up

pytestmark = pytest.mark.gpu

BITS, K, N = 4, 128, 128
ROWS = 65535 * 16


def sampled_rows():
    picks = set(range(20)) | set(range(ROWS - 20, ROWS))
    picks |= {int(v) for v in synth.splitmix64(1401, 64) % np.uint64(ROWS)}
    return np.array(sorted(picks))


def test_largest_row_count(gpu):
    say(f"largest launch: {ROWS} rows, {K}->{N}, {BITS}-bit")
    x = synth.rows(1402, ROWS, K, "f16")
    suh, svh = synth.signs(1403, K), synth.signs(1404, N)
    stream = synth.trellis_words(1405, BITS, K, N)
    idx = sampled_rows()
    it = torch.as_tensor(idx, device=gpu)
    xt, tt, vt = up(x), up(stream), up(svh)
    z = tq.rot_in(xt, up(suh))
    z_s = down(z[it].contiguous())
    z_ref = rot.rot_in(x[idx], "f16", suh)
    assert np.array_equal(z_s, z_ref)
    del xt
    y64 = lin.linear_f64(z_ref, stream, BITS, K, N, svh)
    for engine in ("dot2", "prompt", "mfma"):
        say(f"  {engine}")
        y = tq.linear(z, tt, vt, BITS, N, engine=engine)
        y_s = y[it].contiguous()
        assert lin.gate_error(down(y_s), "f32", y64) <= lin.GATE, engine
        alone = tq.linear(z[it].contiguous(), tt, vt, BITS, N, engine=engine)
        assert torch.equal(alone.view(torch.int32), y_s.view(torch.int32)), engine
        del y
        torch.cuda.empty_cache()


def test_one_row_more_is_refused(gpu):
    z = torch.empty((ROWS + 1, K), dtype=torch.float16, device=gpu)
    t = up(synth.trellis_words(1406, BITS, K, N))
    v = up(synth.signs(1407, N))
    for engine in ("dot2", "prompt", "mfma"):
        with pytest.raises(tq.Exl3Error, match="TF_E_ROWS"):
            tq.linear(z, t, v, BITS, N, engine=engine)
