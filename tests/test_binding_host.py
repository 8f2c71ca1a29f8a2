"""The Python binding's argument checks, on the host (no GPU).

The C ABI receives plain pointers, so it cannot see a buffer's size or element
type: the binding checks them before any call reaches the library. Each
refusal is raised from CPU tensors (the checks need no GPU), and a call whose
every shape and type is right still refuses CPU tensors, because the library
reads device memory. Nothing here launches a kernel.
"""

import pytest
import torch

import trellis_quantized_linear_tf_amd as tq

K, N, BITS = 256, 384, 4
NB = K * N * BITS // 8


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def stream(nbytes=NB):
    return torch.zeros(nbytes // 4, dtype=torch.int32)


def ok_linear(**kw):
    a = dict(z=f16(3, K), trellis=stream(), svh=f16(N), bits=BITS, out_dim=N)
    a.update(kw)
    return a


@pytest.mark.parametrize("bad,msg", [
    (dict(z=f16(K)), "2-D"),
    (dict(z=torch.zeros(3, K, dtype=torch.float32)), "z must have element type"),
    (dict(trellis=stream(NB - 16)), "trellis must hold"),
    (dict(trellis=stream(NB + 16)), "trellis must hold"),
    (dict(bits=3), "trellis must hold"),
    (dict(svh=f16(N - 128)), "svh must have shape"),
    (dict(svh=torch.zeros(N, dtype=torch.float32)), "svh must have element type"),
    (dict(y=torch.zeros(3, N + 128)), "y must have shape"),
    (dict(y=torch.zeros(2, N)), "y must have shape"),
    (dict(y=torch.zeros(3, N, dtype=torch.int32)), "y must have element type"),
    (dict(out_dtype=torch.int8), "out_dtype"),
])
@pytest.mark.parametrize("engine", tq._lib.ENGINES)
def test_linear_refusals(bad, msg, engine):
    with pytest.raises(ValueError, match=msg):
        tq.linear(**ok_linear(**bad), engine=engine)


def test_linear_refuses_cpu_tensors_last():
    with pytest.raises(ValueError, match="on the GPU"):
        tq.linear(**ok_linear())
    with pytest.raises(ValueError, match="engine"):
        tq.linear(**ok_linear(), engine="other")


def test_debug_split_checks_like_linear():
    with pytest.raises(ValueError, match="trellis must hold"):
        tq.debug_linear_split(f16(1, K), stream(NB // 2), f16(N), BITS, N, split=0)


@pytest.mark.parametrize("bad,msg", [
    (dict(x=f16(K)), "2-D"),
    (dict(x=torch.zeros(2, K, dtype=torch.int32)), "x must have element type"),
    (dict(suh=f16(K + 128)), "suh must have shape"),
    (dict(suh=torch.zeros(K)), "suh must have element type"),
    (dict(z=f16(2, K - 128)), "z must have shape"),
    (dict(z=torch.zeros(2, K, dtype=torch.bfloat16)), "z must have element type"),
])
def test_rot_in_refusals(bad, msg):
    a = dict(x=f16(2, K), suh=f16(K), z=None)
    a.update(bad)
    with pytest.raises(ValueError, match=msg):
        tq.rot_in(a["x"], a["suh"], a["z"])


def test_rot_in_accepts_every_row_type_then_refuses_the_host():
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        with pytest.raises(ValueError, match="on the GPU"):
            tq.rot_in(torch.zeros(2, K, dtype=dt), f16(K))


@pytest.mark.parametrize("bad,msg", [
    (dict(suh=f16(K - 128)), "suh must have shape"),
    (dict(trellis=stream(NB * 2)), "trellis must hold"),
    (dict(svh=f16(N + 128)), "svh must have shape"),
    (dict(y=torch.zeros(1, N)), "y must have shape"),
    (dict(x=torch.zeros(2, K, dtype=torch.int16)), "x must have element type"),
])
def test_project_refusals(bad, msg):
    a = dict(x=f16(2, K), suh=f16(K), trellis=stream(), svh=f16(N), bits=BITS, out_dim=N)
    a.update(bad)
    with pytest.raises(ValueError, match=msg):
        tq.project(**a)


def test_repack_and_decode_check_the_stream_size():
    with pytest.raises(ValueError, match="trellis must hold"):
        tq.repack_strips(stream(NB - 4), BITS, K, N)
    with pytest.raises(ValueError, match="out must hold"):
        tq.repack_strips(stream(), BITS, K, N, out=stream(NB // 2))
    with pytest.raises(ValueError, match="trellis must hold"):
        tq.debug_decode_tiles(stream(NB + 4), BITS, K, N)


def test_calibration_buffers():
    with pytest.raises(ValueError, match="dst must hold"):
        tq.calib_copy(stream(1024), stream(512))
    with pytest.raises(ValueError, match="multiple of 256"):
        tq.calib_stream_read(stream(4096), torch.zeros(100, dtype=torch.int32))
    with pytest.raises(ValueError, match="out must have element type"):
        tq.calib_stream_read(stream(4096), torch.zeros(256, dtype=torch.float32))


def test_refused_shapes_reach_the_library_status():
    """A shape the library refuses (no stream size) is left to its status code."""
    with pytest.raises(ValueError, match="on the GPU"):
        tq.linear(f16(1, 200), stream(16), f16(N), BITS, N)


def test_stream_size_rule_matches_the_library():
    """The binding sizes streams without a library call; its rule must be the library's,
    refusals (0 there, None here) included."""
    from trellis_quantized_linear_tf_amd import _lib

    lib = _lib.load()
    for bits in range(0, 10):
        for k in (0, 64, 128, 200, 256, 5120, 65536, 131072):
            for n in (128, 256, 129280, 262144, 1 << 20):
                want = lib.tf_exl3_trellis_bytes(bits, k, n)
                assert (_lib._stream_bytes(bits, k, n) or 0) == want, (bits, k, n)
