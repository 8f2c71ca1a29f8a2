"""Helpers for the GPU tests: move numpy arrays of the inputs' storage formats to
the device and back, and run the library's entry points on them."""

import sys

import numpy as np
import torch

import trellis_quantized_linear_tf_amd as tq

DEV = torch.device("cuda:0")
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def up(a, dtype=None):
    """uint16 bits -> fp16/bf16 tensor (dtype given), float32 -> float32, uint32 -> int32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(DEV)
        return t.view(TORCH_DT[dtype or "f16"])
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(DEV)
    raise TypeError(a.dtype)


def down(t):
    """Device tensor -> numpy: fp16/bf16 as uint16 bits, float32 as float32."""
    t = t.detach()
    if t.dtype in (torch.float16, torch.bfloat16, torch.int16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    raise TypeError(t.dtype)


def rot_in(x, x_dtype, suh):
    z = tq.rot_in(up(x, x_dtype), up(suh))
    torch.cuda.synchronize()
    return down(z)


def linear(z_bits, stream, svh, bits, n, out="f32", waves=0, stream_t=None, engine="dot2"):
    zt = up(z_bits)
    tt = stream_t if stream_t is not None else up(stream)
    y = tq.linear(zt, tt, up(svh), bits, n, out_dtype=TORCH_DT[out], waves=waves, engine=engine)
    torch.cuda.synchronize()
    return down(y)


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def is_nan_bits(a, fmt):
    a = np.asarray(a)
    if fmt == "f16":
        return ((a & 0x7C00) == 0x7C00) & ((a & 0x3FF) != 0)
    return ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)


def same_bits(a, b, fmt="f16"):
    """Bit equality, with every NaN counted equal to every NaN (payloads are free).
    fmt names the format of uint16 arrays (f16 or bf16)."""
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return False
    if a.dtype == np.float32:
        na, nb = np.isnan(a), np.isnan(b)
        return bool(np.array_equal(na, nb) and np.array_equal(f32_bits(a)[~na], f32_bits(b)[~nb]))
    na, nb = is_nan_bits(a, fmt), is_nan_bits(b, fmt)
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb]))
