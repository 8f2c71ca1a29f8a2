"""128-point Walsh-Hadamard transform and rot_in's fp32 steps.

Test infrastructure only (see oracle/__init__.py).

Source: the TensorFold pull request "hip exl3: the input rotation and trellis
linear for decode rows", section "What this changes" (rot_in multiplies x by
suh in fp32, applies the 128-point butterflies, then the scale, and rounds to
fp16 once) and its "Checks on this head" section (the scale is a multiply by
the fp32 value of 1/sqrt(128), not a division; the product and the fp16
conversion are two roundings, not one fused rounding). Readings taken where the
page is silent:

  R6 butterfly order: Sylvester (natural) order, stages h = 1, 2, 4, ..., 64;
     in each stage the pair (i, i+h) with i & h == 0 becomes (a + b, a - b).
  R7 scale: s = RN32(1/sqrt(128)) = 0x3DB504F3, multiplied after all stages.
  R8 roundings: fp32 rounding after the product, after every butterfly add or
     subtract and after the scale, then one fp16 rounding (nearest even,
     subnormals kept, overflow to infinity).
"""

from __future__ import annotations

import numpy as np

from .numfmt import bits_f32, f16_bits_to_f32, f64_to_f16_bits, input_to_f32

BLOCK = 128
SCALE_F32_BITS = 0x3DB504F3
SCALE_F32 = bits_f32(SCALE_F32_BITS)
SCALE_F64 = 1.0 / np.sqrt(128.0)


def fwht128(v: np.ndarray) -> np.ndarray:
    """Unscaled butterflies over each 128-block of the last axis, in v's own float
    type (float32 gives one fp32 rounding per add/subtract; float64 likewise)."""
    v = np.array(v, copy=True)
    n = v.shape[-1]
    assert n % BLOCK == 0
    lead = v.shape[:-1]
    w = v.reshape(-1, n // BLOCK, BLOCK)
    h = 1
    while h < BLOCK:
        g = w.reshape(w.shape[0], w.shape[1], BLOCK // (2 * h), 2, h)
        a = g[:, :, :, 0, :].copy()
        b = g[:, :, :, 1, :].copy()
        g[:, :, :, 0, :] = a + b
        g[:, :, :, 1, :] = a - b
        h *= 2
    return w.reshape(*lead, n)


def hadamard_matrix(n: int = BLOCK) -> np.ndarray:
    """Explicit Sylvester matrix H[i][j] = (-1)^popcount(i & j), as int64."""
    i = np.arange(n)
    pc = np.vectorize(lambda t: bin(int(t)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rot_in(x: np.ndarray, x_dtype: str, suh_bits: np.ndarray) -> np.ndarray:
    """z = RN16(RN32(FWHT32(RN32(x * suh)) * s)) per 128-block; returns fp16 bits [rows][in_dim]."""
    x32 = input_to_f32(x, x_dtype)
    suh32 = f16_bits_to_f32(suh_bits)
    assert x32.shape[-1] == suh32.shape[-1]
    p = (x32 * suh32).astype(np.float32)
    v = fwht128(p)
    v = (v * SCALE_F32).astype(np.float32)
    return f64_to_f16_bits(v.astype(np.float64))


def rot_in_f64(x: np.ndarray, x_dtype: str, suh_bits: np.ndarray) -> np.ndarray:
    """The same rotation in float64 with no rounding to fp16 (the error reference)."""
    x64 = input_to_f32(x, x_dtype).astype(np.float64)
    suh64 = f16_bits_to_f32(suh_bits).astype(np.float64)
    return fwht128(x64 * suh64) * SCALE_F64
