"""Storage formats: fp16 and bf16 bits, fp32 values, and round-to-nearest-even.

Test infrastructure only (see oracle/__init__.py).

The rounding functions work from the IEEE 754 definition: find the spacing of
the target format at the value's binade, scale the value to an integer count of
that spacing (exact in float64, a power-of-two scaling), round that count to the
nearest integer with ties to even (numpy.rint), and scale back. Overflow goes to
signed infinity, subnormals are kept, NaN maps to the quiet NaN.
"""

from __future__ import annotations

import numpy as np

F16_QNAN = 0x7E00
BF16_QNAN = 0x7FC0


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of fp16 bit patterns: sign, 5-bit exponent (bias 15), 10-bit fraction."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15 == 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1024.0 + f, (e - 25).astype(np.int64))
    sub = np.ldexp(f, -24)
    v = np.where(e == 0, sub, normal)
    v = np.where(e == 31, np.where(f == 0, np.inf, np.nan), v)
    return sign * v


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """fp16 -> fp32 is exact (every fp16 value is an fp32 value)."""
    return f16_bits_to_f64(bits).astype(np.float32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an fp32 pattern."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _round_to_grid(v: np.ndarray, mant_bits: int, emin: int, max_finite: float) -> np.ndarray:
    """Nearest-even value of a binary format with `mant_bits` fraction bits, smallest normal
    exponent `emin` and largest finite value `max_finite`; returns float64 values."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    a = np.where(np.isfinite(a), a, 0.0)  # inf/nan are patched in below
    _, ex = np.frexp(a)  # a = m * 2^ex with m in [0.5, 1)
    e = np.maximum(ex - 1, emin)  # binade exponent, clamped into the subnormal range
    spacing_exp = e - mant_bits
    q = np.ldexp(a, -spacing_exp)  # exact: a / spacing
    r = np.ldexp(np.rint(q), spacing_exp)  # rint rounds half to even
    # Overflow: values at or beyond max_finite + half a spacing of the top binade round to inf.
    top_half_spacing = np.ldexp(1.0, int(np.floor(np.log2(max_finite))) - mant_bits - 1)
    r = np.where(a >= max_finite + top_half_spacing, np.inf, r)
    r = np.where(np.isinf(v), np.inf, r)
    r = np.copysign(r, v)
    return np.where(np.isnan(v), np.nan, r)


def rn_f16_value(v: np.ndarray) -> np.ndarray:
    """Round to fp16 (10 fraction bits, min normal 2^-14, max 65504); float64 result."""
    return _round_to_grid(v, 10, -14, 65504.0)


def rn_bf16_value(v: np.ndarray) -> np.ndarray:
    """Round to bf16 (7 fraction bits, min normal 2^-126, max (2-2^-7)*2^127); float64 result."""
    return _round_to_grid(v, 7, -126, float(np.ldexp(255.0, 120)))


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """fp16 bits of a float64 value rounded once to fp16."""
    r = rn_f16_value(v)
    neg = np.signbit(r)
    a = np.abs(r)
    a = np.where(np.isfinite(a), a, 0.0)  # inf/nan are encoded below
    # Encode the (now exactly representable) magnitude.
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -14)
    frac = np.ldexp(a, -(e - 10)).astype(np.int64)  # integer count of spacings, < 2048
    is_sub = a < 2.0 ** -14
    enc = np.where(is_sub, frac, ((e + 15) << 10) | (frac - 1024))
    enc = np.where(a == 0, 0, enc)
    enc = np.where(np.isinf(r), 0x7C00, enc)
    enc = np.where(neg, enc | 0x8000, enc)
    enc = np.where(np.isnan(r), F16_QNAN, enc)
    return enc.astype(np.uint16)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bits of a float64 value rounded once to bf16."""
    r = rn_bf16_value(v)
    # The rounded value is an fp32 value whose low 16 bits are zero.
    u = r.astype(np.float32).view(np.uint32)
    out = (u >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(r), np.uint16(BF16_QNAN) | (out & np.uint16(0x8000)), out).astype(np.uint16)


def f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float32)


def f32_bits(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float32).view(np.uint32)


def bits_f32(u: int) -> np.float32:
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def input_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored rows to fp32 (exact for all three input types)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return f16_bits_to_f32(x)
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    raise ValueError(dtype)


def f32_to_output(y32: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 results to the output type: f32 unchanged, f16/bf16 bits rounded once."""
    y32 = np.asarray(y32, dtype=np.float32)
    if dtype == "f32":
        return y32
    if dtype == "f16":
        return f64_to_f16_bits(y32.astype(np.float64))
    if dtype == "bf16":
        return f64_to_bf16_bits(y32.astype(np.float64))
    raise ValueError(dtype)


def output_to_f64(y: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(y, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return f16_bits_to_f64(y)
    if dtype == "bf16":
        return bf16_bits_to_f32(y).astype(np.float64)
    raise ValueError(dtype)
