"""Seeded synthetic inputs for the EXL3 decode-row projection.

This module is the only code that the GPU path's tests and bench share with the
CPU oracle's tests. It draws random numbers and stores them in the input formats
(uint32 trellis words, fp32/fp16/bf16 rows, fp16 sign vectors). It contains none
of the projection's arithmetic: no trellis decoding, no codebook, no Hadamard
rotation and no output rounding rule.

Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014). The i-th output (i = 1, 2, ...) of a stream
with seed S is mix(S + i * 0x9E3779B97F4A7C15), where mix is the published
finalizer. Being counter-based, any slice of a stream can be drawn on its own.

Seeds follow one rule: seed = 1000 * workload + stream, with streams
0 = trellis words, 1 = input rows, 2 = suh, 3 = svh, 4 = extra rows.
"""

from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

STREAM_TRELLIS = 0
STREAM_ROWS = 1
STREAM_SUH = 2
STREAM_SVH = 3
STREAM_EXTRA = 4

F16_ONE = 0x3C00
F16_MINUS_ONE = 0xBC00


def seed_for(workload: int, stream: int) -> int:
    return 1000 * int(workload) + int(stream)


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset+1 .. offset+n of the SplitMix64 stream `seed` (uint64)."""
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        return z ^ (z >> np.uint64(31))


def uniform_words(seed: int, n_words: int, chunk: int = 1 << 23) -> np.ndarray:
    """n_words i.i.d. uniform uint32 words; draw i gives words 2i (low) and 2i+1 (high)."""
    out = np.empty(n_words + (n_words & 1), dtype=np.uint32)
    n_draws = out.size // 2
    for d0 in range(0, n_draws, chunk):
        d1 = min(n_draws, d0 + chunk)
        r = splitmix64(seed, d1 - d0, d0)
        out[2 * d0 : 2 * d1 : 2] = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32)
        out[2 * d0 + 1 : 2 * d1 : 2] = (r >> np.uint64(32)).astype(np.uint32)
    return out[:n_words]


def trellis_words(seed: int, bits: int, in_dim: int, out_dim: int) -> np.ndarray:
    """Uniform random stream bits for an in_dim x out_dim trellis at `bits` bits per weight."""
    n_bytes = in_dim * out_dim * bits // 8
    assert n_bytes % 4 == 0
    return uniform_words(seed, n_bytes // 4)


def constant_trellis(bits: int, in_dim: int, out_dim: int, ones: bool) -> np.ndarray:
    """A stream whose every bit is 1 (ones=True) or 0."""
    n = in_dim * out_dim * bits // 32
    return np.full(n, 0xFFFFFFFF if ones else 0, dtype=np.uint32)


def _unit_open(r: np.ndarray) -> np.ndarray:
    """(0, 1] from the top 53 bits."""
    return ((r >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def _unit_closed(r: np.ndarray) -> np.ndarray:
    """[0, 1) from the top 53 bits."""
    return (r >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normals(seed: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """n draws of N(0, sigma^2) in float64 by the Box-Muller transform."""
    m = (n + 1) // 2
    r = splitmix64(seed, 2 * m)
    u1 = _unit_open(r[0::2])
    u2 = _unit_closed(r[1::2])
    rad = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = rad * np.cos(2.0 * np.pi * u2)
    out[1::2] = rad * np.sin(2.0 * np.pi * u2)
    return out[:n] * sigma


def student_t3(seed: int, n: int, scale: float = 4.0) -> np.ndarray:
    """n draws of scale * t with 3 degrees of freedom: Z / sqrt((Z1^2+Z2^2+Z3^2)/3)."""
    g = normals(seed, 4 * n).reshape(n, 4)
    chi = (g[:, 1] ** 2 + g[:, 2] ** 2 + g[:, 3] ** 2) / 3.0
    return scale * g[:, 0] / np.sqrt(chi)


# ---------------------------------------------------------------------------
# Storage formats of the inputs. These round a float64 draw to the storage
# type once (round to nearest, ties to even) and return the stored bits.


def store_f32(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def store_f16(v: np.ndarray) -> np.ndarray:
    """float64 -> fp16 bits (numpy's conversion rounds to nearest even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def store_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> fp32 -> bf16 bits, each step to nearest even (finite inputs)."""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def store(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return store_f32(v)
    if dtype == "f16":
        return store_f16(v)
    if dtype == "bf16":
        return store_bf16(v)
    raise ValueError(dtype)


def rows(seed: int, n_rows: int, in_dim: int, dtype: str, sigma: float = 1.0) -> np.ndarray:
    """[n_rows][in_dim] rows ~ N(0, sigma^2) in storage dtype (f32 array or u16 bits)."""
    v = normals(seed, n_rows * in_dim, sigma).reshape(n_rows, in_dim)
    return store(v, dtype)


def heavy_rows(seed: int, n_rows: int, in_dim: int, scale: float = 4.0) -> np.ndarray:
    """[n_rows][in_dim] fp32 rows drawn scale * t_3 (heavy tailed)."""
    return store_f32(student_t3(seed, n_rows * in_dim, scale).reshape(n_rows, in_dim))


def signs(seed: int, n: int) -> np.ndarray:
    """n random +-1 values as fp16 bits (bit 0 of each draw picks the sign)."""
    r = splitmix64(seed, n)
    neg = (r & np.uint64(1)).astype(bool)
    return np.where(neg, F16_MINUS_ONE, F16_ONE).astype(np.uint16)


def scales(seed: int, n: int, lo: float = 0.5, hi: float = 2.0) -> np.ndarray:
    """n random fp16 values of random sign and magnitude in [lo, hi) (non +-1 scale vectors)."""
    r = splitmix64(seed, n)
    mag = lo + (hi - lo) * _unit_closed(r)
    sgn = np.where((r & np.uint64(1)).astype(bool), -1.0, 1.0)
    return store_f16(sgn * mag)


def symbols_to_words(symbols: np.ndarray, bits: int) -> np.ndarray:
    """Pack a sequence of b-bit symbols, first symbol in the lowest bits of word 0,
    little-endian and LSB-first, into uint32 words (the storage order of the stream)."""
    symbols = np.asarray(symbols, dtype=np.uint64)
    n_bits = symbols.size * bits
    assert n_bits % 32 == 0
    bitarr = ((symbols[:, None] >> np.arange(bits, dtype=np.uint64)) & np.uint64(1)).astype(np.uint8)
    flat = bitarr.reshape(-1, 32).astype(np.uint64)
    return (flat << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
