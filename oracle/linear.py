"""The trellis linear: float64 evaluation, fp32 finish and a dense brute force.

Test infrastructure only (see oracle/__init__.py).

Source: the TensorFold pull request "hip exl3: the input rotation and trellis
linear for decode rows". Section "What this changes": the linear sums a row's
products of fp16 inputs and decoded fp16 weights in fp32, adds the waves'
partial sums, then applies the output rotation and svh. Section "Kernel
contract": the float64 reference does the unscaled butterflies first and the
scale afterwards (so exact zeros stay zero), and the identity test repeats the
kernel's fp32 butterflies on the host. Readings:

  R9  orientation: W is in_dim x out_dim and acc = z . W (inputs "in" to "out").
  R10 finish: y = cast_T(RN32(RN32(FWHT32(acc) * s) * svh)) per 128-column block,
      with the same butterfly order and scale as rot_in.
  R11 float64 reference: y64 = FWHT64(z64 . W64) * (1/sqrt(128)) * svh, on the
      kernel's own fp16 z and the exactly decoded W.
  R12 gate: max|y - y64| / rms(y64) <= 2e-3 for fp32 outputs; fp16/bf16
      outputs are allowed half an output ulp more. Non-finite outputs must have
      the same class (NaN, +inf, -inf) as y64.
"""

from __future__ import annotations

import os

import numpy as np

from .numfmt import (
    f16_bits_to_f32,
    f16_bits_to_f64,
    f32_to_output,
    input_to_f32,
    output_to_f64,
)
from .rotation import BLOCK, SCALE_F32, SCALE_F64, fwht128, hadamard_matrix
from .trellis import strip_tile_cols, unpack_columns

GATE = 2e-3


def accumulate_f64(z_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """acc64[r][n] = sum_k z[r][k] * W[k][n] in float64 (a library matmul)."""
    z64 = f16_bits_to_f64(np.atleast_2d(z_bits))
    w64 = f16_bits_to_f64(w_bits)
    return z64 @ w64


def finish_f64(acc64: np.ndarray, svh_bits: np.ndarray) -> np.ndarray:
    """Unscaled float64 butterflies per 128 columns, then the scale, then svh (R11)."""
    return fwht128(np.asarray(acc64, dtype=np.float64)) * SCALE_F64 * f16_bits_to_f64(svh_bits)


def finish_f32(acc32: np.ndarray, svh_bits: np.ndarray, out_dtype: str) -> np.ndarray:
    """The fp32 finish (R10): butterflies, scale and svh, each op rounded to fp32, then the cast."""
    v = fwht128(np.asarray(acc32, dtype=np.float32))
    v = (v * SCALE_F32).astype(np.float32)
    v = (v * f16_bits_to_f32(svh_bits)).astype(np.float32)
    return f32_to_output(v, out_dtype)


def reference_threads() -> int:
    """Host cores this process may run on (the threaded reference's width), capped by
    OMP_NUM_THREADS where the environment sets a CPU share."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # platforms without CPU affinity
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def linear_f64(z_bits: np.ndarray, trellis: np.ndarray, bits: int, in_dim: int, out_dim: int,
               svh_bits: np.ndarray, strips=None, strip_chunk: int | None = None, threads: int = 1) -> np.ndarray:
    """y64 [rows][128 * len(strips)] for the given 128-column strips (default: all).

    The strips are taken in chunks of `strip_chunk` (default 32, or fewer so that every
    thread of the pool gets a chunk); each chunk unpacks its columns'
    weights, sums z . W in float64 and finishes its blocks. With threads > 1 the chunks
    are spread over a pool of that many threads (the page's float64 references split
    their work by ranges of columns in the same way). A chunk's arithmetic does not
    depend on which thread runs it, and every output keeps its own k order, so the
    result is bit-identical to one thread's."""
    z_bits = np.atleast_2d(np.asarray(z_bits, dtype=np.uint16))
    assert z_bits.shape[1] == in_dim
    if strips is None:
        strips = np.arange(out_dim // BLOCK)
    strips = np.asarray(strips, dtype=np.int64).reshape(-1)
    out = np.empty((z_bits.shape[0], BLOCK * strips.size), dtype=np.float64)
    svh_bits = np.asarray(svh_bits, dtype=np.uint16)
    if strip_chunk is None:
        strip_chunk = max(1, min(32, -(-strips.size // max(1, threads))))

    def chunk(i0: int) -> None:
        sel = strips[i0 : i0 + strip_chunk]
        w = unpack_columns(trellis, bits, in_dim, out_dim, strip_tile_cols(sel))
        acc = accumulate_f64(z_bits, w)
        cols = (BLOCK * sel[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)
        out[:, BLOCK * i0 : BLOCK * (i0 + sel.size)] = finish_f64(acc, svh_bits[cols])

    starts = range(0, strips.size, strip_chunk)
    if threads <= 1 or len(starts) <= 1:
        for i0 in starts:
            chunk(i0)
        return out
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    # One BLAS thread per worker: the pool is the parallelism.
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=threads) as pool:
        for f in [pool.submit(chunk, i0) for i0 in starts]:
            f.result()
    return out


def strip_columns(strips) -> np.ndarray:
    strips = np.asarray(strips, dtype=np.int64).reshape(-1)
    return (BLOCK * strips[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)


# ---------------------------------------------------------------------------
# Dense brute force on tiny shapes: explicit rotation matrices, no butterflies.


def block_hadamard(n: int) -> np.ndarray:
    """Block-diagonal of explicit 128 x 128 Sylvester matrices, scaled by 1/sqrt(128)."""
    h = hadamard_matrix(BLOCK).astype(np.float64) * SCALE_F64
    return np.kron(np.eye(n // BLOCK), h)


def dense_from_z(z_bits: np.ndarray, w_bits: np.ndarray, svh_bits: np.ndarray) -> np.ndarray:
    """y = z . W . H_N . diag(svh) with explicit matrices."""
    n = w_bits.shape[1]
    z64 = f16_bits_to_f64(np.atleast_2d(z_bits))
    w64 = f16_bits_to_f64(w_bits)
    return z64 @ w64 @ block_hadamard(n) @ np.diag(f16_bits_to_f64(svh_bits))


def dense_from_x(x: np.ndarray, x_dtype: str, suh_bits: np.ndarray, w_bits: np.ndarray,
                 svh_bits: np.ndarray) -> np.ndarray:
    """y = x . diag(suh) . H_K . W . H_N . diag(svh): the whole projection without z's rounding."""
    k, n = w_bits.shape
    x64 = input_to_f32(np.atleast_2d(x), x_dtype).astype(np.float64)
    w_eff = (np.diag(f16_bits_to_f64(suh_bits)) @ block_hadamard(k) @ f16_bits_to_f64(w_bits)
             @ block_hadamard(n) @ np.diag(f16_bits_to_f64(svh_bits)))
    return x64 @ w_eff


# ---------------------------------------------------------------------------
# The gate (R12).


def half_ulp(v64: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the output type at |v| (0 for fp32 outputs)."""
    if dtype == "f32":
        return np.zeros_like(v64)
    mant, emin = (10, -14) if dtype == "f16" else (7, -126)
    a = np.abs(np.where(np.isfinite(v64), v64, 0.0))
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, emin)
    return np.ldexp(1.0, e - mant - 1)


def classes(v: np.ndarray) -> np.ndarray:
    """0 finite, 1 NaN, 2 +inf, 3 -inf."""
    v = np.asarray(v, dtype=np.float64)
    return np.select([np.isnan(v), v == np.inf, v == -np.inf], [1, 2, 3], 0)


def gate_error(y: np.ndarray, y_dtype: str, y64: np.ndarray) -> float:
    """max(|y - y64| - half_ulp_T(y64)) / rms(y64) over finite outputs; inf if classes differ."""
    yv = output_to_f64(y, y_dtype)
    y64 = np.asarray(y64, dtype=np.float64)
    assert yv.shape == y64.shape
    if not np.array_equal(classes(yv), classes(y64)):
        return float("inf")
    fin = np.isfinite(y64)
    if not fin.any():
        return 0.0
    ref = y64[fin]
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.maximum(np.abs(yv[fin] - ref) - half_ulp(ref, y_dtype), 0.0)
    if rms == 0.0:
        return 0.0 if float(d.max()) == 0.0 else float("inf")
    return float(d.max()) / rms
