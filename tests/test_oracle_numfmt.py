"""Pins for oracle/numfmt.py: the fp16 / bf16 codecs and round-to-nearest-even.

Checked against what IEEE 754 fixes, through routes that share nothing with the
oracle's code: numpy's and torch's own conversions, exhaustive enumeration of
all 65,536 fp16 patterns, and a brute-force nearest search with exact rationals.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import numfmt as nf

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_f16_decode_all_patterns_match_numpy():
    ours = nf.f16_bits_to_f64(ALL16)
    ref = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_round_trip_all_patterns():
    v = nf.f16_bits_to_f64(ALL16)
    back = nf.f64_to_f16_bits(v)
    keep = ~np.isnan(v)
    assert np.array_equal(back[keep], ALL16[keep])
    assert np.all(back[~keep] == nf.F16_QNAN)


def _wide_values(n, seed):
    mag = np.exp(synth.normals(seed, n, 9.0))
    sgn = np.where(synth.splitmix64(seed + 1, n) & np.uint64(1), -1.0, 1.0)
    return (sgn * mag).astype(np.float32)


def test_rn16_matches_numpy_on_wide_range():
    v = _wide_values(400_000, 11)
    assert np.array_equal(nf.f64_to_f16_bits(v.astype(np.float64)), v.astype(np.float16).view(np.uint16))


def test_rn16_ties_go_to_even():
    finite = ALL16[(ALL16 & 0x7C00) != 0x7C00]
    pos = finite[finite < 0x7BFF]  # positive, with a finite successor
    a = nf.f16_bits_to_f64(pos)
    b = nf.f16_bits_to_f64(pos + 1)
    mid = (a + b) / 2.0  # exact in float64
    got = nf.f64_to_f16_bits(mid)
    even = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(got, even.astype(np.uint16))


def test_rn16_overflow_boundary():
    got = nf.f64_to_f16_bits(np.array([65504.0, 65519.999, 65520.0, -65520.0, 1e9, np.inf, -np.inf]))
    assert [hex(v) for v in got] == ["0x7bff", "0x7bff", "0x7c00", "0xfc00", "0x7c00", "0x7c00", "0xfc00"]


def test_rn16_brute_force_nearest():
    """Nearest finite fp16 by exhaustive search with exact rationals, ties to even."""
    finite = ALL16[((ALL16 & 0x7C00) != 0x7C00)]
    finite = finite[finite < 0x8000]  # non-negative
    vals = nf.f16_bits_to_f64(finite)
    order = np.argsort(vals)
    vals, finite = vals[order], finite[order]
    x = np.abs(_wide_values(300, 5)).astype(np.float64) % 60000.0
    x = np.concatenate([x, [2.0 ** -25, 3 * 2.0 ** -26, 1e-7, 0.0]])
    for xi in x:
        q = Fraction(float(xi))
        j = int(np.searchsorted(vals, xi))
        cands = [i for i in (j - 1, j, j + 1) if 0 <= i < vals.size]
        best = min(cands, key=lambda i: (abs(Fraction(float(vals[i])) - q), int(finite[i]) & 1))
        assert nf.f64_to_f16_bits(np.array([xi]))[0] == finite[best], xi


def test_rnbf16_matches_torch():
    torch = pytest.importorskip("torch")
    v = _wide_values(400_000, 23) * np.float32(1e30)
    v = np.concatenate([v, _wide_values(100_000, 29) * np.float32(1e-35)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf.f64_to_bf16_bits(v.astype(np.float64)), ref)


def test_bf16_widen_is_top_half():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F80, 0x0000, 0x8000], dtype=np.uint16)
    v = nf.bf16_bits_to_f32(bits)
    assert list(v[:2]) == [1.0, -1.0]
    assert v[2] == np.float32(2.0 ** -133)
    assert np.isinf(v[3]) and v[4] == 0 and np.signbit(v[5])
