"""Pins for oracle/trellis.py: the stream readers, the tile layout and the codebook.

The pages name the trellis and the mul1 codebook but print no constants, so the
format is this build's reading (stated in oracle/trellis.py and include/tf_exl3.h).
What pins the oracle to that reading, independently of its own code:
  - a bit-at-a-time reader against the vectorized word reader;
  - states rebuilt from the symbols a stream was packed from, with Python big
    integers (a third route);
  - streams whose tiles are constant or carry their own position, checking the
    value and tile order;
  - the codebook evaluated with exact rationals and a brute-force nearest fp16
    search; its distribution (mean ~0, sd ~1, no zero or subnormal weights);
  - the all-ones stream decoding to one weight at every width, which the exact
    linear gate builds on.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import numfmt as nf
from oracle import trellis as tr

WIDTHS = tr.WIDTHS


@pytest.mark.parametrize("bits", WIDTHS)
def test_two_readers_agree(bits):
    words = synth.uniform_words(100 + bits, 8 * bits * 6).reshape(6, 8 * bits)
    fast = tr.tile_states(words, bits)
    for t in range(6):
        assert list(fast[t]) == tr.tile_states_bitwise(words[t], bits)


@pytest.mark.parametrize("bits", WIDTHS)
def test_states_from_packed_symbols(bits):
    sym = (synth.splitmix64(300 + bits, 256) % np.uint64(1 << bits)).astype(np.uint64)
    words = synth.symbols_to_words(sym, bits)
    stream = 0
    for i, s in enumerate(sym):
        stream |= int(s) << (bits * i)
    n = 256 * bits
    doubled = stream | (stream << n)  # the window wraps inside the tile
    expect = [(doubled >> (bits * j)) & 0xFFFF for j in range(256)]
    assert list(tr.tile_states(words, bits)) == expect
    assert tr.tile_states_bitwise(words, bits) == expect


def _planted_states(words, bits, plant):
    """A copy of the word reader with one mistake planted: the second window of
    each pair starts one bit late, or the last windows of a tile read past its
    end instead of wrapping to its first word."""
    nw = tr.tile_words(bits)
    j = np.arange(256, dtype=np.int64)
    p = j * bits + ((j & 1) if plant == "odd_window_one_bit_late" else 0)
    w = np.concatenate([np.asarray(words, dtype=np.uint64), np.zeros(2, dtype=np.uint64)])
    w0 = (p >> 5) % nw
    w1 = (w0 + 1) % nw if plant != "no_wrap" else w0 + 1
    pair = (w[w1] << np.uint64(32)) | w[w0]
    return ((pair >> (p & 31).astype(np.uint64)) & np.uint64(0xFFFF)).astype(np.uint32)


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("plant", ["odd_window_one_bit_late", "no_wrap"])
def test_planted_reader_mistakes_fail_the_reader_pins(bits, plant):
    """The page's decode plant (the second window of each pair one bit off) and a
    dropped tail wrap each fail the random-tile reader pins above: the bit-at-a-time
    reader and the states rebuilt from packed symbols both disagree with them."""
    words = synth.uniform_words(700 + bits, 8 * bits)
    assert np.array_equal(_planted_states(words, bits, "none"), tr.tile_states(words, bits))  # the copy itself
    assert list(_planted_states(words, bits, plant)) != tr.tile_states_bitwise(words, bits)
    sym = (synth.splitmix64(710 + bits, 256) % np.uint64(1 << bits)).astype(np.uint64)
    packed = synth.symbols_to_words(sym, bits)
    assert not np.array_equal(_planted_states(packed, bits, plant), tr.tile_states(packed, bits))


@pytest.mark.parametrize("bits", WIDTHS)
def test_constant_streams_cannot_see_the_window_plant(bits):
    """Why the reader pins use random tiles: an all-ones stream gives 0xFFFF in every
    window wherever it starts, so it passes the planted reader too."""
    ones = np.full(8 * bits, 0xFFFFFFFF, dtype=np.uint32)
    assert (_planted_states(ones, bits, "odd_window_one_bit_late") == 0xFFFF).all()


def _hand_f16(bits16: int) -> Fraction:
    e = (bits16 >> 10) & 0x1F
    f = bits16 & 0x3FF
    mag = Fraction(1024 + f, 2 ** (25 - e)) if e else Fraction(f, 2 ** 24)
    return -mag if bits16 >> 15 else mag


def _nearest_f16_brute(q: Fraction) -> int:
    finite = [b for b in range(65536) if (b & 0x7C00) != 0x7C00]
    vals = nf.f16_bits_to_f64(np.array(finite, dtype=np.uint16))
    j = int(np.argmin(np.abs(vals - float(q))))
    cands = [finite[i] for i in range(max(0, j - 2), min(len(finite), j + 3))]
    return min(cands, key=lambda b: (abs(_hand_f16(b) - q), b & 1))


def test_codebook_against_exact_rationals():
    states = [0, 1, 2, 0xFFFF, 0x8000, 0x1234] + [int(s) for s in synth.splitmix64(7, 40) % np.uint64(65536)]
    a = _hand_f16(0x1EEE)
    b = _hand_f16(0xC931)
    for s in states:
        x = (s * 0x9E3779) % (1 << 32)
        h = sum(x.to_bytes(4, "little"))
        want = _nearest_f16_brute((1024 + h) * a + b)
        got = int(tr.decode_states(np.array([s]))[0])
        assert got == want, (hex(s), hex(got), hex(want))


def test_codebook_constants_are_the_stated_roundings():
    # A is the nearest fp16 to sqrt(3)/256 and B the nearest fp16 to -1534*A.
    import math

    assert _nearest_f16_brute(Fraction(math.sqrt(3) / 256)) == tr.CB_SCALE_BITS
    assert _nearest_f16_brute(-1534 * _hand_f16(tr.CB_SCALE_BITS)) == tr.CB_BIAS_BITS


def test_codebook_distribution():
    w = nf.f16_bits_to_f64(tr.decode_states(np.arange(65536)))
    assert abs(w.mean()) < 0.01
    assert 0.99 < w.std() < 1.01
    assert np.all(np.abs(w) >= 2.0 ** -14)  # no zero or subnormal weight
    assert np.abs(w).max() < 3.5
    assert len(np.unique(w)) <= 1021  # one value per byte sum h = 0..1020


def test_codebook_is_monotone_in_byte_sum():
    s = np.arange(65536, dtype=np.uint64)
    x = (s * np.uint64(0x9E3779)) & np.uint64(0xFFFFFFFF)
    h = sum((x >> np.uint64(8 * i)) & np.uint64(0xFF) for i in range(4)).astype(np.int64)
    w = nf.f16_bits_to_f64(tr.decode_states(s))
    order = np.argsort(h, kind="stable")
    assert np.all(np.diff(w[order]) >= 0)


def test_1024_plus_h_is_fp16_pattern_0x6400_plus_h():
    h = np.arange(1024)
    assert np.array_equal(nf.f16_bits_to_f64((0x6400 + h).astype(np.uint16)), 1024.0 + h)


@pytest.mark.parametrize("bits", WIDTHS)
def test_constant_streams(bits):
    ones = synth.constant_trellis(bits, 32, 256, ones=True)
    zeros = synth.constant_trellis(bits, 32, 256, ones=False)
    w1 = tr.unpack(ones, bits, 32, 256)
    w0 = tr.unpack(zeros, bits, 32, 256)
    assert np.all(w1 == w1.flat[0]) and np.all(w0 == w0.flat[0])
    assert w1.flat[0] == _nearest_f16_brute(Fraction(1024 + 607) * _hand_f16(0x1EEE) + _hand_f16(0xC931))
    assert nf.f16_bits_to_f64(w1.flat[0]) * 4096 == 2682.0  # an integer: the exact gate uses it


@pytest.mark.parametrize("bits", WIDTHS)
def test_tile_order(bits):
    """Tile (kt, nt) filled with one repeated symbol decodes to one constant block there."""
    k, n = 64, 384
    kt_n, nt_n = k // 16, n // 16
    sym_of = lambda kt, nt: (7 * kt + 3 * nt + 1) % (1 << bits)
    tiles = []
    for kt in range(kt_n):
        for nt in range(nt_n):
            tiles.append(synth.symbols_to_words(np.full(256, sym_of(kt, nt), dtype=np.uint64), bits))
    stream = np.concatenate(tiles)
    w = tr.unpack(stream, bits, k, n)
    for kt in range(kt_n):
        for nt in range(nt_n):
            c = sym_of(kt, nt)
            state = 0
            for m in range(0, 16 + bits, bits):
                state |= c << m
            want = tr.decode_states(np.array([state & 0xFFFF]))[0]
            assert np.all(w[16 * kt : 16 * kt + 16, 16 * nt : 16 * nt + 16] == want)


def test_value_order_inside_a_tile():
    """At 8 bits, symbol j = j makes value j's state j | (j+1) << 8; it must land at k = j%16, n = j//16."""
    words = synth.symbols_to_words(np.arange(256, dtype=np.uint64), 8)
    w = tr.unpack(words, 8, 16, 16)
    for j in range(256):
        state = j | (((j + 1) % 256) << 8)
        assert w[j % 16, j // 16] == tr.decode_states(np.array([state]))[0]


def test_trellis_bytes():
    assert tr.trellis_bytes(4, 5120, 129280) == 330_956_800
    assert tr.trellis_bytes(8, 5120, 129280) == 661_913_600
    assert tr.trellis_bytes(3, 6144, 25600) == 58_982_400


@pytest.mark.parametrize("bits", WIDTHS)
def test_strips_layout_places_each_tile(bits):
    """Each tile, tagged with its (kt, nt), sits at the stated strips-layout offset, and
    strip s's region holds exactly its 8 tile columns, tile rows in ascending kt."""
    k, n = 64, 384
    kt_n, nt_n, tw = k // 16, n // 16, 8 * bits
    tiles = np.empty((kt_n, nt_n, tw), dtype=np.uint32)
    for kt in range(kt_n):
        for nt in range(nt_n):
            tiles[kt, nt] = (kt << 16) | nt
    strips = tr.tiles_to_strips(tiles.reshape(-1), bits, k, n)
    for kt in range(kt_n):
        for nt in range(nt_n):
            o = tr.strips_tile_offset(bits, k, kt, nt)
            assert np.all(strips[o : o + tw] == ((kt << 16) | nt))
    region = kt_n * 8 * tw
    for s in range(nt_n // 8):
        tags = strips[s * region : (s + 1) * region : tw]
        want = [(kt << 16) | (8 * s + t) for kt in range(kt_n) for t in range(8)]
        assert tags.tolist() == want


@pytest.mark.parametrize("bits", WIDTHS)
def test_strips_round_trip(bits):
    k, n = 256, 640
    stream = synth.trellis_words(3000 + bits, bits, k, n)
    strips = tr.tiles_to_strips(stream, bits, k, n)
    assert strips.size == stream.size and not np.array_equal(strips, stream)
    assert np.array_equal(tr.strips_to_tiles(strips, bits, k, n), stream)
    assert np.array_equal(np.sort(strips), np.sort(stream))


def test_strips_layout_of_one_strip_is_the_tile_layout():
    """With 128 columns there is one strip, and both layouts coincide."""
    stream = synth.trellis_words(3100, 4, 512, 128)
    assert np.array_equal(tr.tiles_to_strips(stream, 4, 512, 128), stream)
