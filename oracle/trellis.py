"""Trellis stream reader and the mul1-style codebook.

Test infrastructure only (see oracle/__init__.py).

Source: the TensorFold pull request "hip exl3: the input rotation and trellis
linear for decode rows" (section "What this changes") describes a K-bit
shift-register trellis over 16 x 16 weight tiles, decoded through the mul1
codebook with one fp16 fused multiply-add per value; its "Kernel contract"
section sizes each tile at 256 * K bits (the static LDS records hold eight
tiles per wave at each width). The page prints no codebook constants and no bit
or value order, so this module fixes one concrete format (readings, in order):

  R1 stream bits: a tile is 8*K little-endian uint32 words; bit i of the tile is
     (word[i >> 5] >> (i & 31)) & 1 (least significant bit first).
  R2 states: value j (0..255) of a tile has the 16-bit state whose bit t is
     stream bit (j*K + t) mod (256*K): a window that advances K bits per value
     and wraps inside the tile (tail-biting), so any 256*K-bit string is a tile.
  R3 value order: value j sits at row k = j mod 16, column n = j div 16 of the
     tile, so a column's 16 weights are 16 consecutive windows and (k, k+1)
     pairs are adjacent values.
  R4 tile order: tile (kt, nt) of an in_dim x out_dim matrix starts at word
     (kt * out_dim/16 + nt) * 8K (row-major tiles, the "tile layout").
  R21 strips layout (the identity test of "Checks on this head" also runs on a
     layout it calls the strips layout, at 8 waves, and does not define it):
     the same tiles, ordered so that each
     128-column strip (8 tile columns) is one contiguous stream: tile (kt, nt)
     starts at word ((nt div 8) * in_dim/16 + kt) * 8 + nt mod 8, times 8K.
  R5 codebook: x = (state * 0x9E3779) mod 2^32 (a 24-bit Fibonacci-hashing
     multiplier, floor(2^24 / golden ratio) rounded to odd); h = sum of the four
     bytes of x (0..1020); w = RN16((1024 + h) * A + B) with A = 0x1EEE and
     B = 0xC931 as fp16, evaluated exactly and rounded to fp16 once (one fma).
"""

from __future__ import annotations

import numpy as np

from .numfmt import f16_bits_to_f64, f64_to_f16_bits

WIDTHS = (2, 3, 4, 5, 6, 8)
HASH_MUL = 0x9E3779
CB_SCALE_BITS = 0x1EEE  # fp16 0.00676727294921875, nearest fp16 to sqrt(3)/256
CB_BIAS_BITS = 0xC931  # fp16 -10.3828125, nearest fp16 to -1534 * CB_SCALE
TILE_VALUES = 256


def tile_words(bits: int) -> int:
    """uint32 words per 16 x 16 tile at `bits` bits per weight."""
    return 8 * bits


def trellis_bytes(bits: int, in_dim: int, out_dim: int) -> int:
    return in_dim * out_dim * bits // 8


# ---------------------------------------------------------------------------
# Two independent readers of a tile's states (R1, R2).


def tile_states_bitwise(words, bits: int) -> list[int]:
    """Reads one tile a bit at a time, straight from R1 and R2 (slow, for tiny cases)."""
    n = TILE_VALUES * bits
    words = [int(w) for w in words]
    assert len(words) == tile_words(bits)

    def bit(i: int) -> int:
        return (words[i >> 5] >> (i & 31)) & 1

    states = []
    for j in range(TILE_VALUES):
        s = 0
        for t in range(16):
            s |= bit((j * bits + t) % n) << t
        states.append(s)
    return states


def tile_states(words: np.ndarray, bits: int) -> np.ndarray:
    """Vectorized word/shift reader: words [..., 8*bits] uint32 -> states [..., 256] uint32.

    The window of value j starts at bit p = j*bits, inside word p >> 5 at offset
    p & 31; 16 bits never reach past the following word (wrapping to word 0 at
    the tile's end), so each state is a shift of a 64-bit word pair.
    """
    nw = tile_words(bits)
    words = np.asarray(words, dtype=np.uint32)
    assert words.shape[-1] == nw
    p = np.arange(TILE_VALUES, dtype=np.int64) * bits
    w0 = p >> 5
    w1 = (w0 + 1) % nw
    sh = (p & 31).astype(np.uint64)
    w64 = words.astype(np.uint64)
    pair = (w64[..., w1] << np.uint64(32)) | w64[..., w0]
    return ((pair >> sh) & np.uint64(0xFFFF)).astype(np.uint32)


# ---------------------------------------------------------------------------
# Codebook (R5).


def codebook_exact(states: np.ndarray) -> np.ndarray:
    """Exact value (1024 + h) * A + B before the fp16 rounding, as float64.

    (1024 + h) * A is an integer times 2^-18 below 2^22 * 2^-18 and B is a
    multiple of 2^-7, so the sum is exact in float64.
    """
    s = np.asarray(states, dtype=np.uint64)
    assert np.all(s < 65536)
    x = (s * np.uint64(HASH_MUL)) & np.uint64(0xFFFFFFFF)
    h = (
        (x & np.uint64(0xFF))
        + ((x >> np.uint64(8)) & np.uint64(0xFF))
        + ((x >> np.uint64(16)) & np.uint64(0xFF))
        + ((x >> np.uint64(24)) & np.uint64(0xFF))
    ).astype(np.float64)
    a = f16_bits_to_f64(np.uint16(CB_SCALE_BITS))
    b = f16_bits_to_f64(np.uint16(CB_BIAS_BITS))
    return (1024.0 + h) * a + b


def decode_states(states: np.ndarray) -> np.ndarray:
    """fp16 bits of the weights of the given 16-bit states (one rounding)."""
    return f64_to_f16_bits(codebook_exact(states))


# ---------------------------------------------------------------------------
# Whole matrices (R4).


def tile_grid(trellis: np.ndarray, bits: int, in_dim: int, out_dim: int) -> np.ndarray:
    """View the stream as [in_dim/16][out_dim/16][8*bits] words."""
    t = np.asarray(trellis, dtype=np.uint32)
    assert t.size == trellis_bytes(bits, in_dim, out_dim) // 4
    return t.reshape(in_dim // 16, out_dim // 16, tile_words(bits))


def unpack_columns(trellis: np.ndarray, bits: int, in_dim: int, out_dim: int,
                   tile_cols: np.ndarray | None = None, kt_chunk: int = 64) -> np.ndarray:
    """Decoded weights W[k][n] as fp16 bits for the tile columns `tile_cols`
    (default all), shape [in_dim][16 * len(tile_cols)]."""
    grid = tile_grid(trellis, bits, in_dim, out_dim)
    if tile_cols is None:
        tile_cols = np.arange(out_dim // 16)
    tile_cols = np.asarray(tile_cols, dtype=np.int64)
    nt = tile_cols.size
    out = np.empty((in_dim, 16 * nt), dtype=np.uint16)
    for k0 in range(0, in_dim // 16, kt_chunk):
        k1 = min(in_dim // 16, k0 + kt_chunk)
        sub = grid[k0:k1][:, tile_cols]  # [kc][nt][8b]
        w = decode_states(tile_states(sub, bits))  # [kc][nt][256], j = 16 n + k
        w = w.reshape(k1 - k0, nt, 16, 16)  # [kc][nt][n_local][k_local]
        out[16 * k0 : 16 * k1] = w.transpose(0, 3, 1, 2).reshape(16 * (k1 - k0), 16 * nt)
    return out


def unpack(trellis: np.ndarray, bits: int, in_dim: int, out_dim: int) -> np.ndarray:
    """All of W as fp16 bits [in_dim][out_dim]."""
    return unpack_columns(trellis, bits, in_dim, out_dim)


def strip_tile_cols(strips) -> np.ndarray:
    """Tile columns of the given 128-column strips."""
    strips = np.asarray(strips, dtype=np.int64).reshape(-1)
    return (8 * strips[:, None] + np.arange(8)[None, :]).reshape(-1)


# ---------------------------------------------------------------------------
# The strips layout (R21).


def strips_tile_offset(bits: int, in_dim: int, kt: int, nt: int) -> int:
    """Word offset of tile (kt, nt) in the strips layout."""
    strip, t = divmod(nt, 8)
    return ((strip * (in_dim // 16) + kt) * 8 + t) * tile_words(bits)


def _strips_tile_index(in_dim: int, out_dim: int) -> np.ndarray:
    """[in_dim/16][out_dim/16] -> tile index (in tiles) in the strips layout."""
    kt = np.arange(in_dim // 16, dtype=np.int64)[:, None]
    nt = np.arange(out_dim // 16, dtype=np.int64)[None, :]
    return ((nt // 8) * (in_dim // 16) + kt) * 8 + nt % 8


def tiles_to_strips(trellis: np.ndarray, bits: int, in_dim: int, out_dim: int) -> np.ndarray:
    """The stream in the strips layout: every tile copied to its strips-layout offset."""
    grid = tile_grid(trellis, bits, in_dim, out_dim)
    tw = tile_words(bits)
    out = np.empty(grid.size, dtype=np.uint32)
    out.reshape(-1, tw)[_strips_tile_index(in_dim, out_dim).reshape(-1)] = grid.reshape(-1, tw)
    return out


def strips_to_tiles(strips: np.ndarray, bits: int, in_dim: int, out_dim: int) -> np.ndarray:
    """The stream in the tile layout (R4) from a strips-layout stream."""
    tw = tile_words(bits)
    src = np.asarray(strips, dtype=np.uint32).reshape(-1, tw)
    assert src.size * 4 == trellis_bytes(bits, in_dim, out_dim)
    return src[_strips_tile_index(in_dim, out_dim).reshape(-1)].reshape(-1)
