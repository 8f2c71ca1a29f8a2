"""Facts the pages print, held against the oracle and the format (fixtures in tests/golden/)."""

from pathlib import Path

import numpy as np
import pytest

import synth
from oracle import numfmt as nf
from oracle import trellis as tr

GOLDEN = Path(__file__).parent / "golden"


def table(name):
    rows = []
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(line.split())
    return rows


def facts():
    return {k: int(v) for k, v, *_ in table("exactness_facts.txt")}


def test_lds_records_imply_32_bits_bytes_per_tile():
    rows = table("lds_records_gfx1151.txt")
    assert len(rows) == 12
    for name, k, waves, lds in rows:
        bits = int(k) // 2
        assert bits in tr.WIDTHS
        tile_bytes = int(lds) // (8 * int(waves))
        assert tile_bytes * 8 * int(waves) == int(lds)
        assert tile_bytes == tr.trellis_bytes(bits, 16, 16) == 4 * tr.tile_words(bits)


def test_wave_plan_shapes_are_multiples_of_the_block():
    for out_dim, in_dim, waves, *_ in table("wave_plan.txt"):
        assert int(out_dim) % 128 == 0 and int(in_dim) % 128 == 0
        assert int(waves) == (8 if int(out_dim) >= 8192 else 4)


def test_exact_gate_arithmetic_for_this_codebook():
    f = facts()
    w1 = nf.f16_bits_to_f64(tr.decode_states(np.array([0xFFFF]))[0])
    term = f["linear_gate_input"] * w1
    assert term == int(term)
    total = f["linear_gate_k"] * int(term)
    assert total < f["fp32_exact_integer_limit"]
    assert total > f["fp16_max_finite"]


def test_rot_in_rounding_count_recipe():
    f = facts()
    blocks_per_dtype = (4 * 6144 + 16 * 5120 + 32 * 512 + 60 * 128) // f["rotation_block"]
    assert 3 * blocks_per_dtype * f["rotation_block"] == f["rot_in_roundings"]


def test_rot_in_gate_inputs_keep_fp32_exact():
    f = facts()
    assert f["rotation_block"] * f["rot_in_gate_input_max"] < f["fp32_exact_integer_limit"]
