"""The seeded input generator: SplitMix64 against its published reference outputs,
determinism, slicing, and the storage formats of the inputs."""

import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # First five outputs for seed 1234567 of the reference implementation
    # (Vigna's splitmix64.c, the finalizer of Steele, Lea and Flood 2014).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [int(v) for v in synth.splitmix64(1234567, 5)] == want


def test_counter_based_slices():
    full = synth.splitmix64(42, 1000)
    assert np.array_equal(full[300:700], synth.splitmix64(42, 400, offset=300))
    w = synth.uniform_words(9, 2 ** 20 + 6, chunk=1 << 12)
    assert np.array_equal(w, synth.uniform_words(9, 2 ** 20 + 6))


def test_deterministic_and_seed_sensitive():
    a = synth.rows(5, 3, 256, "bf16")
    assert np.array_equal(a, synth.rows(5, 3, 256, "bf16"))
    assert not np.array_equal(a, synth.rows(6, 3, 256, "bf16"))


def test_normals_moments():
    v = synth.normals(3, 200_000, 0.5)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 0.5) < 0.01


def test_signs_are_pm_one():
    s = synth.signs(4, 10_000)
    assert set(np.unique(s)) == {synth.F16_ONE, synth.F16_MINUS_ONE}
    assert 0.45 < np.mean(s == synth.F16_ONE) < 0.55


def test_student_t_is_heavy_tailed():
    t = synth.student_t3(8, 100_000)
    assert np.max(np.abs(t)) > 40  # scale 4 times a t3 draw reaches far past a normal's range


def test_store_bf16_is_nearest():
    v = np.array([1.0, 1.00390625, 1.01171875, -3.0, 1e-40])
    bits = synth.store_bf16(v)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert list(back[:4]) == [1.0, 1.0, 1.015625, -3.0]


def test_symbol_packing_is_lsb_first():
    w = synth.symbols_to_words(np.array([1, 2, 3, 0] * 8, dtype=np.uint64), 4)
    assert w.tolist() == [0x03210321 & 0xFFFFFFFF, 0x03210321 & 0xFFFFFFFF, 0x03210321, 0x03210321]
