"""The C ABI on the host, with no GPU: the library loads, exports what the header
declares, plans launches like the page's planner, and refuses bad arguments before
any launch (fake pointers never reach the device)."""

import ctypes
import subprocess

import pytest

import trellis_quantized_linear_tf_amd as tq
from trellis_quantized_linear_tf_amd import _lib
from tests.test_golden import table


@pytest.fixture(scope="module")
def lib():
    if not _lib.LIB_PATH.exists():
        from trellis_quantized_linear_tf_amd._build import build

        build()
    return _lib.load()


def test_header_declares_the_expected_calls():
    names = _lib.header_functions()
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _lib.header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)], capture_output=True, text=True)
    if out.returncode == 0:
        exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
        assert set(_lib.header_functions()) <= exported


def test_status_strings(lib):
    for code in range(0, -10, -1):
        assert tq.status_string(code) != "unknown status"
    assert tq.status_string(-99) == "unknown status"


def test_trellis_bytes(lib):
    assert tq.trellis_bytes(4, 5120, 129280) == 330_956_800
    assert tq.trellis_bytes(8, 5120, 129280) == 661_913_600
    assert tq.trellis_bytes(7, 128, 128) == 0
    assert tq.trellis_bytes(4, 100, 128) == 0
    assert tq.trellis_bytes(8, 65536, 65536) == 0  # 4 GiB: refused


@pytest.mark.parametrize("row", table("wave_plan.txt"))
def test_wave_plan_matches_the_page(lib, row):
    out_dim, in_dim, waves = int(row[0]), int(row[1]), int(row[2])
    assert tq.linear_plan(4, 1, in_dim, out_dim)["waves"] == waves


def test_plan_fields(lib):
    p = tq.linear_plan(4, 16, 5120, 129280)
    assert p == {"width_index": 2, "waves": 8, "threads": 512, "grid_x": 1010, "passes": 1,
                 "rows_last_pass": 16, "rows_kernel": 16,
                 "lds_bytes": 8 * 16 * 128 * 4 + 8 * 32 * 16, "column_split": 0}
    p = tq.linear_plan(2, 64, 6144, 25600, waves=4)
    assert (p["waves"], p["passes"], p["rows_last_pass"]) == (4, 4, 16)
    p = tq.linear_plan(6, 17, 256, 256)
    assert (p["passes"], p["rows_last_pass"], p["rows_kernel"]) == (2, 1, 16)
    p = tq.linear_plan(3, 3, 256, 256)  # 2 strips x 4 waves: column-split, 8 waves a block
    assert (p["passes"], p["rows_kernel"], p["column_split"], p["threads"]) == (1, 4, 1, 512)
    assert p["lds_bytes"] == 4 * 4 * 128 * 4 + 8 * 8 * 16
    p = tq.linear_plan(3, 10, 256, 256)
    assert (p["passes"], p["rows_kernel"], p["lds_bytes"]) == (1, 12, 4 * 12 * 128 * 4 + 8 * 24 * 16)
    # Engram (200 strips at 4 waves: 800 waves) splits; the LM head (1010 x 8) does not,
    # nor does a 64-row width sweep's first launch (4 passes x 200 strips x 8 waves).
    assert tq.linear_plan(3, 1, 6144, 25600, waves=4)["column_split"] == 1
    assert tq.linear_plan(4, 1, 5120, 129280)["column_split"] == 0
    assert tq.linear_plan(4, 64, 6144, 25600, waves=8)["column_split"] == 0
    assert tq.linear_plan(4, 16, 6144, 25600, waves=8)["column_split"] == 1
    assert tq.linear_plan(5, 0, 128, 128)["passes"] == 0
    assert [tq.linear_plan(b, 1, 128, 128)["width_index"] for b in tq.WIDTHS] == [0, 1, 2, 3, 4, 5]


@pytest.mark.parametrize("args,code", [
    ((7, 1, 128, 128, 0), -1), ((1, 1, 128, 128, 0), -1),
    ((4, 1, 100, 128, 0), -2), ((4, 1, 128, 0, 0), -2), ((4, 1, 64, 128, 0), -2),
    ((4, -1, 128, 128, 0), -3), ((4, 1048561, 128, 128, 0), -3), ((4, 1, 128, 128, 6), -8),
    ((4, 1, 128, 128, 16), -8),
])
def test_plan_refusals(lib, args, code):
    p = _lib.Plan()
    assert lib.tf_exl3_linear_plan(*args, ctypes.byref(p)) == code
    assert lib.tf_exl3_linear_plan(4, 1, 128, 128, 0, None) == -5


def test_plan_accepts_the_largest_row_count(lib):
    p = _lib.Plan()
    assert lib.tf_exl3_linear_plan(4, 1048560, 128, 128, 0, ctypes.byref(p)) == 0
    assert p.passes == 65535


FAKE = 0x7F0000000000  # never dereferenced: every call below is refused on the host


@pytest.mark.parametrize("entry", ["tf_exl3_linear", "tf_exl3_linear_mfma", "tf_exl3_linear_prompt",
                                   "tf_exl3_linear_strips"])
def test_linear_refusals(lib, entry):
    f = getattr(lib, entry)
    ok = dict(bits=4, rows=2, k=256, n=256, z=FAKE, t=FAKE + 0x100000, s=FAKE + 0x200000, y=FAKE + 0x300000,
              dt=0, w=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["bits"], a["rows"], a["k"], a["n"], a["z"], a["t"], a["s"], a["y"], a["dt"], a["w"], None)

    assert call(bits=9) == -1
    assert call(k=300) == -2
    assert call(rows=-2) == -3
    assert call(rows=1048561) == -3  # more than 65535 passes of 16 rows
    assert call(dt=3) == -4
    assert call(z=None) == -5 and call(t=None) == -5 and call(s=None) == -5 and call(y=None) == -5
    assert call(z=FAKE + 8) == -6 and call(t=FAKE + 0x100004) == -6 and call(y=FAKE + 0x300002) == -6
    assert call(y=FAKE + 0x100) == -7  # y overlaps z
    assert call(y=FAKE + 0x100000 + 64) == -7  # y overlaps the trellis
    assert call(w=2) == -8
    assert call(rows=0, z=None, y=None) == 0  # nothing to do, nothing launched


def test_repack_refusals(lib):
    f = lib.tf_exl3_repack_strips
    n = tq.trellis_bytes(4, 256, 256)
    assert f(7, 256, 256, FAKE, FAKE + 0x100000, None) == -1
    assert f(4, 256, 200, FAKE, FAKE + 0x100000, None) == -2
    assert f(4, 256, 256, None, FAKE + 0x100000, None) == -5
    assert f(4, 256, 256, FAKE, FAKE + 0x100004, None) == -6
    assert f(4, 256, 256, FAKE, FAKE + n - 16, None) == -7  # overlap: not in place
    assert f(4, 256, 256, FAKE, FAKE, None) == -7


def test_rot_in_refusals(lib):
    f = lib.tf_exl3_rot_in
    assert f(FAKE, 3, FAKE + 0x10000, FAKE + 0x20000, 1, 128, None) == -4
    assert f(FAKE, 0, FAKE + 0x10000, FAKE + 0x20000, 1, 100, None) == -2
    assert f(FAKE, 0, FAKE + 0x10000, FAKE + 0x20000, -1, 128, None) == -3
    assert f(None, 0, FAKE + 0x10000, FAKE + 0x20000, 1, 128, None) == -5
    assert f(FAKE, 0, FAKE + 0x10000, FAKE + 0x20008, 1, 128, None) == -6
    assert f(FAKE + 2, 0, FAKE + 0x10000, FAKE + 0x20000, 1, 128, None) == -6  # fp32 rows need 4-byte alignment
    assert f(FAKE, 0, FAKE + 0x10000, FAKE + 0x100, 1, 128, None) == -7  # z overlaps x
    assert f(FAKE, 1, FAKE + 0x10000, FAKE + 0x20000, 0, 128, None) == 0
    # A grid beyond 2^31 workgroups of four 128-blocks is refused, not truncated.
    assert f(FAKE, 1, FAKE + 0x10000, FAKE + 0x20000, 2**31 - 1, 128 * 8, None) == -3


def test_debug_split_refusals(lib):
    for f, top in ((lib.tf_exl3_debug_linear_split, 1), (lib.tf_exl3_debug_linear_mfma_split, 1)):
        args = [4, 2, 256, 256, FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, 0, 4]
        assert f(*args, top + 1, None) == -2  # split outside the forms
        assert f(*args, -1, None) == -2
        assert f(4, 2, 256, 200, *args[4:], 0, None) == -2
        assert f(*args[:4], None, *args[5:], 0, None) == -5
    # The matrix-core column split exists at 4 waves only.
    for split in (1,):
        assert lib.tf_exl3_debug_linear_mfma_split(4, 2, 256, 256, FAKE, FAKE + 0x100000, FAKE + 0x200000,
                                                   FAKE + 0x300000, 0, 8, split, None) == -2


def test_debug_refusals(lib):
    assert lib.tf_exl3_debug_decode_states(FAKE, FAKE + 0x10, 64, None) == -7
    assert lib.tf_exl3_debug_decode_states(None, FAKE, 1, None) == -5
    assert lib.tf_exl3_debug_decode_states(FAKE, FAKE, -1, None) == -2
    assert lib.tf_exl3_debug_decode_tiles(7, 128, 128, FAKE, FAKE + 0x100000, None) == -1
    assert lib.tf_exl3_debug_decode_tiles(4, 128, 120, FAKE, FAKE + 0x100000, None) == -2


def test_header_is_c_and_a_c_program_links(lib, tmp_path):
    """include/tf_exl3.h compiles as C11 with warnings as errors, and a C program linked
    against the library gets the planner, sizes, strings and host refusals right."""
    import shutil

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = _lib.PKG.parent
    exe = tmp_path / "host_calls"
    build = subprocess.run(
        [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", f"-I{root / 'include'}",
         str(root / "tests" / "c_abi" / "host_calls.c"), "-o", str(exe),
         f"-L{_lib.LIB_PATH.parent}", "-ltf_exl3", f"-Wl,-rpath,{_lib.LIB_PATH.parent}"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0 and "c abi ok" in run.stdout, run.stderr
