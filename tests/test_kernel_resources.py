"""Every kernel's compiler resource record: no scratch, no spills, within gfx950's
registers and LDS (the page's "Kernel contract" records each kernel's VGPRs, SGPRs
and LDS and states that none uses private scratch; these are gfx950's records).

The build compiles every HIP source with the compiler's resource remarks and keeps
them beside the library; this test reads that record (rebuilding if a source is
newer) and fails on any kernel that uses scratch or spills. No GPU is needed.
"""

import re

import pytest

from trellis_quantized_linear_tf_amd import _build

WIDTHS = (2, 3, 4, 5, 6, 8)


@pytest.fixture(scope="module")
def record():
    return _build.load_resources()


def test_record_names_the_compiler_and_target(record):
    assert record["arch"] == "gfx950"
    assert "HIP version" in record["compiler"] and "clang" in record["compiler"]


def test_no_kernel_uses_scratch_or_spills(record):
    assert record["kernels"], "no kernels in the record"
    assert _build.resource_problems(record) == []


# The kernels the measured workloads run: these may not spill at all.
HOT = ["tf_exl3::linear_kernel<4, 8, 1>", "tf_exl3::linear_mfma_kernel<4, 8, 1>",
       "tf_exl3::linear_lds_kernel<4, 8, 16>", "tf_exl3::rot_in_kernel<1>", "tf_exl3::rot_in_kernel<2>"]


def test_hot_kernels_spill_no_register(record):
    for name in HOT:
        k = record["kernels"][name]
        assert k["sgpr_spill"] == 0 and k["vgpr_spill"] == 0, (name, k)


def test_sgpr_spills_stay_in_registers(record):
    """A few 2- and 4-row variants keep more scalar values than a wave has SGPRs and
    park some in VGPR lanes (v_writelane before the tile-row loop, v_readlane after
    it). That is register traffic, not memory: every such kernel has no scratch."""
    spills = _build.sgpr_lane_spills(record)
    for name in spills:
        assert record["kernels"][name]["scratch_bytes_per_lane"] == 0
    assert sum(spills.values()) <= 100, spills


def test_every_width_and_wave_count_is_built(record):
    names = set(record["kernels"])
    for bits in WIDTHS:
        for waves in (4, 8):
            for nr in (1, 2, 4):
                assert f"tf_exl3::linear_kernel<{bits}, {waves}, {nr}>" in names
            for nr in (8, 12, 16, 32):
                assert f"tf_exl3::linear_lds_kernel<{bits}, {waves}, {nr}>" in names
        for halves in (1, 2):
            assert f"tf_exl3::linear_mfma_kernel<{bits}, 4, {halves}>" in names
        assert f"tf_exl3::linear_mfma_kernel<{bits}, 8, 1>" in names
    for xdt in (0, 1, 2):
        assert f"tf_exl3::rot_in_kernel<{xdt}>" in names


def test_rot_in_is_small(record):
    """rot_in is one wave per 128-block in registers: no LDS (the page's record has
    none either) and few registers."""
    for name, k in record["kernels"].items():
        if name.startswith("tf_exl3::rot_in_kernel"):
            assert k["lds_bytes"] == 0 and k["vgprs"] <= 32, (name, k)


def test_checker_catches_planted_records():
    """The checker flags a record with scratch, a spill or too much LDS (planted on the
    host: a parsed remark text, not a kernel)."""
    text = "\n".join(f"x.hip:1:1: remark: {line} [-Rpass-analysis=kernel-resource-usage]" for line in [
        "Function Name: _Z1kv", "TotalSGPRs: 40", "VGPRs: 128", "AGPRs: 0", "ScratchSize [bytes/lane]: 16",
        "Dynamic Stack: False", "Occupancy [waves/SIMD]: 4", "SGPRs Spill: 0", "VGPRs Spill: 3",
        "LDS Size [bytes/block]: 200000",
    ])
    parsed = _build.parse_resource_remarks(text)
    assert parsed == {"_Z1kv": {"sgprs": 40, "vgprs": 128, "agprs": 0, "scratch_bytes_per_lane": 16,
                                "dynamic_stack": False, "occupancy_waves_per_simd": 4, "sgpr_spill": 0,
                                "vgpr_spill": 3, "lds_bytes": 200000}}
    problems = _build.resource_problems({"kernels": parsed})
    assert len(problems) == 3 and any(re.search("scratch", p) for p in problems)
    assert any(re.search("spills 3 VGPRs", p) for p in problems)
