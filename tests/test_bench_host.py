"""Host-side pins of bench.py's accounting: the algorithmic bytes and VALU work of one
launch on the LM head, the VALU peak, the traffic record's code hash, the one-GPU
refusal. No GPU is touched."""

from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]
K, N = 5120, 129280


def test_algorithmic_bytes_lm_head():
    # 4-bit stream K*N/2, z fp16, y fp32, svh fp16.
    ab = bench.algorithmic_bytes(1)
    assert ab["stream"] == K * N // 2 == 330_956_800
    assert ab["total"] == 330_956_800 + 2 * K + 4 * N + 2 * N == 331_742_720
    assert bench.algorithmic_bytes(16)["total"] == 330_956_800 + 16 * 2 * K + 16 * 4 * N + 2 * N


def test_valu_peak_from_unit_counts():
    # 256 CUs x 4 SIMDs x 16 lanes per cycle at 2.4 GHz.
    assert abs(bench.VALU_PEAK_TOPS - 39.3216) < 1e-9


def test_algorithmic_valu_ops():
    # Decode 92 instructions per 32 weights, one v_dot2 per 2 weights and row, 9 per output.
    assert bench.algorithmic_valu_ops("dot2", 1) == K * N * (92 / 32 + 0.5) + 9 * N
    assert bench.algorithmic_valu_ops("dot2", 1) == 2_235_121_920
    assert bench.algorithmic_valu_ops("dot2", 16) == K * N * (92 / 32 + 8) + 9 * 16 * N
    # The matrix-core engine sums on the MFMA units: decode and finish only.
    assert bench.algorithmic_valu_ops("mfma", 16) == K * N * 92 / 32 + 9 * 16 * N
    # More VALU work per stream byte than the chip supplies at HBM peak (the roofline is the VALU's).
    ops_per_byte = bench.algorithmic_valu_ops("dot2", 1) / bench.algorithmic_bytes(1)["stream"]
    assert ops_per_byte > bench.VALU_PEAK_TOPS * 1e12 / (bench.HBM_PEAK_GBPS * 1e9)


def test_code_hash_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* note */ }\n"
    b = "int f(int x) { return 2 * x; }"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text("int f(int x) { return 3 * x; }")
    files = {"exl3_device.hpp": "a", "exl3_strip.hpp": "b", "exl3_linear.hip": "c", "exl3_linear_cs.hip": "d"}
    h0 = bench.kernel_source_hash("dot2", read=files.__getitem__)
    files["exl3_linear.hip"] = "c // comment"
    assert bench.kernel_source_hash("dot2", read=files.__getitem__) == h0
    files["exl3_linear.hip"] = "c2"
    assert bench.kernel_source_hash("dot2", read=files.__getitem__) != h0


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_count_the_stream_once_per_pass():
    # 64 rows run four passes of 16, each streaming the weights once.
    s8 = K * N
    ab = bench.algorithmic_bytes(64, 8, K, N, 4)
    assert ab["stream"] == s8
    assert ab["total"] == 4 * s8 + 64 * 2 * K + 64 * 4 * N + 2 * N
    assert bench.passes(1) == bench.passes(16) == 1 and bench.passes(17) == 2
    # fp16 outputs (Engram) count two bytes each.
    assert bench.algorithmic_bytes(2, 3, 6144, 25600, 2)["total"] == 6144 * 25600 * 3 // 8 + 2 * 2 * 6144 \
        + 2 * 2 * 25600 + 2 * 25600
