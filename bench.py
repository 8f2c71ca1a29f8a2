#!/usr/bin/env python3
"""Throughput of the EXL3 decode-row projection on one MI355X.

Workload: the LM head, 5120 -> 129,280 at 4 bits, fp16 input rows ~N(0, 0.5),
+-1 suh/svh, fp32 logits. One step is rot_in on the rows followed by the trellis
linear: the whole path, on inputs already resident in HBM. The headline value is
one row per step (a decode token); a second timed region runs 16 rows per step.

The weight stream is 331 MB; steps alternate between two copies of it (662 MB,
more than the 256 MB Infinity Cache and the L2s together), so no step reads a
stream that the previous step left in a cache.

Prints one JSON line (see the fields at the end of main()).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "weight-stream GB/s and rows/s per MI355X (LM head 5120→129280, 4-bit, 1–16 rows)"
HBM_PEAK_GBPS = 8000.0
# VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes per cycle x 2.4 GHz. Every decode and
# dot instruction of the path (v_mul_u32_u24, v_sad_u8, v_alignbit_b32, v_pk_fma_f16,
# v_dot2) issues one wave64 instruction per 4 cycles per SIMD on gfx950.
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# VALU instructions per weight of the 4-bit decode (per tile row and lane: 32 window
# products, 16 + 16 byte sums, 16 packed fp16 fmas, 12 funnel shifts = 92 for 32
# weights), and per weight and row of the v_dot2 sums (one instruction per 2 k).
DECODE_OPS_PER_WEIGHT = 92 / 32
DOT_OPS_PER_WEIGHT_ROW = 0.5
FINISH_OPS_PER_OUTPUT = 9  # cross-wave sums, butterflies, scale, svh per output
BITS, IN_DIM, OUT_DIM = 4, 5120, 129280
WORKLOAD_ID = 3  # seeds: 1000 * workload + stream
CPU_SAMPLE_STRIPS = 384  # about 10-15 s of oracle work on one core
WARMUP_S = 0.5
TRAFFIC_FILE = ROOT / "profiles" / "traffic_linear_lmhead_4bit.json"
# The sources each engine's linear kernel is built from (the traffic record is keyed on them).
_COMMON = ["exl3_device.hpp", "exl3_strip.hpp"]
ENGINE_SOURCES = {
    "dot2": _COMMON + ["exl3_linear.hip", "exl3_linear_cs.hip"],
    "strips": _COMMON + ["exl3_linear.hip", "exl3_linear_cs.hip"],
    "prompt": _COMMON + ["exl3_linear.hip", "exl3_linear_cs.hip"],
    "mfma": _COMMON + ["exl3_linear_mfma.hip"],
    "fused": _COMMON + ["exl3_project.hip"],
}
PROMPT_ROWS = 128
# (engine, rows) regions whose HBM counters ingest_counters reads.
COUNTER_REGIONS = [("dot2", 1), ("dot2", 16), ("mfma", 1), ("mfma", 16), ("fused", 1), ("strips", 1)]


def _bucket(rows: int) -> int:
    return next(c for c in (1, 2, 4, 8, 12, 16) if rows <= c)


def kernel_name(engine: str, rows: int) -> str:
    """The kernel that does the linear's work for `rows` rows on the LM head (first pass)."""
    if engine == "mfma":
        return f"linear_mfma_kernel<{BITS}, 8, 1>"
    if engine == "fused":
        import trellis_quantized_linear_tf_amd as tq

        return f"project_kernel<{BITS}, 8, {tq.project_pass_rows(rows, IN_DIM, OUT_DIM)}>"
    if engine == "prompt" and rows >= 32:
        return f"linear_lds_kernel<{BITS}, 8, 32>"
    b = _bucket(min(rows, 16))
    return f"linear_kernel<{BITS}, 8, {b}>" if b <= 4 else f"linear_lds_kernel<{BITS}, 8, {b}>"
PROMPT_ROWS = 128


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace collapsed (the kernels' code only)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(engine: str, read=None) -> str:
    """Hash of an engine's kernel code (comments and layout ignored), keying its traffic record."""
    read = read or (lambda name: (ROOT / "trellis_quantized_linear_tf_amd" / "csrc" / name).read_text())
    h = hashlib.sha256()
    for name in ENGINE_SOURCES[engine]:
        h.update(code_text(read(name)).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(rows: int) -> dict:
    """Bytes the linear must move per launch: the stream, z, y, svh."""
    stream = IN_DIM * OUT_DIM * BITS // 8
    z = rows * IN_DIM * 2
    y = rows * OUT_DIM * 4
    svh = OUT_DIM * 2
    return {"stream": stream, "total": stream + z + y + svh}


def algorithmic_valu_ops(engine: str, rows: int) -> float:
    """VALU lane-instructions the linear needs per launch: the decode of every weight,
    the v_dot2 sums of every row (on the matrix cores for the mfma engine), the finish."""
    weights = IN_DIM * OUT_DIM
    dot = 0.0 if engine == "mfma" else DOT_OPS_PER_WEIGHT_ROW * rows
    return weights * (DECODE_OPS_PER_WEIGHT + dot) + rows * OUT_DIM * FINISH_OPS_PER_OUTPUT


def load_traffic(engine: str, rows: int):
    """Counter-measured HBM bytes per launch, if taken on the engine's current kernel code."""
    if not TRAFFIC_FILE.exists():
        return None
    rec = json.loads(TRAFFIC_FILE.read_text())
    key = f"{engine}:{rows}"
    if rec.get("code_hash", {}).get(key) != kernel_source_hash(engine):
        return None
    return rec.get("per_launch_bytes", {}).get(key)


def make_inputs(torch, dev, rows: int, copies: int):
    import numpy as np

    import synth

    stream = synth.trellis_words(synth.seed_for(WORKLOAD_ID, synth.STREAM_TRELLIS), BITS, IN_DIM, OUT_DIM)
    x = synth.rows(synth.seed_for(WORKLOAD_ID, synth.STREAM_ROWS), rows, IN_DIM, "f16", 0.5)
    suh = synth.signs(synth.seed_for(WORKLOAD_ID, synth.STREAM_SUH), IN_DIM)
    svh = synth.signs(synth.seed_for(WORKLOAD_ID, synth.STREAM_SVH), OUT_DIM)
    t_host = torch.from_numpy(stream.view(np.int32))
    trellis = [t_host.to(dev) for _ in range(copies)]
    xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.float16)
    suh_t = torch.from_numpy(suh.view(np.int16)).to(dev).view(torch.float16)
    svh_t = torch.from_numpy(svh.view(np.int16)).to(dev).view(torch.float16)
    return trellis, xt, suh_t, svh_t, (stream, x, suh, svh)


def time_steps(torch, tq, trellis, xt, suh_t, svh_t, steps: int, warmup: int, engine: str = "dot2"):
    """Warm up, then two timed regions of exactly `steps` steps each: the steps alone
    (events only before and after: ms per step), then the same steps with HIP events
    around every launch of the linear's kernel, on its stream (its duration: the
    events themselves cost the step a few microseconds, so they stay out of the first
    region)."""
    rows = xt.shape[0]
    z = torch.empty((rows, IN_DIM), dtype=torch.float16, device=xt.device)
    y = torch.empty((rows, OUT_DIM), dtype=torch.float32, device=xt.device)
    copies = len(trellis)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if engine == "fused":
            if ev:
                ev[0].record(stream)
            tq.project(xt, suh_t, trellis[i % copies], svh_t, BITS, OUT_DIM, y=y)
        else:
            tq.rot_in(xt, suh_t, z)
            if ev:
                ev[0].record(stream)
            tq.linear(z, trellis[i % copies], svh_t, BITS, OUT_DIM, y=y, engine=engine)
        if ev:
            ev[1].record(stream)

    # At least `warmup` steps and at least WARMUP_S seconds, so clocks settle first.
    t_start = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_start < WARMUP_S:
        step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    lin_ms = [a.elapsed_time(b) for a, b in ev]
    return total_ms, lin_ms, wall, y


def _percentiles(v):
    s = sorted(v)
    return [s[int(q * (len(s) - 1))] for q in (0.1, 0.5, 0.9)]


def cpu_baseline(host_inputs, rows: int) -> dict:
    """The oracle (rot_in fp32 steps + float64 linear) on a bounded sample of strips."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import linear as lin
    from oracle import rotation as rot

    stream, x, suh, svh = host_inputs
    strips = np.arange(CPU_SAMPLE_STRIPS)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        z = rot.rot_in(x[:rows], "f16", suh)
        lin.linear_f64(z, stream, BITS, IN_DIM, OUT_DIM, svh, strips=strips)
        dt = time.perf_counter() - t0
    sample_stream_bytes = IN_DIM * 128 * CPU_SAMPLE_STRIPS * BITS // 8
    return {
        "value": round(sample_stream_bytes / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{rows} row, {CPU_SAMPLE_STRIPS} of 1010 strips ({IN_DIM} x {128 * CPU_SAMPLE_STRIPS} weights), "
                  f"rot_in + float64 linear, {dt:.1f} s",
        "rows_per_s": round(rows * CPU_SAMPLE_STRIPS / 1010 / dt, 6),
    }


COPY_BYTES = 1 << 30


def calibrate_copy(torch, tq, dev, steps: int) -> None:
    """The library's plain copy kernel on 1 GiB (for scaling the HBM byte counters)."""
    a = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    for _ in range(steps):
        tq.calib_copy(a, b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "launches": steps}))


def read_ceiling(torch, tq, dev, launches: int = 20) -> float:
    """GB/s of the library's read-only stream kernel over 1 GiB buffers (two, alternating)."""
    bufs = [torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev) for _ in range(2)]
    out = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    for i in range(3):
        tq.calib_stream_read(bufs[i % 2], out)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(launches):
        tq.calib_stream_read(bufs[i % 2], out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / launches
    del bufs
    return COPY_BYTES / (ms * 1e-3) / 1e9


def _counter_means(directory: Path, kernel_substr: str) -> dict:
    """Mean per dispatch of each counter for kernels whose name contains kernel_substr."""
    import csv
    import glob

    files = glob.glob(str(directory / "**" / "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    vals: dict = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if kernel_substr in row["Kernel_Name"]:
                vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def ingest_counters(base: Path) -> dict:
    """Build the traffic record from rocprofv3 --pmc runs under `base`: copy_fetch/, copy_write/
    (bench.py --calibrate-copy) and {engine}_r{R}_fetch/, {engine}_r{R}_write/ (bench.py --engine E --rows R)."""
    copy_fetch = _counter_means(base / "copy_fetch", "copy_kernel")["FETCH_SIZE"]
    copy_write = _counter_means(base / "copy_write", "copy_kernel")["WRITE_SIZE"]
    f_read = COPY_BYTES / (copy_fetch * 1024)
    f_write = COPY_BYTES / (copy_write * 1024)
    per = {}
    raw = {}
    for engine, rows in COUNTER_REGIONS:
        d_f, d_w = base / f"{engine}_r{rows}_fetch", base / f"{engine}_r{rows}_write"
        if d_f.exists():
            name = kernel_name(engine, rows)
            fetch = _counter_means(d_f, name)["FETCH_SIZE"]
            write = _counter_means(d_w, name)["WRITE_SIZE"]
            raw[f"{engine}:{rows}"] = {"FETCH_SIZE": fetch, "WRITE_SIZE": write}
            per[f"{engine}:{rows}"] = int(round(fetch * 1024 * f_read + write * 1024 * f_write))
    rec = {
        "code_hash": {k: kernel_source_hash(k.split(":")[0]) for k in per},
        "copy_kib_per_launch": {"FETCH_SIZE": copy_fetch, "WRITE_SIZE": copy_write},
        "scale": {"read": f_read, "write": f_write},
        "linear_kib_per_launch": raw,
        "per_launch_bytes": per,
        "algorithmic_bytes": {k: algorithmic_bytes(int(k.split(":")[1]))["total"] for k in per},
    }
    TRAFFIC_FILE.parent.mkdir(exist_ok=True)
    TRAFFIC_FILE.write_text(json.dumps(rec, indent=1) + "\n")
    return rec


# The test suite's workloads (shape, widths, rows, input and output types, waves).
CONFIGS = [
    ("indexer wk 512->128", 1, 512, 128, (4,), (1,), "f16", "f32", 0),
    ("Engram wkv 6144->25600", 2, 6144, 25600, (3, 4), (1, 2, 8, 16), "bf16", "f16", 4),
    ("LM head 5120->129280", 3, 5120, 129280, (4,), (1, 16), "f16", "f32", 0),
    ("width sweep 6144->25600", 4, 6144, 25600, (2, 3, 4, 5, 6, 8), (64,), "f16", "f32", 8),
    ("stress LM head 8-bit", 5, 5120, 129280, (8,), (64,), "bf16", "f32", 0),
]


def time_configs(torch, tq, steps: int) -> list:
    """Step time (rot_in + linear) of every workload, both engines, HIP events around
    the steps only, median of five blocks (one stream copy: these shapes' streams are not all larger than the
    Infinity Cache, so the small ones may run from it)."""
    import numpy as np

    import synth

    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    out = []
    for name, wid, k, n, widths, row_counts, xdt, ydt, waves in CONFIGS:
        suh = torch.from_numpy(synth.signs(synth.seed_for(wid, synth.STREAM_SUH), k).view(np.int16)).to(dev)
        svh = torch.from_numpy(synth.signs(synth.seed_for(wid, synth.STREAM_SVH), n).view(np.int16)).to(dev)
        for bits in widths:
            stream = synth.trellis_words(synth.seed_for(wid, synth.STREAM_TRELLIS), bits, k, n)
            tt = torch.from_numpy(stream.view(np.int32)).to(dev)
            for rows in row_counts:
                x = synth.rows(synth.seed_for(wid, synth.STREAM_ROWS), rows, k, xdt, 1.0)
                xt = torch.from_numpy(x.view(np.int16 if xdt != "f32" else np.float32)).to(dev)
                if xdt != "f32":
                    xt = xt.view(tdt[xdt])
                z = torch.empty((rows, k), dtype=torch.float16, device=dev)
                y = torch.empty((rows, n), dtype=tdt[ydt], device=dev)
                rec = {"workload": name, "bits": bits, "rows": rows, "x": xdt, "y": ydt,
                       "waves": tq.linear_plan(bits, rows, k, n, waves)["waves"]}
                for engine in ("dot2", "mfma"):
                    def step():
                        tq.rot_in(xt, suh, z)
                        tq.linear(z, tt, svh, bits, n, y=y, waves=waves, engine=engine)

                    t_start = time.perf_counter()
                    while time.perf_counter() - t_start < 0.2:
                        step()
                    torch.cuda.synchronize()
                    # The median of five blocks of `steps` steps: one block that meets a
                    # clock or power transient does not set the figure.
                    blocks = []
                    for _ in range(5):
                        a = torch.cuda.Event(enable_timing=True)
                        b = torch.cuda.Event(enable_timing=True)
                        a.record()
                        for _ in range(steps):
                            step()
                        b.record()
                        torch.cuda.synchronize()
                        blocks.append(a.elapsed_time(b) / steps * 1e3)
                    us = sorted(blocks)[2]
                    rec[f"{engine}_us"] = round(us, 2)
                    rec[f"{engine}_stream_gbps"] = round(k * n * bits / 8 / (us * 1e-6) / 1e9, 1)
                    rec[f"{engine}_rows_per_s"] = round(rows / (us * 1e-6), 1)
                out.append(rec)
                print(json.dumps(rec), file=sys.stderr, flush=True)
    return out


def run_env(torch) -> dict:
    """The device and software the numbers come from."""
    props = torch.cuda.get_device_properties(0)
    return {
        "device": props.name,
        "arch": getattr(props, "gcnArchName", ""),
        "compute_units": props.multi_processor_count,
        "torch": torch.__version__,
        "hip": torch.version.hip,
        "seeds": {"workload": WORKLOAD_ID, "rule": "1000 * workload + stream"},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rows", type=int, default=1, help="rows of the headline region")
    ap.add_argument("--engine", choices=["dot2", "mfma", "fused", "prompt", "strips"], default="dot2",
                    help="headline path: rot_in + v_dot2 linear, rot_in + matrix-core linear, the "
                         "single-launch projection (rot_in fused into the v_dot2 linear), or rot_in + the "
                         "prompt path (32-row passes, bit-equal to the v_dot2 linear), or rot_in + the v_dot2 "
                         "linear on the strips layout")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-r16", action="store_true", help="skip the 16-row region")
    ap.add_argument("--calibrate-copy", action="store_true", help="run only a 1 GiB copy (counter scale)")
    ap.add_argument("--ingest-counters", metavar="DIR", help="write the traffic record from --pmc runs in DIR")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload of the test suite (both engines) and print one JSON line")
    args = ap.parse_args()

    if args.ingest_counters:
        print(json.dumps(ingest_counters(Path(args.ingest_counters))))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the projection shards by "
              "output columns with no exchange, so N GPUs each run this kernel on N-th of the strips).",
              file=sys.stderr)
        return 2

    import torch

    import trellis_quantized_linear_tf_amd as tq
    from trellis_quantized_linear_tf_amd import _lib

    if not _lib.LIB_PATH.exists():
        from trellis_quantized_linear_tf_amd._build import build

        build()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(torch, tq, dev, args.steps)
        return 0
    if args.configs:
        print(json.dumps({"configs": time_configs(torch, tq, max(10, args.steps // 4))}))
        return 0

    rows = args.rows
    trellis, xt, suh_t, svh_t, host = make_inputs(torch, dev, 16, copies=2)
    engine = args.engine
    head = [tq.repack_strips(t, BITS, IN_DIM, OUT_DIM) for t in trellis] if engine == "strips" else trellis
    total_ms, lin_ms, wall, y = time_steps(torch, tq, head, xt[:rows].contiguous(), suh_t, svh_t,
                                           args.steps, args.warmup, engine)
    del head
    ms_per_step = total_ms / args.steps
    lin_avg_ms = sum(lin_ms) / len(lin_ms)
    ab = algorithmic_bytes(rows)
    stream_gbps = ab["stream"] / (ms_per_step * 1e-3) / 1e9
    achieved = ab["total"] / (lin_avg_ms * 1e-3) / 1e9
    valu_ops = algorithmic_valu_ops(engine, rows)
    valu_achieved = valu_ops / (lin_avg_ms * 1e-3) / 1e12
    traffic = load_traffic(engine, rows)

    extra = {}
    if not args.no_r16:
        # Both engines at 1, 2, 4, 8 and 16 rows (the metric's range), and the fused path at 1
        # and 2, same inputs and protocol (the headline is one of them).
        table = {}
        for eng in ("dot2", "mfma", "fused"):
            for r in ((1, 2) if eng == "fused" else (1, 2, 4, 8, 16)):
                t, l, _, _ = time_steps(torch, tq, trellis, xt[:r].contiguous(), suh_t, svh_t, args.steps,
                                        args.warmup, eng)
                abr = algorithmic_bytes(r)
                l_avg = sum(l) / len(l)
                table[f"{eng}_rows{r}"] = {
                    "ms_per_step": round(t / args.steps, 5),
                    "value": round(abr["stream"] / (t / args.steps * 1e-3) / 1e9, 2),
                    "rows_per_s": round(r / (t / args.steps * 1e-3), 1),
                    "linear_ms": round(l_avg, 5),
                    "linear_ms_p10_p50_p90": [round(v, 5) for v in _percentiles(l)],
                    "hbm_frac": round(abr["total"] / (l_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "valu_frac": round(algorithmic_valu_ops(eng, r) / (l_avg * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                }
        # The strips layout (each strip one contiguous stream), same stream repacked.
        strips = [tq.repack_strips(t, BITS, IN_DIM, OUT_DIM) for t in trellis]
        torch.cuda.synchronize()
        for r in (1, 16):
            t, l, _, _ = time_steps(torch, tq, strips, xt[:r].contiguous(), suh_t, svh_t, args.steps,
                                    args.warmup, "strips")
            abr = algorithmic_bytes(r)
            l_avg = sum(l) / len(l)
            table[f"strips_rows{r}"] = {
                "ms_per_step": round(t / args.steps, 5),
                "value": round(abr["stream"] / (t / args.steps * 1e-3) / 1e9, 2),
                "rows_per_s": round(r / (t / args.steps * 1e-3), 1),
                "linear_ms": round(l_avg, 5),
                "linear_ms_p10_p50_p90": [round(v, 5) for v in _percentiles(l)],
                "hbm_frac": round(abr["total"] / (l_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "valu_frac": round(algorithmic_valu_ops("strips", r) / (l_avg * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
            }
        del strips

        # The prompt path against the decode linear on a 128-row prompt (fewer steps: ~2 ms each).
        import numpy as np

        import synth

        xp = synth.rows(synth.seed_for(WORKLOAD_ID, synth.STREAM_ROWS), PROMPT_ROWS, IN_DIM, "f16", 0.5)
        xpt = torch.from_numpy(xp.view(np.int16)).to(dev).view(torch.float16)
        psteps = max(10, args.steps // 10)
        for eng in ("dot2", "prompt"):
            t, l, _, _ = time_steps(torch, tq, trellis, xpt, suh_t, svh_t, psteps, args.warmup, eng)
            table[f"{eng}_rows{PROMPT_ROWS}"] = {
                "ms_per_step": round(t / psteps, 5),
                "rows_per_s": round(PROMPT_ROWS / (t / psteps * 1e-3), 1),
                "linear_ms": round(sum(l) / len(l), 5),
                "steps": psteps,
            }
        extra["engines"] = table

    ceiling = read_ceiling(torch, tq, dev)
    cpu = None if args.no_cpu else cpu_baseline(host, rows)

    out = {
        "metric": METRIC,
        "value": round(stream_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"LM head {IN_DIM}->{OUT_DIM}, {BITS}-bit trellis, {rows} fp16 row(s) ~N(0,0.5), "
                        "+-1 suh/svh, fp32 out; step = rot_in + linear",
            "in_dim": IN_DIM, "out_dim": OUT_DIM, "bits": BITS, "rows": rows,
            "waves": tq.linear_plan(BITS, rows, IN_DIM, OUT_DIM)["waves"],
            "engine": engine,
            "stream_copies": len(trellis),
        },
        "rows_per_s": round(rows / (ms_per_step * 1e-3), 1),
        # The linear issues more VALU work per byte than the chip supplies at its HBM
        # rate (the same kernel reading an L2-resident stream takes as many cycles), so
        # its roofline is the VALU's; the HBM side stands next to it.
        "roofline": {
            "bound": "alu",
            "achieved": round(valu_achieved, 3),
            "peak": round(VALU_PEAK_TOPS, 3),
            "unit": "T VALU lane-instr/s",
            "frac": round(valu_achieved / VALU_PEAK_TOPS, 4),
            "traffic": traffic,
            "kernel": "tf_exl3::" + kernel_name(engine, rows),
            "kernel_ms": round(lin_avg_ms, 5),
            "kernel_ms_p10_p50_p90": [round(v, 5) for v in _percentiles(lin_ms)],
            "ops_per_launch": int(valu_ops),
            "hbm": {
                "achieved": round(achieved, 2),
                "peak": HBM_PEAK_GBPS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "bytes_per_launch": ab["total"],
                "read_ceiling": round(ceiling, 2),
                "frac_of_read_ceiling": round(achieved / ceiling, 4),
            },
        },
        "cpu_baseline": cpu,
        "wall_s": round(wall, 4),
        "env": run_env(torch),
        **extra,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
