#!/usr/bin/env python3
"""Throughput of the EXL3 decode-row projection on one MI355X.

Headline workload: the LM head, 5120 -> 129,280 at 4 bits, fp16 input rows
~N(0, 0.5), +-1 suh/svh, fp32 logits. One step is rot_in on the rows followed by
the trellis linear: the whole path, on inputs already resident in HBM. The
headline value is one row per step (a decode token); further regions run 2, 4, 8
and 16 rows on both engines, and every workload of the test suite.

Cache protocol: each timed region rotates through copies of its weight stream
that together exceed ROTATE_BYTES (1.2 GB: more than the 256 MB Infinity Cache and
the L2s together), taking consecutive steps from copies written longest ago, so
no step reads a stream that an earlier step or the setup left in a cache.

Prints one JSON line (see the fields at the end of main()).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import subprocess
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
ROWS_PER_PASS = 16
ROTATE_BYTES = 1_200_000_000
WARMUP_S = 0.5
ROW_COUNTS = (1, 2, 4, 8, 16)
TRAFFIC_FILE = ROOT / "profiles" / "traffic_linear_lmhead_4bit.json"
RESOURCES_FILE = ROOT / "trellis_quantized_linear_tf_amd" / "libtf_exl3.resources.json"
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


def passes(rows: int) -> int:
    return max(1, math.ceil(rows / ROWS_PER_PASS))


def algorithmic_bytes(rows: int, bits: int = BITS, k: int = IN_DIM, n: int = OUT_DIM, y_size: int = 4) -> dict:
    """Bytes one launch of the linear must move: the stream once per pass of 16 rows,
    z, y and svh (suh belongs to rot_in)."""
    stream = k * n * bits // 8
    total = passes(rows) * stream + rows * k * 2 + rows * n * y_size + 2 * n
    return {"stream": stream, "total": total}


def algorithmic_valu_ops(engine: str, rows: int, k: int = IN_DIM, n: int = OUT_DIM) -> float:
    """VALU lane-instructions the linear needs per launch (4-bit decode): the decode of
    every weight once per pass, the v_dot2 sums of every row (on the matrix cores for the
    mfma engine), the finish."""
    weights = k * n
    dot = 0.0 if engine == "mfma" else DOT_OPS_PER_WEIGHT_ROW * rows
    return weights * (DECODE_OPS_PER_WEIGHT * passes(rows) + dot) + rows * n * FINISH_OPS_PER_OUTPUT


def load_traffic(engine: str, rows: int):
    """Counter-measured HBM bytes per launch, if taken on the engine's current kernel code."""
    if not TRAFFIC_FILE.exists():
        return None
    rec = json.loads(TRAFFIC_FILE.read_text())
    key = f"{engine}:{rows}"
    if rec.get("code_hash", {}).get(key) != kernel_source_hash(engine):
        return None
    return rec.get("per_launch_bytes", {}).get(key)


def rotating_copies(torch, dev, stream_np, min_bytes: int = ROTATE_BYTES):
    """Views of ceil(min_bytes / stream bytes) (at least 2) copies of the stream in one
    device buffer, in the order they were written."""
    import numpy as np

    words = stream_np.size
    nbytes = words * 4
    copies = max(2, math.ceil(min_bytes / nbytes))
    src = torch.from_numpy(stream_np.view(np.int32)).to(dev)
    buf = torch.empty((copies, words), dtype=torch.int32, device=dev)
    buf.copy_(src.unsqueeze(0).expand(copies, words))
    del src
    return [buf[i] for i in range(copies)]


def make_inputs(torch, dev, rows: int):
    import numpy as np

    import synth

    stream = synth.trellis_words(synth.seed_for(WORKLOAD_ID, synth.STREAM_TRELLIS), BITS, IN_DIM, OUT_DIM)
    x = synth.rows(synth.seed_for(WORKLOAD_ID, synth.STREAM_ROWS), rows, IN_DIM, "f16", 0.5)
    suh = synth.signs(synth.seed_for(WORKLOAD_ID, synth.STREAM_SUH), IN_DIM)
    svh = synth.signs(synth.seed_for(WORKLOAD_ID, synth.STREAM_SVH), OUT_DIM)
    trellis = rotating_copies(torch, dev, stream)
    xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.float16)
    suh_t = torch.from_numpy(suh.view(np.int16)).to(dev).view(torch.float16)
    svh_t = torch.from_numpy(svh.view(np.int16)).to(dev).view(torch.float16)
    return trellis, xt, suh_t, svh_t, (stream, x, suh, svh)


class Shape:
    """The linear's arguments that stay fixed in a timed region."""

    def __init__(self, bits=BITS, k=IN_DIM, n=OUT_DIM, waves=0, y_dtype=None):
        self.bits, self.k, self.n, self.waves, self.y_dtype = bits, k, n, waves, y_dtype


def time_steps(torch, tq, trellis, xt, suh_t, svh_t, steps: int, warmup: int, engine: str = "dot2",
               shape: Shape | None = None):
    """Warm up, then three timed regions of exactly `steps` steps each, on the stream the
    kernels are launched on:
      1. the steps alone, one event pair around the region: ms per step;
      2. the linear's launches alone, back to back on the same z (rot_in ran once before),
         one event pair around the region: the kernel's average launch duration (it
         includes the short gap between back-to-back kernels, not a dispatch latency);
      3. the steps with an event pair around every linear launch: the spread (p10, p50,
         p90) of single launches, whose pairs also span the dispatch latency.
    Step i reads stream copy (warmup + i) mod copies, so the timed steps start on the
    copies written longest ago. Returns (region-1 ms, region-2 ms per launch, region-3
    per-launch ms list, wall seconds of region 1, y)."""
    sh = shape or Shape()
    rows = xt.shape[0]
    z = torch.empty((rows, sh.k), dtype=torch.float16, device=xt.device)
    y = torch.empty((rows, sh.n), dtype=sh.y_dtype or torch.float32, device=xt.device)
    copies = len(trellis)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        t = trellis[i % copies]
        if engine == "fused":
            if ev:
                ev[0].record(stream)
            tq.project(xt, suh_t, t, svh_t, sh.bits, sh.n, y=y, waves=sh.waves)
        else:
            tq.rot_in(xt, suh_t, z)
            if ev:
                ev[0].record(stream)
            tq.linear(z, t, svh_t, sh.bits, sh.n, y=y, waves=sh.waves, engine=engine)
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
    base = i
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for j in range(steps):
        step(base + j)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)

    def launch(i):
        t = trellis[i % copies]
        if engine == "fused":
            tq.project(xt, suh_t, t, svh_t, sh.bits, sh.n, y=y, waves=sh.waves)
        else:
            tq.linear(z, t, svh_t, sh.bits, sh.n, y=y, waves=sh.waves, engine=engine)

    if engine != "fused":
        tq.rot_in(xt, suh_t, z)
    torch.cuda.synchronize()
    t0.record(stream)
    for j in range(steps):
        launch(base + steps + j)
    t1.record(stream)
    torch.cuda.synchronize()
    kernel_ms = t0.elapsed_time(t1) / steps

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for j in range(steps):
        step(base + 2 * steps + j, ev[j])
    torch.cuda.synchronize()
    lin_ms = [a.elapsed_time(b) for a, b in ev]
    return total_ms, kernel_ms, lin_ms, wall, y


def _percentiles(v):
    s = sorted(v)
    return [s[int(q * (len(s) - 1))] for q in (0.1, 0.5, 0.9)]


def cpu_baseline(host_inputs, rows: int) -> dict:
    """The oracle as it stands, timed on this host: its float64 linear threaded over
    strips on the host cores (the threaded reference, bit-identical to one thread),
    and rot_in's fp32 steps separately (one thread: a row is 40 blocks)."""
    import numpy as np

    from oracle import linear as lin
    from oracle import rotation as rot

    stream, x, suh, svh = host_inputs
    threads = lin.reference_threads()
    n_strips = OUT_DIM // 128
    # A bounded sample: 32 strips per thread (about 0.11 s of CPU work per strip, so
    # about 30 s of CPU work on 16 threads), spread evenly over the head's strips.
    sample = min(n_strips, 32 * threads)
    strips = np.linspace(0, n_strips - 1, sample).round().astype(np.int64)
    z = rot.rot_in(x[:rows], "f16", suh)
    t0 = time.perf_counter()
    lin.linear_f64(z, stream, BITS, IN_DIM, OUT_DIM, svh, strips=strips, threads=threads)
    dt = time.perf_counter() - t0
    reps, t1 = 0, time.perf_counter()
    while reps < 3 or time.perf_counter() - t1 < 0.5:
        rot.rot_in(x[:rows], "f16", suh)
        reps += 1
    rot_s = (time.perf_counter() - t1) / reps
    sample_stream_bytes = IN_DIM * 128 * sample * BITS // 8
    linear_s = dt * n_strips / sample
    return {
        "value": round(sample_stream_bytes / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} fp16 row(s): float64 linear over {sample} of {n_strips} strips, spread evenly "
                  f"({IN_DIM} x {128 * sample} weights) on {threads} threads, {dt:.1f} s of wall time, "
                  f"extrapolated to all strips; rot_in (fp32 steps, 1 thread) timed alone",
        "rows_per_s": round(rows / (linear_s + rot_s), 6),
        "linear_s_per_step": round(linear_s, 4),
        "rot_in": {"s_per_step": round(rot_s, 6), "rows_per_s": round(rows / rot_s, 2), "cores": 1},
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
    ("indexer wk 512->128", 1, 512, 128, (4,), (1,), "f16", "f32", 0, 1.0),
    ("Engram wkv 6144->25600", 2, 6144, 25600, (3, 4), (1, 2, 8, 16), "bf16", "f16", 4, 1.0),
    ("LM head 5120->129280", 3, 5120, 129280, (4,), (1, 16), "f16", "f32", 0, 0.5),
    ("width sweep 6144->25600", 4, 6144, 25600, (2, 3, 4, 5, 6, 8), (64,), "f16", "f32", 8, 1.0),
    ("stress LM head 8-bit", 5, 5120, 129280, (8,), (64,), "bf16", "f32", 0, 1.0),
]
_TDT = {"f32": 4, "f16": 2, "bf16": 2}


def time_configs(torch, tq, steps: int, warmup: int) -> list:
    """Every workload on both engines, and through the single launch where one pass holds
    its rows, under the bench's protocol (rotating stream copies over 1.2 GB, warm-up, us
    per step from a region of whole steps, the kernel's time from a region of its
    launches back to back; for the single launch that kernel is the whole step). Each
    also reports the step replayed from HIP graphs (time_graph_steps), which removes the
    per-launch overhead that dominates the latency-bound shapes."""
    import numpy as np

    import synth

    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    out = []
    for name, wid, k, n, widths, row_counts, xdt, ydt, waves, sigma in CONFIGS:
        suh = torch.from_numpy(synth.signs(synth.seed_for(wid, synth.STREAM_SUH), k).view(np.int16)).to(dev)
        svh = torch.from_numpy(synth.signs(synth.seed_for(wid, synth.STREAM_SVH), n).view(np.int16)).to(dev)
        suh, svh = suh.view(torch.float16), svh.view(torch.float16)
        for bits in widths:
            stream = synth.trellis_words(synth.seed_for(wid, synth.STREAM_TRELLIS) + 10 * bits, bits, k, n)
            copies = rotating_copies(torch, dev, stream)
            for rows in row_counts:
                x = synth.rows(synth.seed_for(wid, synth.STREAM_ROWS), rows, k, xdt, sigma)
                xt = torch.from_numpy(x.view(np.int16 if xdt != "f32" else np.float32)).to(dev)
                if xdt != "f32":
                    xt = xt.view(tdt[xdt])
                shape = Shape(bits, k, n, waves, tdt[ydt])
                ab = algorithmic_bytes(rows, bits, k, n, _TDT[ydt])
                rec = {"workload": name, "bits": bits, "rows": rows, "x": xdt, "y": ydt,
                       "waves": tq.linear_plan(bits, rows, k, n, waves)["waves"], "stream_copies": len(copies),
                       "bytes_per_launch": ab["total"]}
                # The single launch (rot_in fused into the v_dot2 linear) where one launch
                # holds all the rows: it saves a launch, which matters on latency-bound shapes.
                fused = rows <= tq.project_pass_rows(rows, k, n, waves)
                for engine in ("dot2", "mfma") + (("fused",) if fused else ()):
                    total_ms, kernel_ms, _, _, _ = time_steps(torch, tq, copies, xt, suh, svh, steps, warmup,
                                                              engine, shape)
                    us = total_ms / steps * 1e3
                    lin_us = kernel_ms * 1e3
                    rec[engine] = {
                        "us_per_step": round(us, 2),
                        "graph_us_per_step": round(time_graph_steps(torch, tq, copies, xt, suh, svh, engine, shape), 2),
                        "stream_gbps": round(passes(rows) * ab["stream"] / (us * 1e-6) / 1e9, 1),
                        "rows_per_s": round(rows / (us * 1e-6), 1),
                        "linear_us": round(lin_us, 2),
                        "hbm_frac": round(ab["total"] / (lin_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    }
                out.append(rec)
                print(json.dumps(rec), file=sys.stderr, flush=True)
            del copies
    return out


GRAPH_STEPS = 32  # steps per captured graph (each on its own stream copy)


def time_graph_steps(torch, tq, trellis, xt, suh_t, svh_t, engine: str, shape: Shape, replays: int = 20) -> float:
    """us per step when a caller replays its steps as HIP graphs: four graphs of
    GRAPH_STEPS steps each (rot_in + linear, or the single launch), step i of graph j on
    stream copy (j * GRAPH_STEPS + i) mod copies, captured once and replayed in turn; one
    event pair around `replays` replays."""
    sh = shape
    rows = xt.shape[0]
    z = torch.empty((rows, sh.k), dtype=torch.float16, device=xt.device)
    y = torch.empty((rows, sh.n), dtype=sh.y_dtype or torch.float32, device=xt.device)
    copies = len(trellis)

    def step(t):
        if engine == "fused":
            tq.project(xt, suh_t, t, svh_t, sh.bits, sh.n, y=y, waves=sh.waves)
        else:
            tq.rot_in(xt, suh_t, z)
            tq.linear(z, t, svh_t, sh.bits, sh.n, y=y, waves=sh.waves, engine=engine)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(trellis[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for j in range(4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(GRAPH_STEPS):
                step(trellis[(j * GRAPH_STEPS + i) % copies])
        graphs.append(g)
    for r in range(8):
        graphs[r % 4].replay()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for r in range(replays):
        graphs[r % 4].replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / (replays * GRAPH_STEPS) * 1e3
    del graphs
    return us


def _versions() -> dict:
    """hipcc and ROCm versions on this machine (the library was built with the compiler
    its resource record names)."""
    v = {}
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True, timeout=30)
        v["hipcc"] = "; ".join(l.strip() for l in r.stdout.splitlines()[:2])
    except (OSError, subprocess.SubprocessError):
        v["hipcc"] = None
    try:
        v["rocm"] = Path("/opt/rocm/.info/version").read_text().strip()
    except OSError:
        v["rocm"] = None
    return v


def kernel_resources(names) -> dict:
    """The compiler's record (registers, LDS, scratch, spills) of the named kernels."""
    if not RESOURCES_FILE.exists():
        return {"record": None}
    rec = json.loads(RESOURCES_FILE.read_text())
    keep = ("vgprs", "agprs", "sgprs", "lds_bytes", "scratch_bytes_per_lane", "sgpr_spill", "vgpr_spill",
            "occupancy_waves_per_simd")
    out = {"compiler": rec.get("compiler"),
           "all_kernels_scratch_free": all(k.get("scratch_bytes_per_lane", 0) == 0 for k in rec["kernels"].values())}
    for nm in names:
        k = rec["kernels"].get("tf_exl3::" + nm)
        if k is not None:
            out[nm] = {f: k[f] for f in keep if f in k}
    return out


def run_env(torch, kernels) -> dict:
    """The device and software the numbers come from."""
    props = torch.cuda.get_device_properties(0)
    return {
        "device": props.name,
        "arch": getattr(props, "gcnArchName", ""),
        "compute_units": props.multi_processor_count,
        "torch": torch.__version__,
        "hip_runtime": torch.version.hip,
        **_versions(),
        "kernel_resources": kernel_resources(kernels),
        "seeds": {"workload": WORKLOAD_ID, "rule": "1000 * workload + stream"},
    }


def region(torch, tq, trellis, xt, suh_t, svh_t, rows, steps, warmup, engine) -> dict:
    t, l_avg, l, _, _ = time_steps(torch, tq, trellis, xt[:rows].contiguous(), suh_t, svh_t, steps, warmup, engine)
    abr = algorithmic_bytes(rows)
    return {
        "ms_per_step": round(t / steps, 5),
        "value": round(abr["stream"] / (t / steps * 1e-3) / 1e9, 2),
        "rows_per_s": round(rows / (t / steps * 1e-3), 1),
        "kernel": kernel_name(engine, rows),
        "linear_ms": round(l_avg, 5),
        "single_launch_ms_p10_p50_p90": [round(v, 5) for v in _percentiles(l)],
        "hbm_gbps": round(abr["total"] / (l_avg * 1e-3) / 1e9, 2),
        "hbm_frac": round(abr["total"] / (l_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "valu_frac": round(algorithmic_valu_ops(engine, rows) / (l_avg * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
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
    ap.add_argument("--no-r16", action="store_true", help="skip the regions beyond the headline")
    ap.add_argument("--no-configs", action="store_true", help="skip the test suite's workloads")
    ap.add_argument("--calibrate-copy", action="store_true", help="run only a 1 GiB copy (counter scale)")
    ap.add_argument("--ingest-counters", metavar="DIR", help="write the traffic record from --pmc runs in DIR")
    ap.add_argument("--configs", action="store_true", help="time only the test suite's workloads")
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
    csteps = max(10, args.steps // 2)
    if args.configs:
        print(json.dumps({"configs": time_configs(torch, tq, csteps, args.warmup)}))
        return 0

    rows = args.rows
    trellis, xt, suh_t, svh_t, host = make_inputs(torch, dev, 16)
    engine = args.engine
    n_copies = len(trellis)
    head = [tq.repack_strips(t, BITS, IN_DIM, OUT_DIM) for t in trellis] if engine == "strips" else trellis
    total_ms, lin_avg_ms, lin_ms, wall, y = time_steps(torch, tq, head, xt[:rows].contiguous(), suh_t, svh_t,
                                                       args.steps, args.warmup, engine)
    head = None
    ms_per_step = total_ms / args.steps
    ab = algorithmic_bytes(rows)
    stream_gbps = passes(rows) * ab["stream"] / (ms_per_step * 1e-3) / 1e9
    achieved = ab["total"] / (lin_avg_ms * 1e-3) / 1e9
    valu_ops = algorithmic_valu_ops(engine, rows)
    valu_achieved = valu_ops / (lin_avg_ms * 1e-3) / 1e12
    traffic = load_traffic(engine, rows)

    extra = {}
    per_rows = {}
    kernels = {kernel_name(engine, rows)}
    if not args.no_r16:
        # Both engines at 1, 2, 4, 8 and 16 rows (the metric's range), the fused path at 1
        # and 2, the strips layout at 1 and 16, same inputs and protocol.
        table = {}
        for eng in ("dot2", "mfma"):
            for r in ROW_COUNTS:
                table[f"{eng}_rows{r}"] = region(torch, tq, trellis, xt, suh_t, svh_t, r, args.steps, args.warmup,
                                                 eng)
                kernels.add(kernel_name(eng, r))
        for r in (1, 2):
            table[f"fused_rows{r}"] = region(torch, tq, trellis, xt, suh_t, svh_t, r, args.steps, args.warmup,
                                             "fused")
            kernels.add(kernel_name("fused", r))
        strips = [tq.repack_strips(t, BITS, IN_DIM, OUT_DIM) for t in trellis]
        torch.cuda.synchronize()
        for r in (1, 16):
            table[f"strips_rows{r}"] = region(torch, tq, strips, xt, suh_t, svh_t, r, args.steps, args.warmup,
                                              "strips")
        del strips
        # The best engine at each row count: the roofline of the metric's whole range.
        for r in ROW_COUNTS:
            best = min(("dot2", "mfma"), key=lambda e: table[f"{e}_rows{r}"]["linear_ms"])
            t = table[f"{best}_rows{r}"]
            per_rows[str(r)] = {"engine": best, "kernel": "tf_exl3::" + t["kernel"], "kernel_ms": t["linear_ms"],
                                "achieved_gbps": t["hbm_gbps"], "frac": t["hbm_frac"], "valu_frac": t["valu_frac"],
                                "ms_per_step": t["ms_per_step"], "rows_per_s": t["rows_per_s"]}

        # The prompt path against the decode linear on a 128-row prompt (fewer steps: ~2 ms each).
        import numpy as np

        import synth

        xp = synth.rows(synth.seed_for(WORKLOAD_ID, synth.STREAM_ROWS), PROMPT_ROWS, IN_DIM, "f16", 0.5)
        xpt = torch.from_numpy(xp.view(np.int16)).to(dev).view(torch.float16)
        psteps = max(10, args.steps // 10)
        for eng in ("dot2", "prompt"):
            t, l_avg, _, _, _ = time_steps(torch, tq, trellis, xpt, suh_t, svh_t, psteps, args.warmup, eng)
            table[f"{eng}_rows{PROMPT_ROWS}"] = {
                "ms_per_step": round(t / psteps, 5),
                "rows_per_s": round(PROMPT_ROWS / (t / psteps * 1e-3), 1),
                "linear_ms": round(l_avg, 5),
                "steps": psteps,
            }
        extra["engines"] = table
    del trellis
    torch.cuda.empty_cache()
    if not args.no_configs:
        extra["configs"] = time_configs(torch, tq, csteps, args.warmup)

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
            "stream_copies": n_copies,
        },
        "rows_per_s": round(rows / (ms_per_step * 1e-3), 1),
        # The HBM roofline of the dominant kernel: algorithmic bytes per launch over its
        # average duration (HIP events on its stream) against 8 TB/s. The same launch's
        # VALU fraction stands beside it (the 1-row decode issues more VALU work per byte
        # than the chip supplies at its HBM rate, so the VALU is what binds it).
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "tf_exl3::" + kernel_name(engine, rows),
            "kernel_ms": round(lin_avg_ms, 5),
            "kernel_ms_timing": "events around the region of back-to-back launches of the kernel",
            "single_launch_ms_p10_p50_p90": [round(v, 5) for v in _percentiles(lin_ms)],
            "bytes_per_launch": ab["total"],
            "read_ceiling_gbps": round(ceiling, 2),
            "frac_of_read_ceiling": round(achieved / ceiling, 4),
            "valu": {
                "achieved": round(valu_achieved, 3),
                "peak": round(VALU_PEAK_TOPS, 3),
                "unit": "T VALU lane-instr/s",
                "frac": round(valu_achieved / VALU_PEAK_TOPS, 4),
                "ops_per_launch": int(valu_ops),
            },
            "per_rows": per_rows,
        },
        "cpu_baseline": cpu,
        "wall_s": round(wall, 4),
        "env": run_env(torch, sorted(kernels)),
        **extra,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
