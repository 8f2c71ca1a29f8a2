"""Builds libtf_exl3.so (gfx950) in the package directory with hipcc.

Every HIP source is compiled with:
  -ffp-contract=off   no implicit fma contraction: each fp32 add, subtract and
                      multiply of the rotations rounds on its own;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions are generated;
  -Rpass-analysis=kernel-resource-usage
                      the compiler reports each kernel's registers, LDS, scratch
                      and spills; the build writes them, with the compiler's
                      version, to libtf_exl3.resources.json beside the library.
"""

from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB_NAME = "libtf_exl3.so"
RESOURCES_NAME = "libtf_exl3.resources.json"
ARCH = "gfx950"
RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtf_exl3.so)")


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build(verbose: bool = False, jobs: int = 8) -> Path:
    """Compile each source to an object in parallel, then link the shared library."""
    cc = hipcc()
    obj_dir = PKG / "_build"
    obj_dir.mkdir(exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = obj_dir / (src.name + ".o")
        objs.append(obj)
        cmd = [cc, *common_flags(), "-c", str(src), "-o", str(obj)]
        if src.suffix == ".hip":
            cmd[1:1] = ["-x", "hip"]
            cmd.append(RESOURCE_REMARK)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    kernels: dict = {}
    for src, p in procs:
        out, _ = p.communicate()
        kernels.update(parse_resource_remarks(out))
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops" not in l and l.strip() and not _is_remark_line(l))
        if out and (verbose or p.returncode != 0):
            print(out, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src.name)
    if failed:
        raise RuntimeError(f"hipcc failed on: {', '.join(failed)}")
    lib = PKG / LIB_NAME
    tmp = PKG / (LIB_NAME + ".tmp")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    record = {"arch": ARCH, "compiler": compiler_version(cc), "kernels": dict(sorted(demangle(kernels).items()))}
    (PKG / RESOURCES_NAME).write_text(json.dumps(record, indent=1) + "\n")
    return lib


# ---------------------------------------------------------------------------
# Kernel resource records from the compiler's remarks.

_REMARK = re.compile(r"remark:\s+(.*?)\s*\[-Rpass-analysis=kernel-resource-usage\]")
_FIELDS = {
    "TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
    "Dynamic Stack": "dynamic_stack", "Occupancy [waves/SIMD]": "occupancy_waves_per_simd",
    "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes",
}


def _is_remark_line(line: str) -> bool:
    return "kernel-resource-usage" in line or bool(re.match(r"^\s*(\d+\s*\||\|)", line))


def parse_resource_remarks(text: str) -> dict:
    """{mangled kernel name: {field: value}} from -Rpass-analysis=kernel-resource-usage output."""
    out: dict = {}
    cur = None
    for m in _REMARK.finditer(text):
        body = m.group(1)
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
            continue
        key, _, val = body.partition(":")
        field = _FIELDS.get(key.strip())
        if cur is None or field is None:
            continue
        val = val.strip()
        out[cur][field] = (val == "True") if val in ("True", "False") else int(val)
    return out


def demangle(kernels: dict) -> dict:
    """Readable kernel names (llvm-cxxfilt from the ROCm toolchain; mangled names if it is missing)."""
    tool = next((c for c in ("/opt/rocm/llvm/bin/llvm-cxxfilt", shutil.which("llvm-cxxfilt") or "",
                             shutil.which("c++filt") or "") if c and Path(c).exists()), None)
    names = list(kernels)
    if tool is None or not names:
        return kernels
    res = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
    pretty = res.stdout.splitlines() if res.returncode == 0 else names
    if len(pretty) != len(names):
        return kernels
    return {p.split("(")[0].replace("void ", "", 1): dict(kernels[n], mangled=n) for p, n in zip(pretty, names)}


def compiler_version(cc: str) -> str:
    res = subprocess.run([cc, "--version"], capture_output=True, text=True)
    lines = [l.strip() for l in res.stdout.splitlines() if l.strip()]
    return "; ".join(lines[:2])


# gfx950: 512 vector registers per lane (VGPRs and AGPRs together), 160 KiB of LDS per CU.
MAX_REGS = 512
MAX_LDS = 160 * 1024


def resource_problems(record: dict) -> list[str]:
    """Kernels that use scratch memory, spill VGPRs, need a dynamic stack, or exceed the
    CU's limits. (An SGPR spill with no scratch goes to a VGPR lane: see sgpr_lane_spills.)"""
    bad = []
    for name, k in record["kernels"].items():
        if k.get("scratch_bytes_per_lane", 0) != 0:
            bad.append(f"{name}: {k['scratch_bytes_per_lane']} bytes of scratch per lane")
        if k.get("vgpr_spill", 0):
            bad.append(f"{name}: spills {k['vgpr_spill']} VGPRs")
        if k.get("dynamic_stack"):
            bad.append(f"{name}: dynamic stack")
        if k.get("vgprs", 0) + k.get("agprs", 0) > MAX_REGS:
            bad.append(f"{name}: {k['vgprs']} + {k['agprs']} vector registers")
        if k.get("lds_bytes", 0) > MAX_LDS:
            bad.append(f"{name}: {k['lds_bytes']} bytes of LDS")
    return bad


def sgpr_lane_spills(record: dict) -> dict:
    """{kernel: SGPRs spilled} for kernels that spill SGPRs without scratch (into VGPR lanes)."""
    return {n: k["sgpr_spill"] for n, k in record["kernels"].items()
            if k.get("sgpr_spill", 0) and k.get("scratch_bytes_per_lane", 0) == 0}


def load_resources(rebuild_if_stale: bool = True) -> dict:
    """The build's resource record; rebuilds first if it is missing or older than a source."""
    path = PKG / RESOURCES_NAME
    newest = max(p.stat().st_mtime for p in list(sources()) + list(CSRC.glob("*.hpp")) + [INCLUDE / "tf_exl3.h"])
    if rebuild_if_stale and (not path.exists() or path.stat().st_mtime < newest):
        build()
    return json.loads(path.read_text())


def resources_markdown(record: dict, hot=()) -> str:
    """Summary of the resource record: the named kernels in full, then every kernel
    family (template) with the range of each figure over its instantiations."""
    ks = record["kernels"]
    head = "| kernel | VGPRs | AGPRs | SGPRs | LDS bytes | scratch B/lane | SGPR/VGPR spills | waves/SIMD |"
    rows = [head, "|---|---|---|---|---|---|---|---|"]
    for name in hot:
        k = ks[name]
        rows.append(f"| `{name}` | {k['vgprs']} | {k['agprs']} | {k['sgprs']} | {k['lds_bytes']} | "
                    f"{k['scratch_bytes_per_lane']} | {k['sgpr_spill']}/{k['vgpr_spill']} | "
                    f"{k['occupancy_waves_per_simd']} |")
    fam: dict = {}
    for name, k in ks.items():
        fam.setdefault(name.split("<")[0], []).append(k)

    def rng(vals):
        lo, hi = min(vals), max(vals)
        return f"{lo}" if lo == hi else f"{lo}-{hi}"

    rows += ["", "| family | kernels | VGPRs | SGPRs | LDS bytes | max scratch | SGPR spills (sum) | VGPR spills |",
             "|---|---|---|---|---|---|---|---|"]
    for f, kk in sorted(fam.items()):
        rows.append(f"| `{f}` | {len(kk)} | {rng([k['vgprs'] for k in kk])} | {rng([k['sgprs'] for k in kk])} | "
                    f"{rng([k['lds_bytes'] for k in kk])} | {max(k['scratch_bytes_per_lane'] for k in kk)} | "
                    f"{sum(k['sgpr_spill'] for k in kk)} | {sum(k['vgpr_spill'] for k in kk)} |")
    return "\n".join(rows) + "\n"


HOT_KERNELS = ("tf_exl3::rot_in_kernel<1>", "tf_exl3::linear_kernel<4, 8, 1>", "tf_exl3::linear_lds_kernel<4, 8, 16>",
               "tf_exl3::linear_mfma_kernel<4, 8, 1>", "tf_exl3::linear_mfma_kernel<4, 4, 2>",
               "tf_exl3::linear_cs_kernel<4, 4, 1>", "tf_exl3::project_kernel<4, 8, 1>")


if __name__ == "__main__":
    if "--resources-md" in sys.argv:
        rec = json.loads((PKG / RESOURCES_NAME).read_text())
        print(f"Compiler: {rec['compiler']}; arch {rec['arch']}; {len(rec['kernels'])} kernels.\n")
        print(resources_markdown(rec, [h for h in HOT_KERNELS if h in rec["kernels"]]), end="")
    else:
        print(build(verbose="-v" in sys.argv))
