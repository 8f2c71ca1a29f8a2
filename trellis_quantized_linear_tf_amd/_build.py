"""Builds libtf_exl3.so (gfx950) in the package directory with hipcc.

Every HIP source is compiled with:
  -ffp-contract=off   no implicit fma contraction: each fp32 add, subtract and
                      multiply of the rotations rounds on its own;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed fp32 instructions are generated.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB_NAME = "libtf_exl3.so"
ARCH = "gfx950"


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
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
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
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
