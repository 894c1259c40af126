"""Builds librglru.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m gated_linear_recurrence_amd.build

Every call recompiles. hipcc cross-compiles for gfx950 on a machine without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "librglru.so"
ARCH = "gfx950"

SOURCES = ["rglru_scan.hip", "rglru_proj.hip", "delta_rule.hip", "delta_chunk.hip", "delta_bwd.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed-FP32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librglru)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"librglru build failed:\n{msg}")
    if verbose and msg.strip():
        print(msg)


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc(), *compile_flags, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
