"""Builds libmoe.so for gfx950 from the HIP sources in csrc/ (hipcc, in-tree).

    python -m dispatch_expert_gemm_amd.build

Each source compiles to an object under _build/ in parallel, then one shared library is linked
next to this file. Every call rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.cpp", "route.hip", "layout.hip", "combine.hip", "ffn.hip", "placement.hip", "gate.hip",
           "shuffle.hip", "fused.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-munsafe-fp-atomics",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, defines=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [hipcc(), *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compiles every source and links `out`; `defines` are extra -D macros (tuning variants)."""
    build_dir = BUILD if not defines else os.path.join(BUILD, "_".join(defines))
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
