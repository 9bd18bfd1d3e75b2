"""Builds libkda_tree.so in-tree with hipcc for gfx950.

    python -m tree_packed_chunkwise_amd.build

Every HIP source is compiled for --offload-arch=gfx950 only, with the packed
FP32 instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops:
the compiler would otherwise form v_pk_* FP32 ops by itself).  The host-side
planner and C-ABI are plain C++17.  Objects go to _build/ (git-ignored); the
shared library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libkda_tree.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: Path) -> Path:
    obj = BUILD / (src.name + ".o")
    if src.suffix == ".hip":
        cmd = [HIPCC, *HIP_FLAGS, *COMMON, "-c", str(src), "-o", str(obj)]
    else:  # host C++ that includes the HIP runtime headers
        cmd = [HIPCC, *HIP_FLAGS, *COMMON, "-x", "hip", "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
