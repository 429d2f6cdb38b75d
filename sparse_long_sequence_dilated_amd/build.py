"""Build libdla.so in-tree for gfx950 (MI355X) with hipcc.

    python -m sparse_long_sequence_dilated_amd.build

Objects go to _build/ at the repository root; the library is written next to
this file so that it travels with the source tree.  The host planner
(dla_plan.cpp) has no HIP code and is compiled with g++; every .hip file is
compiled for gfx950 only, with packed fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC]

HOST_SOURCES = ["dla_plan.cpp"]
HIP_SOURCES = ["dla_api.hip", "dla_bwd_api.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip",
               "combine.hip", "attn_bwd_bf16.hip", "bwd_misc.hip", "dla_timing.hip",
               "shard.hip", "dla_layer.hip", "quant.hip"]
LINK_FLAGS = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".cpp"):
        _run([CXX, *CXX_FLAGS, "-c", path, "-o", obj])
    else:
        _run([HIPCC, *HIP_FLAGS, "-c", path, "-o", obj])
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libdla.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    sources = HOST_SOURCES + [s for s in HIP_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *LINK_FLAGS, "-o", tmp])
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
