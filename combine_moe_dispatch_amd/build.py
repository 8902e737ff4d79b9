"""Build libmoe_dispatch.so in-tree with hipcc for gfx950.

Usage: python -m combine_moe_dispatch_amd.build   (or call build()).
Each .hip source compiles to an object in parallel, then one link step.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_dispatch.so")
# streaming read/write/copy kernels for the benchmark's measured floor
CEILING_LIB = os.path.join(HERE, "libmoe_ceiling.so")
CEILING_SOURCE = "ceiling.hip"
# the same sources with phase stamps (-DMOE_PHASE_STAMPS): bench.py --timeline
TRACE_LIB = os.path.join(HERE, "libmoe_trace.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["capi.hip", "route_topk.hip", "dispatch.hip", "sources.hip", "combine.hip",
           "combine_partial.hip", "gemm_io.hip", "expert_scale.hip", "dispatch_static.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # IEEE fp32 semantics: correctly rounded division, no implicit contraction
    "-ffp-contract=off", "-fno-fast-math",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, trace: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + (".trace.o" if trace else ".o"))
    extra = ["-DMOE_PHASE_STAMPS"] if trace else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(src, False) for src in SOURCES + [CEILING_SOURCE]] + [(src, True) for src in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + 1], CEILING_LIB)
    _link(objs[n + 1:], TRACE_LIB)
    if verbose:
        print("built", LIB, CEILING_LIB, "and", TRACE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
