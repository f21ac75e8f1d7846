"""Build libmhc.so in-tree with hipcc for gfx950.

Each source under ``csrc/`` is compiled to an object in parallel, then linked
into ``mhc_hyper_connections_amd/libmhc.so``.  The benchmark's streaming-copy
reference (``csrc/bench_copy.hip``) goes into a library of its own,
``libmhc_bench.so``.  All device code is compiled with packed-fp32
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmhc.so")
BENCH_LIB = os.path.join(HERE, "libmhc_bench.so")
SOURCES = ["capi.cpp", "pre.hip", "pre8.hip", "pre_fused.hip", "post.hip", "amax.hip", "bwd.hip", "noalloc.hip"]
BENCH_SOURCES = ["bench_copy.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmhc")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out:
        print(out, file=sys.stderr)
    return obj


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source and link libmhc.so; returns its path."""
    if not force and os.path.exists(LIB):
        return LIB
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    for lib, names in ((LIB, SOURCES), (BENCH_LIB, BENCH_SOURCES)):
        tmp = lib + ".tmp"
        cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *(objs[n] for n in names)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
        os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(force=True, verbose=True)
