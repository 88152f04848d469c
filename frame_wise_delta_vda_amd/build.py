"""Ahead-of-time build of libvda.so (gfx950) with hipcc.

Usage: python -m frame_wise_delta_vda_amd.build  [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libvda.so")
SOURCES = ["vda_api.cpp", "stats.hip", "scan.hip", "readout.hip", "bwd.hip", "noalloc.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops (v_pk_fma_f32 and friends) are switched off for all device
# code; the compiler otherwise forms them from plain float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source into libvda.so next to this file; returns its path.  The sources
    compile in parallel (one hipcc process each), then link."""
    from concurrent.futures import ThreadPoolExecutor

    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, src + ".o")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
               "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
            cmd += DEVICE_FLAGS
        cmd += list(extra)
        jobs.append((cmd, obj))

    def compile_one(job):
        cmd, _ = job
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(compile_one, jobs))
    objs = [obj for _, obj in jobs]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv,
          extra=[a for a in sys.argv[1:] if a != "--verbose"])
