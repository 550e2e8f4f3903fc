"""Build the HIP library libkdtopk.so in-tree for gfx950.

Usage: python chunked_top_kl_amd/build.py   (or call build_library()). Run it as
a file, not as a module of the package: importing the package loads the
library that this script rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkdtopk.so")

SOURCES = ["kd_api.hip", "kd_sweep.hip", "kd_gemm.hip", "kd_prepass.hip", "kd_select.hip",
           "kd_teacher.hip", "kd_signals.hip", "kd_sample.hip", "kd_compare.hip"]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# The fp64 band refinement keeps its MFMA accumulators in VGPRs: with the
# default form the compiler copies them between AGPRs and VGPRs on every step
# of its loop. The selection kernels are the file's only MFMA users.
FILE_FLAGS = {"kd_select.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source and link libkdtopk.so next to this file. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([hipcc, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
