"""Build libuq.so in-tree: HIP kernels for gfx950 plus the host packer.

    python gemm_group_wise_amd/build.py        # or __graft_entry__.build()

The host packer is plain C++ (g++, -ffp-contract=off) so its fp32/fp64
arithmetic is one IEEE operation per step; the kernels and the C ABI are
compiled by hipcc for gfx950 only.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libuq.so")

ARCH = "gfx950"
HIP_SOURCES = ["uq_api.hip", "gemv.hip", "gemv_int2.hip", "gemv_int4.hip", "gemv_int8.hip",
               "gemv_nf4.hip", "gemm.hip", "dequant.hip", "rmsnorm_rope.hip", "gemv_a8.hip", "probe.hip"]
CXX_SOURCES = ["uq_pack.cpp", "uq_gguf.cpp", "rope_table.cpp", "uq_check.cpp", "uq_host_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 (v_pk_*_f32) instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
             "-fno-fast-math", "-pthread", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libuq.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([CXX, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp])
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
