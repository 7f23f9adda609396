"""Builds libpagedkv.so in-tree: HIP kernels for gfx950 with hipcc, host pool with g++.

Usage: python paged_kv_cache_404_amd/build.py [--verbose]   (or __graft_entry__.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

HIP_SOURCES = ["append.hip", "check.hip", "decode.hip", "decode_group.hip", "fp8.hip", "mixed.hip", "mixed_fp8.hip",
               "prefill.hip", "prefill_fp8.hip", "probe.hip"]
HOST_SOURCES = ["pool.cpp", "status.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are switched off for every device compile.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({' '.join(cmd)}):\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    gxx = shutil.which("g++") or "g++"
    for src in HOST_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append([gxx, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(OBJDIR, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
