"""Compile liboscar.so (HIP for gfx950) in-tree.

Usage: python bit_rotated_kv_oscar_amd/build.py (by path: importing the
package would open the library that is about to be rebuilt).
Every source is compiled on every call; objects go to _build/, the library
to bit_rotated_kv_oscar_amd/liboscar.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liboscar.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: hipcc must not form v_pk_{add,mul,fma}_f32 from float code.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# Per-source extra flags.  The write kernels reduce over clipped, finite
# values: without the IEEE NaN mode the min / max row reductions fold their
# DPP lane moves into v_min / v_max (no quieting of each operand).
EXTRA = {"write.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-c", src, "-o", obj] + COMMON + EXTRA.get(os.path.basename(src), [])
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", "-c", src, "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if warn and os.environ.get("OSCAR_BUILD_VERBOSE"):
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, len(sources))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
