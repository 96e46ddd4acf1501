"""Builds libfp8q.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Usage:  python -m fp8_fine_grained_quant_amd.build   (or build_library())

Every source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled on the device (-Xclang -target-feature -Xclang
-packed-fp32-ops; the host pass warns that it does not know the feature) and
without fast-math, so FP32 division stays correctly rounded and denormals are
kept -- the quantizer's scales are required to be bit-exact.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8q.so")
SOURCES = ["fp8q_api.hip", "quant_kernels.hip", "gemm_kernels.hip", "dispatch_kernels.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def build_library(save_temps: bool = False) -> str:
    """Compile every HIP source and link libfp8q.so in the package folder."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    subprocess.check_call([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build_library(save_temps="--save-temps" in sys.argv))
