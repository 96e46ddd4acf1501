"""Builds the GPU probes in this folder (test infrastructure, not the
library): every *.hip here becomes an executable of the same name, compiled
for gfx950 with the library's code-generation flags.

Usage:  python tests/probes/build_probes.py   (also run by __graft_entry__.build())
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build_probes() -> list[str]:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = []
    for src in sorted(glob.glob(os.path.join(HERE, "*.hip"))):
        exe = os.path.splitext(src)[0]
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", src, "-o", exe + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        os.replace(exe + ".tmp", exe)
        out.append(exe)
    return out


if __name__ == "__main__":
    print("\n".join(build_probes()))
