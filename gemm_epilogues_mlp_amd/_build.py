"""Build libswiglu.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage:  python -m gemm_epilogues_mlp_amd._build [--save-temps DIR]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libswiglu.so")
SOURCES = ["swiglu_kernels.hip", "swiglu_table.cpp", "swiglu_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libswiglu.so)")


def flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        # packed fp32 VALU ops stay off: ordinary fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, *extra,
    ]


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    objs = []
    os.makedirs(os.path.join(PKG, "_objs"), exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(PKG, "_objs", src + ".o")
        extra = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [cc, *flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            # keep the device assembly (.s) and IR next to each other in save_temps
            os.makedirs(save_temps, exist_ok=True)
            cmd.insert(1, "-save-temps")
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=save_temps or PKG)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    st = None
    if "--save-temps" in sys.argv:
        st = sys.argv[sys.argv.index("--save-temps") + 1]
    print(build(st, verbose=True))
