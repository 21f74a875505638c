"""Build libgfg.so (HIP kernels for gfx950 + host quantizers) in-tree with hipcc.

    python -m fp8_block_scaled_amd.build          # writes fp8_block_scaled_amd/libgfg.so
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
LIB = os.path.join(PKG, "libgfg.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


# Device code: gfx950 only; packed-fp32 instructions are kept out of the device
# code generation (the host pass ignores the feature with a warning).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    steps = [
        [hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "gfg_gemm.hip"),
         "-o", os.path.join(out_dir, "gfg_gemm.o")],
        [hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "gfg_quant.hip"),
         "-o", os.path.join(out_dir, "gfg_quant.o")],
        ["g++", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-pthread", "-I", INCLUDE, "-I", CSRC, "-c",
         os.path.join(CSRC, "gfg_host.cpp"), "-o", os.path.join(out_dir, "gfg_host.o")],
    ]
    objs = [os.path.join(out_dir, "gfg_gemm.o"), os.path.join(out_dir, "gfg_quant.o"),
            os.path.join(out_dir, "gfg_host.o")]
    tmp = LIB + ".tmp"
    steps.append([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp])
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
