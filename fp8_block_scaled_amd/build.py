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


# The device sources, compiled one object each.
HIP_SOURCES = ["gfg_gemm.hip", "gfg_gemm256.hip", "gfg_quant.hip", "gfg_ceiling.hip"]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    o = lambda n: os.path.join(out_dir, n)
    steps = [[hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
              "-o", o(src.replace(".hip", ".o"))] for src in HIP_SOURCES]
    steps.append(["g++", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-pthread", "-I", INCLUDE, "-I", CSRC,
                  "-c", os.path.join(CSRC, "gfg_host.cpp"), "-o", o("gfg_host.o")])
    objs = [o(src.replace(".hip", ".o")) for src in HIP_SOURCES] + [o("gfg_host.o")]
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


# Host sanitizers for the CPU tests: AddressSanitizer and UndefinedBehavior-
# Sanitizer on the host code only (the device code is built as usual), with
# clang's runtime, which the test process preloads.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (to preload)."""
    clang = "/opt/rocm/llvm/bin/clang++"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Build the library with ASan + UBSan on its host code into out_dir;
    returns the path of the .so (load it with GFG_LIBRARY and the runtime of
    asan_runtime() preloaded)."""
    hipcc = _hipcc()
    clang = "/opt/rocm/llvm/bin/clang++"
    os.makedirs(out_dir, exist_ok=True)
    common = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]
    o = lambda n: os.path.join(out_dir, n)
    steps = [[hipcc, f"--offload-arch={ARCH}", *common, *SAN_HOST, "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-c", os.path.join(CSRC, src), "-o", o(src.replace(".hip", ".o"))]
             for src in HIP_SOURCES]
    steps += [
        [clang, *common, "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
         os.path.join(CSRC, "gfg_host.cpp"), "-o", o("gfg_host.o")],
        [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *SAN_HOST[:4], "-shared-libasan",
         *[o(src.replace(".hip", ".o")) for src in HIP_SOURCES], o("gfg_host.o"), "-o", o("libgfg_san.so")],
    ]
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return o("libgfg_san.so")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
