"""Build libpuro_fp8.so (gfx950) in-tree with hipcc.

    python blockwise_scaled_fp8_quant_amd/build.py        # or __graft_entry__.build()

(run as a file: importing it through the package would first load the library it builds)

Objects go to <repo>/_build/, the shared library next to this file.  Every HIP source
is compiled with packed-fp32 instruction generation disabled.
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
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpuro_fp8.so")
ARCH = "gfx950"

SOURCES = ["quant.hip", "gemm.hip", "gemm_w4.hip", "abi.cpp"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _flags(src: str):
    common = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if src.endswith(".hip"):
        return common + ["-x", "hip", f"--offload-arch={ARCH}",
                         "-mcode-object-version=5",
                         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    return common + ["-D__HIP_PLATFORM_AMD__"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
