"""Build libtpfuse.so in-tree with hipcc for gfx950.

Usage: python -m tensor_gemm_reduction_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libtpfuse.so")

SOURCES = ["tpf_kernels.hip", "tpf_api.cpp"]
HEADERS = ["tpf_device.hpp", "tpf_internal.hpp"]

# Packed-fp32 instructions are disabled for all device code: the compiler
# would otherwise form v_pk_* fp32 ops from plain float code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtpfuse)")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libtpfuse.so; returns its path."""
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs = []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + HIPCC_FLAGS
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
