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
HEADERS = ["tpf_device.hpp", "tpf_internal.hpp", "tpf_gemm.hpp", "tpf_stationary.hpp"]

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


# tpf_kernels.hip is compiled as KERNEL_PARTS translation units (-DTPF_PART=n),
# in parallel; see the part list at the top of that file.
KERNEL_PARTS = 9


def _compile_jobs(cc: str):
    jobs = []
    for part in range(KERNEL_PARTS):
        obj = os.path.join(LIBDIR, f"tpf_kernels_p{part}.o")
        jobs.append((f"tpf_kernels.hip (part {part})", obj,
                     [cc, "-x", "hip", "-c", os.path.join(CSRC, "tpf_kernels.hip"), "-o", obj,
                      f"-DTPF_PART={part}"] + HIPCC_FLAGS))
    for src in SOURCES:
        if src == "tpf_kernels.hip":
            continue
        obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + ".o")
        jobs.append((src, obj, [cc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + HIPCC_FLAGS))
    return jobs


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libtpfuse.so; returns its path."""
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    t0 = time.time()
    jobs = _compile_jobs(cc)
    procs = []
    for name, obj, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = []
    for name, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            failed.append(f"hipcc failed on {name}:\n{out}\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(failed))
    objs = [obj for _, obj, _ in jobs]
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
