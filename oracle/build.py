"""Build the plain C oracle (oracle/tpf_oracle.c) into oracle/lib/libtpf_oracle.so.

Test infrastructure: compiled with the host C compiler, OpenMP over output
rows, no target-specific flags (it runs on whatever host the tests or the
benchmark's CPU baseline run on).

Usage: python -m oracle.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tpf_oracle.c")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libtpf_oracle.so")
CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"]


def compiler() -> str:
    for cand in (os.environ.get("CC"), "gcc", "cc"):
        if cand and shutil.which(cand):
            return cand
    raise RuntimeError("no C compiler found for the oracle")


def build_source(src: str, out: str, extra=()) -> str:
    """Compile one oracle source file into a shared library at `out`."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [compiler()] + CFLAGS + list(extra) + ["-o", tmp, src, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    out = build_source(SRC, LIB)
    if verbose:
        print(f"built {out}", flush=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
