"""Build libmsa.so in-tree with hipcc for gfx950 (no JIT, no torch extension)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmsa.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


BENCH_CSRC = os.path.join(PKG, "bench_csrc")
BENCH_LIB = os.path.join(PKG, "libmsa_bench.so")


def build(verbose: bool = False) -> str:
    """Builds libmsa.so (the library) and libmsa_bench.so (the measurement
    kernels bench.py calibrates with); returns the library's path."""
    _hipcc(sorted(glob.glob(os.path.join(BENCH_CSRC, "*.hip"))), BENCH_LIB, verbose)
    return _hipcc(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), LIB, verbose)


def _hipcc(srcs, lib: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
