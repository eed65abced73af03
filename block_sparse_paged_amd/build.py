"""Build libmsa.so in-tree with hipcc for gfx950 (no JIT, no torch extension)."""
from __future__ import annotations

import glob
import os
import re
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


def scratch_users(remarks: str) -> list:
    """Kernels the compiler gave private (scratch) memory, from its
    kernel-resource-usage remarks: [(kernel, bytes per lane)]."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) and name:
            out.append((name, int(m.group(1))))
    return out


def _hipcc(srcs, lib: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    # The attention kernels wait for their direct-to-LDS loads by counting the
    # wave's outstanding vector memory operations; a register array the
    # compiler moved to scratch memory would add its own loads and stores to
    # that count (and cost far more than the registers).  Such a build fails.
    cmd = [hipcc, *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    lines, skip = [], 0
    for l in r.stderr.splitlines():
        if " remark: " in l:
            skip = 2                     # a remark, its source line and its caret line
            continue
        if skip:
            skip -= 1
            continue
        if noise not in l:
            lines.append(l)
    err = "\n".join(lines)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    spilled = scratch_users(r.stderr)
    if spilled:
        os.remove(tmp)
        raise RuntimeError("kernels given scratch memory: " + ", ".join(f"{n} ({b} B/lane)" for n, b in spilled))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
