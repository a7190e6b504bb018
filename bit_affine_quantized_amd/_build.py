"""Compile libqmv.so (the matvec library) and libqmv_bench.so (measurement
references used only by bench.py) for gfx950 with hipcc, in-tree; the two
compile in parallel."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqmv.so")
BENCH_LIB = os.path.join(PKG, "libqmv_bench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["qmv_api.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # one IEEE operation per source operation: the device quantizer must
    # reproduce the fp32 steps exactly, and the kernels write their FMAs out
    "-ffp-contract=off",
    # packed fp32 math stays off (see the build notes in the design doc)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _start(sources, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                            text=True), tmp, out


def build(verbose: bool = False) -> str:
    jobs = [_start(SOURCES, LIB, verbose), _start(["bench_refs.hip"], BENCH_LIB, verbose)]
    errors = []
    for proc, tmp, out in jobs:
        text = proc.communicate()[0]
        if proc.returncode != 0:
            errors.append(f"hipcc failed for {os.path.basename(out)}:\n{text}")
        else:
            os.replace(tmp, out)
    if errors:
        raise RuntimeError("\n".join(errors))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
