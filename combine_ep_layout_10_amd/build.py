"""Builds libep.so (the HIP library behind include/ep.h) for gfx950, in-tree.

Flags: -O3; -ffp-contract=off so that every fused multiply-add in the
kernels is an explicit one; packed-FP32 instructions disabled (the
`-packed-fp32-ops` target feature); no fast-math, so binary32 division is
correctly rounded and denormals are kept.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libep.so")
SOURCES = ["ep_api.hip", "ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_fused.hip", "ep_gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def command(out: str = LIB, extra=()) -> list:
    return [HIPCC] + FLAGS + list(extra) + ["-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source into libep.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libep.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
