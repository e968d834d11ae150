"""Builds libep.so (the HIP library behind include/ep.h) for gfx950, in-tree,
and libep_ceiling.so (access-pattern reference kernels the benchmark times
beside the path; no part of the API).

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


CEILING_LIB = os.path.join(HERE, "libep_ceiling.so")
CEILING_SOURCES = ["ep_ceiling.hip"]


def command(out: str = LIB, extra=(), sources=SOURCES) -> list:
    return [HIPCC] + FLAGS + list(extra) + ["-o", out] + [os.path.join(CSRC, s) for s in sources]


def _hipcc(out: str, sources, extra=(), verbose: bool = False) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = command(tmp, extra, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % os.path.basename(out))
    os.replace(tmp, out)


TORCH_SRC = os.path.join(CSRC, "ep_torch.cpp")
TORCH_EXT = os.path.join(HERE, "_ep_torch.so")


def build_torch_binding(verbose: bool = False) -> str:
    """Compile the torch binding (csrc/ep_torch.cpp, host C++ against the
    installed torch headers) into _ep_torch.so beside libep.so, which it
    links (rpath $ORIGIN)."""
    import shutil
    from torch.utils import cpp_extension
    bdir = os.path.join(HERE, "_build", "torch_ext")
    os.makedirs(bdir, exist_ok=True)
    cpp_extension.load(name="_ep_torch", sources=[TORCH_SRC], build_directory=bdir, verbose=verbose,
                       with_cuda=False, is_python_module=True, extra_cflags=["-O2"],
                       # runpath $ORIGIN (the package, where the copy below lives) and
                       # $ORIGIN/../.. (the package again, seen from the build folder, where
                       # load() imports it once), escaped for ninja ($$) and the shell (\$)
                       extra_ldflags=["-L" + HERE, "-lep", "-Wl,-rpath,\\$$ORIGIN:\\$$ORIGIN/../.."])
    tmp = TORCH_EXT + ".tmp%d" % os.getpid()
    shutil.copyfile(os.path.join(bdir, "_ep_torch.so"), tmp)
    os.replace(tmp, TORCH_EXT)
    return TORCH_EXT


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source into libep.so, then the torch binding that
    links it, then libep_ceiling.so (always recompiles all three)."""
    _hipcc(LIB, SOURCES, extra, verbose)
    build_torch_binding(verbose)
    _hipcc(CEILING_LIB, CEILING_SOURCES, (), verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
