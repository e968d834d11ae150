"""Kernel resources, checked at build time on the CPU (no GPU needed).

Every kernel of the library is compiled for gfx950 with the library's own
flags and the compiler's resource report (-Rpass-analysis=
kernel-resource-usage). Two properties must hold for every kernel:
  * ScratchSize 0: no register spills to per-lane scratch memory (the
    README's EP_JIT_PTXAS_CHECK asserts the same for its JIT kernels: no
    local memory);
  * no packed binary32 instructions in the device code: the build disables
    them (-packed-fp32-ops), and this checks that the flag took effect.
"""
import os
import re
import subprocess

import pytest

from combine_ep_layout_10_amd import build as B

REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs|Occupancy \[waves/SIMD\]): (\S+)")
PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def compile_reports(tmp_path):
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    procs = []
    for src in B.SOURCES:
        out = tmp_path / (src + ".s")
        cmd = [B.HIPCC] + flags + ["--cuda-device-only", "-S", "-Rpass-analysis=kernel-resource-usage",
                                   "-o", str(out), os.path.join(B.CSRC, src)]
        procs.append((src, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    reports = {}
    for src, out, p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-2000:]
        kernels, cur = {}, None
        for key, val in REMARK.findall(err):
            if key == "Function Name":
                cur = val
                kernels[cur] = {}
            elif cur is not None:
                kernels[cur][key.split()[0]] = val
        reports[src] = (kernels, out.read_text())
    return reports


@pytest.fixture(scope="module")
def reports(tmp_path_factory):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not installed")
    return compile_reports(tmp_path_factory.mktemp("kres"))


def test_every_kernel_has_no_scratch(reports):
    n = 0
    for src, (kernels, _) in reports.items():
        for name, r in kernels.items():
            assert r.get("ScratchSize") == "0", (src, name, r)
            n += 1
    assert n >= 20, n  # every template instance of every kernel was seen


def test_no_packed_fp32_instructions(reports):
    for src, (_, asm) in reports.items():
        hits = PACKED_F32.findall(asm)
        assert not hits, (src, hits[:5])
