"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
libep.so rebuilt with the sanitizers on the host pass only (`-Xarch_host`;
the gfx950 code is compiled as usual and never runs here), then the CPU
ABI tests run against it in a child process with clang's runtime
preloaded: every argument check, the workspace arithmetic and the status
strings, with out-of-range enum values, NULL and misaligned pointers.
Long (a full hipcc build): runs with EP_RUN_SLOW=1."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_host_code_clean_under_sanitizers(tmp_path):
    from combine_ep_layout_10_amd import build as b
    rt = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(b.HIPCC)), "llvm", "lib", "clang", "*",
                                       "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not rt:
        pytest.skip("clang ASan runtime not installed")
    lib = str(tmp_path / "libep_san.so")
    cmd = b.command(lib, ["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
                          "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), lib], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "runtime error" not in r.stderr


if __name__ == "__main__":
    # child process: the sanitized build replaces libep.so for the ABI tests
    sys.path.insert(0, ROOT)
    from combine_ep_layout_10_amd import _ffi
    _ffi.LIB_PATH = sys.argv[1]
    sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_cpu.py")]))
