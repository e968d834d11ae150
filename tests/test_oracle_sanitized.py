"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, gcc): its C source built with `-fsanitize=address,undefined,
float-cast-overflow`, then, in a child process with the sanitizer runtimes
preloaded, (1) a sweep of edge-case shapes through every entry point (empty
batches, ids out of range and negative, FIXED overflow, 32- and 64-bit ids,
top-k up to 8, both padding modes, random bf16 bit patterns including NaN
and infinity, GEMM expert ranges straight from the layouts) and (2) the
oracle's pin tests. Any out-of-bounds access, overflow or invalid
conversion aborts the child. Long: runs with EP_RUN_SLOW=1."""
import itertools
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_layout.py", "test_oracle_numerics.py", "test_oracle_gemm.py"]


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True, check=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_clean_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libep_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC",
                    "-o", lib, os.path.join(ROOT, "oracle", "ep_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan + " " + ubsan, EP_RUN_SLOW="0",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), lib], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "sweep cases 2688" in r.stdout and " passed" in r.stdout


def _sweep(oracle):
    from oracle import MODE_COMPACT, MODE_FIXED
    rng = np.random.default_rng(7)
    n = 0
    for mode, T, E, k, D, bits in itertools.product((MODE_COMPACT, MODE_FIXED), (0, 1, 5, 33), (1, 4, 8),
                                                     (1, 2, 4, 8), (1, 2, 4), (32, 64)):
        if E % D:
            continue
        for a_or_c in (1, 3, 16):
            A, C = (a_or_c, 1) if mode == MODE_COMPACT else (1, a_or_c)
            idx = rng.integers(-2, E + 2, size=(T, k)).astype(np.int64 if bits == 64 else np.int32)
            w = rng.standard_normal((T, k)).astype(np.float32)
            lay = oracle.layout(mode, T, E, k, A, D, C, idx, w)
            R = lay["rows_bound"]
            for H in (128, 256):
                x = rng.integers(0, 1 << 16, size=(T, H)).astype(np.uint16)
                for zp in (True, False):
                    oracle.dispatch_bf16(lay, x, k, None, zp)
                    oracle.dispatch_bf16(lay, x, k, w, zp)
                    oracle.dispatch_fp8(lay, x, k, zp)
                    oracle.dispatch_fp8_prequant(lay, rng.integers(0, 256, (T, H)).astype(np.uint8),
                                                 rng.standard_normal((T, H // 128)).astype(np.float32), k, zp)
                    oracle.combine_backward_fp8(lay, x, k, w, zp)
                y = rng.integers(0, 1 << 16, size=(max(R, 1), H)).astype(np.uint16)
                oracle.combine(lay, y, k, w, rng.standard_normal(max(R, 1)).astype(np.float32), T=T)
                oracle.combine(lay, y, k, None, None, T=T)
                oracle.combine_weight_grad(lay, x, y, k)
                n += 1
                if R == 0:
                    continue
                if mode == MODE_COMPACT:
                    rb = lay["expert_off"][:-1].astype(np.int32)
                    re_ = rb + lay["pad"]
                else:
                    rb = (np.arange(E) * C).astype(np.int32)
                    re_ = rb + np.minimum(lay["cnt"], C).astype(np.int32)
                a = rng.integers(0, 256, (R, H)).astype(np.uint8)
                sa = rng.random((R, H // 128)).astype(np.float32)
                b = rng.integers(0, 256, (E, 128, H)).astype(np.uint8)
                sb = rng.random((E, 1, H // 128)).astype(np.float32)
                oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb)
                pairs = np.stack([rng.integers(0, R, 7), rng.integers(0, 128, 7)], 1)
                oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb, pairs=pairs)
    oracle.e4m3_encode(rng.standard_normal(1000).astype(np.float32) * 1e3)
    oracle.bf16_rne(np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-45], np.float32))
    for code in range(256):
        oracle.e4m3_code_value(code)
    for length in (1, 7, 128, 300):
        oracle.quantize_block(rng.integers(0, 1 << 16, length).astype(np.uint16))
    print("sweep cases", n, flush=True)


if __name__ == "__main__":
    # child process: the sanitized library replaces the oracle's own build
    sys.path.insert(0, ROOT)
    import oracle
    oracle._LIB = sys.argv[1]
    _sweep(oracle)
    sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] +
                         [os.path.join(ROOT, "tests", f) for f in PINS]))
