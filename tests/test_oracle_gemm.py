"""Pins for the oracle's FP8 grouped GEMM (the consumer of the aligned
layout). Independent references: exact integer matmuls (numpy int64),
power-of-two scales (exact scaling), torch float64 matmul of torch's own
float8_e4m3fn decode, torch's bf16 cast on values whose rounding it can
represent exactly, and expert-range bookkeeping."""
import numpy as np
import pytest
import torch

import oracle

E4M3 = {-2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40}


def codes_of(ints: np.ndarray) -> np.ndarray:
    lut = np.zeros(5, np.uint8)
    for v, c in E4M3.items():
        lut[v + 2] = c
    return lut[ints + 2]


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def to_bf16_exact(v: np.ndarray) -> np.ndarray:
    """torch's bf16 cast of float32 values (exact when v is a float32)."""
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_codes(rng, shape):
    """Random E4M3FN codes without the NaN patterns 0x7F / 0xFF."""
    c = rng.integers(0, 254, size=shape, dtype=np.int32)
    c = np.where(c >= 0x7F, c + 1, c)
    return c.astype(np.uint8)


def ranges(counts, align=128):
    begin, end, off = [], [], 0
    for c in counts:
        begin.append(off)
        end.append(off + c)
        off += -(-c // align) * align
    return np.array(begin, np.int32), np.array(end, np.int32), off


def test_integer_matmul_exact():
    """Codes of -1, 0, 1 and unit scales: every output is an integer of
    magnitude <= 256 (exact in bf16), equal to numpy's int64 matmul per
    expert; rows outside the ranges stay untouched."""
    rng = np.random.default_rng(51)
    E, K, N = 3, 256, 256
    rb, re_, R = ranges([130, 0, 45])
    ai = rng.integers(-1, 2, size=(R, K))
    bi = rng.integers(-1, 2, size=(E, N, K))
    C = oracle.grouped_gemm_fp8(rb, re_, codes_of(ai), np.ones((R, K // 128), np.float32), codes_of(bi),
                                np.ones((E, N // 128, K // 128), np.float32))
    for e in range(E):
        for r in range(rb[e], re_[e]):
            want = to_bf16_exact((ai[r] @ bi[e].T).astype(np.float32))
            assert np.array_equal(C[r], want), (e, r)
    inside = np.zeros(R, bool)
    for e in range(E):
        inside[rb[e]:re_[e]] = True
    assert np.all(C[~inside] == 0xFFFF)


def test_power_of_two_scales_exact():
    """Scales 2^i (per row and 1x128 block) and 2^j (per 128x128 weight
    block) multiply the integer block sums exactly."""
    rng = np.random.default_rng(52)
    E, K, N = 2, 384, 256
    rb, re_, R = ranges([128, 100])
    ai = rng.integers(-1, 2, size=(R, K))
    bi = rng.integers(-1, 2, size=(E, N, K))
    pa = rng.integers(-3, 4, size=(R, K // 128))
    pb = rng.integers(-3, 4, size=(E, N // 128, K // 128))
    C = oracle.grouped_gemm_fp8(rb, re_, codes_of(ai), np.ldexp(1.0, pa).astype(np.float32), codes_of(bi),
                                np.ldexp(1.0, pb).astype(np.float32))
    for e in range(E):
        for r in range(rb[e], re_[e]):
            want = np.zeros(N)
            for kb in range(K // 128):
                blk = ai[r, kb * 128:(kb + 1) * 128] @ bi[e, :, kb * 128:(kb + 1) * 128].T
                want += blk * np.ldexp(1.0, pa[r, kb] + pb[e, np.arange(N) // 128, kb])
            # |want| stays far below 2^24, so the float32 cast is exact
            assert np.array_equal(C[r], to_bf16_exact(want.astype(np.float32))), (e, r)


def test_against_torch_float64():
    """Random codes and binary32 scales: within half a bf16 ulp of torch's
    float64 matmul of torch's E4M3 decode (plus torch's own summation error),
    and the sampled form equals the full one."""
    rng = np.random.default_rng(53)
    E, K, N = 3, 512, 384
    rb, re_, R = ranges([140, 60, 128])
    a = random_codes(rng, (R, K))
    b = random_codes(rng, (E, N, K))
    sa = (rng.random((R, K // 128)) * 0.01 + 1e-4).astype(np.float32)
    sb = (rng.random((E, N // 128, K // 128)) * 0.01 + 1e-4).astype(np.float32)
    C = oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb)
    A = torch_decode(a).reshape(R, K // 128, 128)
    for e in range(E):
        B = torch_decode(b[e]).reshape(N, K // 128, 128)
        rows = np.arange(rb[e], re_[e])
        blk = np.einsum("rkc,nkc->rnk", A[rows], B)                 # float64 block sums
        scale = sa[rows][:, None, :].astype(np.float64) * sb[e][np.arange(N) // 128][None, :, :]
        ref = (blk * scale).sum(-1)
        mag = (np.abs(blk) * scale).sum(-1)
        got = (C[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))).astype(int) - 7)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-12 * mag), e
    pairs = np.stack([rng.integers(0, R, 500), rng.integers(0, N, 500)], 1).astype(np.int64)
    at = oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb, pairs=pairs)
    inside = np.zeros(R, bool)
    for e in range(E):
        inside[rb[e]:re_[e]] = True
    for i, (r, n) in enumerate(pairs):
        assert at[i] == (C[r, n] if inside[r] else 0)


def test_bf16_rounding_of_binary64_results():
    """The final rounding is round-to-nearest-even on the binary64 sum:
    results exactly halfway between two bf16 values go to the even one
    (torch's float32 -> bf16 cast is exact for these), a product of scales
    just above the halfway point rounds up and one just below rounds down."""
    E, K, N = 1, 128, 128
    rb, re_ = np.array([0], np.int32), np.array([4], np.int32)
    a = np.zeros((128, K), np.uint8)
    b = np.zeros((1, N, K), np.uint8)
    a[:4, 0] = 0x38                                   # 1.0
    b[0, :, 0] = 0x38
    # block sums are 1; the scale product picks the value
    sa = np.ones((128, 1), np.float32)
    sb = np.ones((1, 1, 1), np.float32)
    for t in [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 + 2 ** -7, 1.0 + 2 ** -9]:
        sa[:4, 0] = np.float32(t)
        got = oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb)[:4, 0]
        assert np.all(got == to_bf16_exact(np.float32(t))), t
    # (1 + 2^-8) * (1 + 2^-22) lies just above the midpoint of 1 and 1 + 2^-7
    sa[:4, 0] = np.float32(1.0 + 2 ** -8)
    sb[0, 0, 0] = np.float32(1.0 + 2 ** -22)
    got = oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb)[:4, 0]
    assert np.all(got == to_bf16_exact(np.float32(1.0 + 2 ** -7)))
    sb[0, 0, 0] = np.float32(1.0 - 2 ** -23)           # just below: rounds down
    got = oracle.grouped_gemm_fp8(rb, re_, a, sa, b, sb)[:4, 0]
    assert np.all(got == to_bf16_exact(np.float32(1.0)))
