"""GPU parity of the FP8 grouped GEMM (the consumer of the receive layout)
against the CPU oracle. A is the GPU's own FP8 dispatch output (itself
bit-exact against the oracle); weights are seeded random E4M3 codes (no NaN
patterns) with random binary32 128x128 scales.

Tolerance, from the arithmetic of gfx950's v_mfma_scale_f32_32x32x64_f8f6f4
as measured on MI355X (one MFMA sums 64 products): the products are aligned
to the largest raw exponent e_a + e_b among them (E4M3 exponent, -6 for
subnormals) and truncated toward zero 2^-13 below it, so products within 7
binades of the largest are exact and a smaller product p loses at most
min(|p|, 2^(E-13)); the running partial carried into the second MFMA of a
128-wide K block is aligned the same way, and the result is rounded to
binary32 (allowed one ulp, 2^-23 relative). The kernel then adds each block
partial times fl(sa * sb) into a binary32 accumulator with one FMA, so the
promotion adds at most (K/128 + 2) * 2^-24 * M, M = sum_kb |sa sb| sum_k
|a b|. Kernel and oracle each round to bf16 once (half an ulp, at most 2^-8
of the value, each): |gpu - oracle| <= 2^-7 |oracle| (1 + 2^-7)
+ sum_kb |sa sb| err_kb (1 + 2^-20) + (K/128 + 2) 2^-24 M. (Checked on
MI355X: on random full-range codes, single and chained MFMA errors stay
within 0.15 of the per-MFMA part of this bound.)"""
import numpy as np
import pytest
import torch

import oracle
from ep_workloads import WORKLOADS, make_inputs, random_routing_table, f32_to_bf16_bits
from gpu_common import log, to_dev, to_dev_bf16, host, cfg_of

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from combine_ep_layout_10_amd import ops


def random_codes(gen, shape):
    """Uniform over the 254 non-NaN E4M3FN codes (0x7F and 0xFF skipped)."""
    c = torch.randint(0, 254, shape, dtype=torch.uint8, device="cuda", generator=gen)
    return torch.where(c >= 0x7F, c + 1, c)


def decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_val(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def raw_exponent(codes: np.ndarray) -> np.ndarray:
    """E4M3 exponent of each code (-6 for subnormals, very small for zero)."""
    c = np.asarray(codes).astype(np.int32)
    ef = (c >> 3) & 15
    ex = np.where(ef > 0, ef - 7, -6)
    return np.where((c & 0x7F) == 0, -1000, ex)


def gemm_bound(a, sa, b, sb, rows, e, cols):
    """Bound on |binary32 result - exact| for rows x cols of expert e, and the
    magnitude M, following the MFMA model in the module docstring."""
    K = a.shape[1]
    KB = K // 128
    va = decode(a[rows]).reshape(len(rows), K // 64, 64)
    vb = decode(b[e][cols]).reshape(len(cols), K // 64, 64)
    xa = raw_exponent(a[rows]).reshape(len(rows), K // 64, 64)
    xb = raw_exponent(b[e][cols]).reshape(len(cols), K // 64, 64)
    scale = np.abs(sa[rows])[:, None, :].astype(np.float64) * np.abs(sb[e][np.asarray(cols) // 128])[None, :, :]
    err = np.zeros((len(rows), len(cols)))
    M = np.zeros((len(rows), len(cols)))
    for kb in range(KB):
        blk_err = np.zeros((len(rows), len(cols)))
        carry = np.zeros((len(rows), len(cols)))
        for half in range(2):
            ch = 2 * kb + half
            p = va[:, None, ch, :] * vb[None, :, ch, :]                    # [r, n, 64]
            E = (xa[:, None, ch, :] + xb[None, :, ch, :]).max(-1)
            if half == 1:
                E = np.maximum(E, np.floor(np.log2(np.maximum(np.abs(carry), 2.0 ** -1000))).astype(int) + 1)
            q = np.ldexp(1.0, E - 13)
            trunc = np.minimum(np.abs(p), q[..., None]).sum(-1) + (q if half == 1 else 0)
            carry = carry + p.sum(-1)
            blk_err += trunc + 2.0 ** -23 * np.abs(carry)
            M += scale[:, :, kb] * np.abs(p).sum(-1)
        err += scale[:, :, kb] * blk_err
    return err * (1 + 2.0 ** -20) + (KB + 2) * 2.0 ** -24 * M, M


def check(got_bits, ref_bits, bound):
    got, ref = bf16_val(got_bits), bf16_val(ref_bits)
    lim = 2.0 ** -7 * np.abs(ref) * (1 + 2.0 ** -7) + bound
    err = np.abs(got - ref)
    assert np.all(err <= lim), float((err / np.maximum(lim, 1e-300)).max())
    return err, lim


def run_case(T, E, k, A, H, N, mode=0, C=0, seed=0, masked=0.0, idx=None):
    log("gemm case T=%d E=%d k=%d A=%d H=%d N=%d mode=%d C=%d" % (T, E, k, A, H, N, mode, C))
    rng = np.random.default_rng(seed)
    if idx is None:
        idx = random_routing_table(rng, T, E, k, masked_frac=masked)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A, capacity=C, mode=mode)
    h = ops.layout(cfg, to_dev(idx))
    q, s = ops.dispatch(h, to_dev_bf16(x), ops.FP8_QUANTIZE)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    b = random_codes(gen, (E, N, H))
    sb = (torch.rand((E, N // 128, H // 128), device="cuda", generator=gen) * 1e-2 + 1e-3)
    out = torch.full((cfg.recv_rows_bound(), N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ops.grouped_gemm_fp8(h, q, s, b, sb, out=out)
    torch.cuda.synchronize()
    qh, sh, bh, sbh = host(q), host(s), host(b), host(sb)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    cnt, pad, R = h.read_counts()
    off = host(h.expert_off)
    if mode == 0:
        rb, re_ = off[:-1], off[1:]             # COMPACT: padding rows included (zero codes)
    else:
        rb = np.arange(E, dtype=np.int32) * C
        re_ = rb + pad                          # FIXED: rows past the count are unspecified
    ref = oracle.grouped_gemm_fp8(rb, re_, qh, sh, bh, sbh)
    for e in range(E):
        rows = np.arange(rb[e], re_[e])
        if rows.size == 0:
            continue
        bound, _ = gemm_bound(qh, sh, bh, sbh, rows, e, np.arange(N))
        check(got[rows], ref[rows], bound)
    written = np.zeros(cfg.recv_rows_bound(), bool)
    for e in range(E):
        lim = re_[e] if mode == 0 else rb[e] + -(-pad[e] // 128) * 128
        written[rb[e]:lim] = True
    assert np.all(got[~written] == 0xFFFF)      # rows the GEMM does not cover are untouched
    return h


@pytest.mark.parametrize("T,E,k,A,H,N", [
    (300, 6, 2, 128, 512, 256),
    (97, 5, 3, 256, 256, 384),     # alignment 256: two tiles per padded group
    (40, 16, 2, 128, 128, 128),    # many experts with no rows
    (60, 4, 2, 128, 128, 256),     # 256-column kernel, one K block: its prologue re-issues the only stage
    (60, 4, 2, 128, 256, 512),     # two K blocks, two column tiles
    (24, 2, 1, 128, 32768, 256),   # the 256-column kernel's largest K (256 blocks of 128)
    (24, 2, 1, 128, 32896, 256),   # one K block more: the 128-column kernel takes it
])
def test_grouped_gemm_compact(T, E, k, A, H, N):
    run_case(T, E, k, A, H, N, seed=T + E)


def test_grouped_gemm_piece_boundaries():
    """Experts holding 0, 1, 32, 33, 64, 65, 96, 97, 128 and 129 pairs: 32-row
    pieces that are padding only are skipped and written as zeros, pieces
    with at least one pair are computed (COMPACT and FIXED)."""
    counts = [0, 1, 32, 33, 64, 65, 96, 97, 128, 129]
    idx = np.concatenate([np.full(c, e, np.int64) for e, c in enumerate(counts)])
    np.random.default_rng(3).shuffle(idx)
    idx = idx[:, None]
    run_case(idx.shape[0], len(counts), 1, 128, 256, 256, seed=11, idx=idx)
    run_case(idx.shape[0], len(counts), 1, 1, 256, 256, mode=1, C=256, seed=12, idx=idx)


def test_grouped_gemm_fixed():
    run_case(128, 8, 2, 1, 256, 256, mode=1, C=128, seed=5)
    run_case(200, 4, 2, 1, 384, 128, mode=1, C=256, seed=6)     # two tile slots per expert


def test_grouped_gemm_masked_and_unsupported():
    run_case(150, 6, 3, 128, 256, 256, seed=7, masked=0.2)
    cfg = ops.Config(max_tokens=8, hidden=256, num_experts=4, num_topk=2, expert_alignment=64)
    h = ops.layout(cfg, torch.zeros((8, 2), dtype=torch.int64, device="cuda"))
    R = cfg.recv_rows_bound()
    with pytest.raises(Exception):                # alignment not a multiple of 128
        ops.grouped_gemm_fp8(h, torch.zeros((R, 256), dtype=torch.uint8, device="cuda"),
                             torch.zeros((R, 2), device="cuda"),
                             torch.zeros((4, 128, 256), dtype=torch.uint8, device="cuda"),
                             torch.zeros((4, 1, 2), device="cuda"))


def test_grouped_gemm_no_zero_pad_and_empty():
    """EP_FLAG_NO_ZERO_PAD: padding rows keep whatever the receive buffer held
    (here E4M3 NaN codes and NaN scales); every row holding a pair is still
    exact within the bound, since an output row depends on its own A row
    only. An empty batch leaves the output untouched."""
    T, E, k, A, H, N = 300, 6, 2, 128, 256, 256
    rng = np.random.default_rng(21)
    idx = random_routing_table(rng, T, E, k)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A,
                     flags=ops.FLAG_NO_ZERO_PAD)
    R = cfg.recv_rows_bound()
    h = ops.layout(cfg, to_dev(idx))
    q = torch.full((R, H), 0x7F, dtype=torch.uint8, device="cuda")
    s = torch.full((R, H // 128), float("nan"), dtype=torch.float32, device="cuda")
    ops.dispatch(h, to_dev_bf16(x), ops.FP8_QUANTIZE, recv=q, recv_scales=s)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    b = random_codes(gen, (E, N, H))
    sb = torch.rand((E, N // 128, H // 128), device="cuda", generator=gen) * 1e-2 + 1e-3
    out = torch.full((R, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ops.grouped_gemm_fp8(h, q, s, b, sb, out=out)
    torch.cuda.synchronize()
    qh, sh, bh, sbh = host(q), host(s), host(b), host(sb)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    cnt, pad, _ = h.read_counts()
    off = host(h.expert_off)
    rb, re_ = off[:-1], off[:-1] + cnt
    ref = oracle.grouped_gemm_fp8(rb, re_, qh, sh, bh, sbh)
    for e in range(E):
        rows = np.arange(rb[e], re_[e])
        if rows.size:
            bound, _ = gemm_bound(qh, sh, bh, sbh, rows, e, np.arange(N))
            check(got[rows], ref[rows], bound)
    # empty batch: nothing is written
    h0 = ops.layout(cfg, torch.zeros((0, k), dtype=torch.int64, device="cuda"))
    out0 = torch.full((R, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ops.grouped_gemm_fp8(h0, q, s, b, sb, out=out0)
    torch.cuda.synchronize()
    assert bool((out0.view(torch.int16) == -1).all())


def test_grouped_gemm_v3_sampled():
    """The V3 receive layout (8192 x 7168, 256 experts, top-8, 80K rows) times
    a 7168 -> 4096 expert matrix per expert (7.5 GB of E4M3 weights): 512
    sampled outputs, each against the oracle on its row and weight rows."""
    wl = WORKLOADS["v3"]
    inp = make_inputs(wl, with_y=False)
    cfg = cfg_of(wl)
    h = ops.layout(cfg, to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
    q, s = ops.dispatch(h, to_dev_bf16(inp["x"]), ops.FP8_QUANTIZE)
    N = 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    b = random_codes(gen, (wl.E, N, wl.H))
    sb = torch.rand((wl.E, N // 128, wl.H // 128), device="cuda", generator=gen) * 1e-2 + 1e-3
    out = ops.grouped_gemm_fp8(h, q, s, b, sb)
    torch.cuda.synchronize()
    off = host(h.expert_off)
    R = int(off[-1])
    rng = np.random.default_rng(12)
    rows = rng.integers(0, R, 512)
    cols = rng.integers(0, N, 512)
    got = out.view(torch.int16)[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy().view(np.uint16)
    for i, (r, n) in enumerate(zip(rows, cols)):
        e = int(np.searchsorted(off, r, side="right") - 1)
        a1 = host(q[r:r + 1])
        s1 = host(s[r:r + 1])
        n0 = (n // 128) * 128
        b1 = host(b[e:e + 1, n0:n0 + 128])
        sb1 = host(sb[e:e + 1, n // 128:n // 128 + 1])
        a_pad = np.zeros((128, wl.H), np.uint8)
        a_pad[0] = a1[0]
        s_pad = np.zeros((128, wl.H // 128), np.float32)
        s_pad[0] = s1[0]
        ref = oracle.grouped_gemm_fp8(np.array([0], np.int32), np.array([1], np.int32), a_pad, s_pad, b1, sb1)[0, n - n0]
        bound, _ = gemm_bound(a_pad, s_pad, b1, sb1, np.array([0]), 0, np.array([n - n0]))
        check(np.array([got[i]]), np.array([ref]), bound[0])
    del b, out
    torch.cuda.empty_cache()
