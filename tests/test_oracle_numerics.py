"""Pins for the oracle's number formats, FP8 quantisation, dispatch copies
and combine reduction.

Independent references used here (none shares code with the oracle):
  * hand-worked fixtures under tests/golden/ (OCP E4M3 codes, combine
    rounding cases) with their derivations;
  * torch's CPU float8_e4m3fn and bfloat16 casts (round to nearest even;
    torch does not saturate, so values are clamped to +-448 first);
  * an exact rational (fractions.Fraction) model of binary32 rounding;
  * numpy float32 arithmetic (IEEE division and multiplication);
  * closed forms: the BF16 identity round trip and the unweighted dual.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from ep_workloads import WORKLOADS, make_inputs, bf16_bits_to_f32, f32_to_bf16_bits, random_routing_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def torch_e4m3(v32: np.ndarray) -> np.ndarray:
    """Library reference: clamp to +-448 (satfinite), then torch's RNE cast."""
    t = torch.from_numpy(np.clip(np.asarray(v32, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_values() -> np.ndarray:
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nearest_code_search(v32: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code by direct search over the decoded code table
    (ties to the even code), saturating. Vectorised, from the table only."""
    vals = torch_e4m3_values()          # codes 0x00..0x7E, increasing
    a = np.abs(np.asarray(v32, np.float32).astype(np.float64))
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= 448.0, 0x7E, code).astype(np.uint8)
    sign = np.signbit(np.asarray(v32, np.float32)).astype(np.uint8) << 7
    return code | sign


def f32_from_bits(b):
    return np.array([b], np.uint32).view(np.float32)[0]


def round_f32_exact(x: Fraction) -> Fraction:
    """Exact binary32 round-to-nearest-even of a rational (normal range)."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = a / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * Fraction(n) * Fraction(2) ** (e - 23)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in the monotone integer map of bf16 patterns (+0 == -0)."""
    def key(u):
        u = np.asarray(u, np.uint16).astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


# ---------------------------------------------------------------- E4M3 codec

def test_e4m3_golden_codes():
    with open(os.path.join(GOLDEN, "e4m3_codes.json")) as f:
        cases = json.load(f)["cases"]
    v = np.array([float(c["v"]) for c in cases], np.float32)
    got = oracle.e4m3_encode(v)
    for c, g in zip(cases, got):
        assert g == int(c["code"], 16), (c, hex(g))


def test_e4m3_code_table_matches_torch():
    vals = torch_e4m3_values()
    for c in range(0x7F):
        assert oracle.e4m3_code_value(c) == vals[c]


def _critical_values():
    """Every code value and every midpoint between neighbouring codes, with
    the 4 binary32 neighbours on each side, both signs."""
    vals = torch_e4m3_values()
    pts = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2, [448.0, 464.0, 480.0, 1e4]])
    pts32 = pts.astype(np.float32)
    out = [pts32]
    for direction in (np.float32(np.inf), np.float32(0)):
        cur = pts32.copy()
        for _ in range(4):
            cur = np.nextafter(cur, direction)
            out.append(cur)
    v = np.concatenate(out)
    return np.concatenate([v, -v])


def test_e4m3_encoder_critical_points():
    v = _critical_values()
    got = oracle.e4m3_encode(v)
    assert np.array_equal(got, torch_e4m3(v))
    assert np.array_equal(got, nearest_code_search(v))


def test_e4m3_encoder_all_bf16_patterns():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    got = oracle.e4m3_encode(v)
    assert np.array_equal(got, torch_e4m3(v))
    assert np.array_equal(got, nearest_code_search(v))


def test_e4m3_encoder_random_binary32():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x43F00000, size=2_000_000, dtype=np.uint32)   # |v| < 480
    v = bits.view(np.float32) * np.where(rng.random(bits.size) < 0.5, -1, 1).astype(np.float32)
    got = oracle.e4m3_encode(v)
    assert np.array_equal(got, torch_e4m3(v))
    assert np.array_equal(got, nearest_code_search(v))


@pytest.mark.slow
def test_e4m3_encoder_exhaustive_nonnegative():
    """Every non-negative binary32 up to and beyond 448 (2^30+ values)."""
    top = int(np.float32(480.0).view(np.uint32))
    step = 1 << 24
    for b0 in range(0, top, step):
        v = np.arange(b0, min(top, b0 + step), dtype=np.uint32).view(np.float32)
        assert np.array_equal(oracle.e4m3_encode(v), torch_e4m3(v)), hex(b0)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_against_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F000000, size=2_000_000, dtype=np.uint32)
    # add exact ties and near-ties
    base = rng.integers(0, 0x7F00, size=20000, dtype=np.uint32) << 16
    bits = np.concatenate([bits, base | 0x8000, base | 0x7FFF, base | 0x8001, base | 0x18000])
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.bf16_rne(v), f32_to_bf16_bits(v))


# ---------------------------------------------------------------- quantisation

def independent_quantize(xb_bits: np.ndarray):
    """numpy float32 steps + torch cast, one 128-block per row of xb_bits."""
    x = bf16_bits_to_f32(xb_bits)
    amax = np.abs(x).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    v = (x / safe[:, None]).astype(np.float32)
    q = torch_e4m3(v)
    q[scale == 0] = 0
    return scale, q


def quant_test_blocks(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x[: n // 4] *= np.float32(100.0) ** rng.integers(-3, 3, size=(n // 4, 1))
    x[n // 4: n // 2, rng.integers(0, 128)] *= 1000.0        # one outlier per block
    x[n // 2: n // 2 + 8] = 0.0                              # zero blocks
    x[n // 2 + 8: n // 2 + 16, :127] = 0.0                   # single non-zero
    x[n // 2 + 16: n // 2 + 24] *= np.float32(2.0 ** -120)   # bf16 subnormal-ish range
    return f32_to_bf16_bits(x)


def test_quantize_blocks_against_independent():
    xb = quant_test_blocks(4000, 11)
    s_ind, q_ind = independent_quantize(xb)
    for i in range(xb.shape[0]):
        s, q = oracle.quantize_block(xb[i])
        assert np.float32(s) == s_ind[i] or (s == 0 and s_ind[i] == 0), i
        assert np.array_equal(q, q_ind[i]), i


def test_quantize_invariants():
    """Error bound of E4M3 with 1x128 scaling; the amax element maps to
    +-448; zero blocks give scale 0 and zero codes."""
    xb = quant_test_blocks(2000, 12)
    vals = torch_e4m3_values()
    for i in range(xb.shape[0]):
        s, q = oracle.quantize_block(xb[i])
        x = bf16_bits_to_f32(xb[i]).astype(np.float64)
        if np.all(x == 0):
            assert s == 0.0 and np.all(q == 0)
            continue
        mag = vals[q & 0x7F] * np.where(q & 0x80, -1.0, 1.0)
        deq = mag * np.float64(s)
        bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) * (1 + 2.0 ** -20)
        assert np.all(np.abs(deq - x) <= bound), i
        assert np.all((q & 0x7F) <= 0x7E)
        j = int(np.argmax(np.abs(x)))
        assert (q[j] & 0x7F) == 0x7E
        assert np.float32(s) == np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))


# ---------------------------------------------------------------- dispatch

def _layout_for(wl, inp):
    return oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, inp["topk_idx"], inp["topk_w"])


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_dispatch_bf16_copies(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl, with_y=False)
    lay = _layout_for(wl, inp)
    recv = oracle.dispatch_bf16(lay, inp["x"], wl.k)
    slot = lay["slot"]
    tok = np.arange(wl.T * wl.k) // wl.k
    assert np.array_equal(recv[slot], inp["x"][tok])
    for e in range(wl.E):
        r0 = lay["expert_off"][e] + lay["cnt"][e]
        assert np.all(recv[r0:lay["expert_off"][e + 1]] == 0)
    assert np.all(recv[lay["rows"]:] == 0xFFFF)       # beyond R: untouched


def test_dispatch_bf16_weighted_copies():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl, with_y=False)
    lay = _layout_for(wl, inp)
    recv = oracle.combine_backward_bf16(lay, inp["x"], wl.k, inp["topk_w"])
    x32 = torch.from_numpy(bf16_bits_to_f32(inp["x"]))
    w = torch.from_numpy(inp["topk_w"])
    for j in range(wl.k):
        ref = (w[:, j:j + 1] * x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(recv[lay["slot"][j::wl.k]], ref)


def test_dispatch_fp8_rows():
    wl = WORKLOADS["decode"]
    inp = make_inputs(wl, with_y=False)
    lay = _layout_for(wl, inp)
    q, s = oracle.dispatch_fp8(lay, inp["x"], wl.k)
    nb = wl.H // 128
    s_ind, q_ind = independent_quantize(inp["x"].reshape(-1, 128))
    q_ind = q_ind.reshape(wl.T, wl.H)
    s_ind = s_ind.reshape(wl.T, nb)
    tok = np.arange(wl.T * wl.k) // wl.k
    assert np.array_equal(q[lay["slot"]], q_ind[tok])
    assert np.array_equal(s[lay["slot"]], s_ind[tok])


def test_dispatch_fp8_padding_and_prequant():
    wl = WORKLOADS["tiny"]
    wl = type(wl)(**{**wl.__dict__, "A": 8, "D": 4, "dispatch": "fp8"})
    inp = make_inputs(wl, with_y=False)
    lay = _layout_for(wl, inp)
    q, s = oracle.dispatch_fp8(lay, inp["x"], wl.k)
    for e in range(wl.E):
        r0, r1 = lay["expert_off"][e] + lay["cnt"][e], lay["expert_off"][e + 1]
        assert np.all(q[r0:r1] == 0) and np.all(s[r0:r1] == 0)
    # pre-quantised input: per-token codes/scales copied bitwise
    xq = np.zeros((wl.T, wl.H), np.uint8)
    xs = np.zeros((wl.T, wl.H // 128), np.float32)
    for t in range(wl.T):
        for b in range(wl.H // 128):
            xs[t, b], xq[t, b * 128:(b + 1) * 128] = oracle.quantize_block(inp["x"][t, b * 128:(b + 1) * 128])
    q2, s2 = oracle.dispatch_fp8_prequant(lay, xq, xs, wl.k)
    R = lay["rows"]
    assert np.array_equal(q2[:R], q[:R]) and np.array_equal(s2[:R], s[:R])


# ---------------------------------------------------------------- combine

def test_combine_golden_rounding_cases():
    """Fused multiply-add in k order (hand-derived, and checked here with
    exact rational arithmetic to discriminate the alternatives)."""
    with open(os.path.join(GOLDEN, "combine_rounding.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k = c["k"]
        w = np.array([int(b, 16) for b in c["w_bits"]], np.uint32).view(np.float32)[None, :]
        y = np.array([int(b, 16) for b in c["y_bits"]], np.uint16)[:, None]
        lay = {"slot": np.arange(k, dtype=np.int32)}
        out, _ = oracle.combine(lay, y, k, w)
        assert int(out[0, 0]) == int(c["expect_bits"], 16), c["name"]
        # the alternative reading really differs (exact arithmetic)
        yv = [Fraction(float(v)) for v in bf16_bits_to_f32(y[:, 0])]
        wv = [Fraction(float(v)) for v in w[0]]
        fused = Fraction(0)
        for j in range(k):
            fused = round_f32_exact(wv[j] * yv[j] + fused)
        unfused = Fraction(0)
        for j in range(k):
            unfused = round_f32_exact(round_f32_exact(wv[j] * yv[j]) + unfused)
        rev = Fraction(0)
        for j in reversed(range(k)):
            rev = round_f32_exact(wv[j] * yv[j] + rev)
        to_b = lambda fr: int(f32_to_bf16_bits(np.array([float(fr)], np.float32))[0])
        assert to_b(fused) == int(c["expect_bits"], 16)
        assert int(c["other_reading_bits"], 16) in (to_b(unfused), to_b(rev))


def test_combine_exact_model_random():
    """Random small combines against the exact rational model."""
    rng = np.random.default_rng(5)
    T, H, k = 6, 16, 4
    y = f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    slot = rng.permutation(T * k).astype(np.int32)
    slot[3] = -1
    lay = {"slot": slot}
    out, _ = oracle.combine(lay, y, k, w)
    yf = bf16_bits_to_f32(y)
    for t in range(T):
        for h in range(H):
            acc = Fraction(0)
            for j in range(k):
                s = slot[t * k + j]
                if s >= 0:
                    acc = round_f32_exact(Fraction(float(w[t, j])) * Fraction(float(yf[s, h])) + acc)
            assert out[t, h] == f32_to_bf16_bits(np.array([float(acc)], np.float32))[0]


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_identity_round_trip(name):
    """dispatch then identity experts then combine with softmax (unit-sum)
    weights reproduces x bit-exactly."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl, with_y=False)
    lay = _layout_for(wl, inp)
    recv = oracle.dispatch_bf16(lay, inp["x"], wl.k)
    out, _ = oracle.combine(lay, recv, wl.k, inp["topk_w"])
    # the sum starts at +0, so a -0 input comes back as +0
    assert np.array_equal(out, np.where(inp["x"] == 0x8000, 0, inp["x"]))


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_unweighted_dual_is_k_times_x(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl, with_y=False)
    lay = _layout_for(wl, inp)
    recv = oracle.dispatch_bf16(lay, inp["x"], wl.k)
    out, _ = oracle.dispatch_backward(lay, recv, wl.k)
    ref = f32_to_bf16_bits(np.float32(wl.k) * bf16_bits_to_f32(inp["x"]))
    assert np.array_equal(out, np.where(ref == 0x8000, 0, ref))


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_combine_against_torch_sum(name):
    """Against torch's float64 sum of the gathered, weighted rows: within the
    binary32 accumulation bound plus bfloat16 rounding everywhere, and within
    1 bf16 ulp of torch's float32 sum wherever there is no cancellation."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    lay = _layout_for(wl, inp)
    out, vals = oracle.combine(lay, inp["y"], wl.k, inp["topk_w"], row_vals=lay["row_w"])
    y = torch.from_numpy(bf16_bits_to_f32(inp["y"])).double()
    g = y[torch.from_numpy(lay["slot"].astype(np.int64))].view(wl.T, wl.k, wl.H)
    terms = torch.from_numpy(inp["topk_w"]).double()[..., None] * g
    ref = terms.sum(1).numpy()
    mag = terms.abs().sum(1).numpy()
    got = bf16_bits_to_f32(out).astype(np.float64)
    e_acc = wl.k * 2.0 ** -24 * mag
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * (np.abs(ref) + e_acc) + e_acc)
    ref32 = terms.float().sum(1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    clear = np.abs(ref) >= 0.5 * mag
    assert bf16_ulp_distance(out, ref32)[clear].max() <= 1
    # gather of per-row values back to pairs returns the pair weights
    assert np.array_equal(vals, inp["topk_w"])


def test_combine_masked_pairs_and_fp8_identity():
    """Masked pairs contribute nothing; FP8 round trip: combining the
    dequantised rows with one expert per token gives bf16(q * scale)."""
    rng = np.random.default_rng(9)
    T, E, k, H = 20, 6, 2, 256
    idx = random_routing_table(rng, T, E, k, masked_frac=0.3)
    w = rng.random((T, k)).astype(np.float32)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = oracle.layout(0, T, E, k, 4, 1, 0, idx, w)
    recv = oracle.dispatch_bf16(lay, x, k)
    out, _ = oracle.combine(lay, recv, k, w)
    x32 = bf16_bits_to_f32(x)
    for t in range(T):
        live = [j for j in range(k) if idx[t, j] >= 0]
        if not live:
            assert np.all(out[t] == 0)
        if len(live) == 1:
            j = live[0]
            ref = f32_to_bf16_bits((w[t, j] * x32[t]).astype(np.float32))
            assert np.array_equal(out[t], np.where(ref == 0x8000, 0, ref))
    q, s = oracle.dispatch_fp8(lay, x, k)
    vals = torch_e4m3_values()
    R = lay["rows"]
    deq = (vals[q[:R] & 0x7F] * np.where(q[:R] & 0x80, -1.0, 1.0)).reshape(R, H // 128, 128)
    deq = (deq * s[:R, :, None].astype(np.float64)).reshape(R, H).astype(np.float32)
    yq = f32_to_bf16_bits(deq)
    one = np.ones((T, k), np.float32)
    idx1 = idx.copy()
    idx1[:, 1] = -1
    lay1 = oracle.layout(0, T, E, k, 4, 1, 0, idx1, one)
    q1, s1 = oracle.dispatch_fp8(lay1, x, k)
    R1 = lay1["rows"]
    deq1 = (vals[q1[:R1] & 0x7F] * np.where(q1[:R1] & 0x80, -1.0, 1.0)).reshape(R1, H // 128, 128)
    deq1 = (deq1 * s1[:R1, :, None].astype(np.float64)).reshape(R1, H).astype(np.float32)
    out1, _ = oracle.combine(lay1, f32_to_bf16_bits(deq1), k, one)
    for t in range(T):
        if idx1[t, 0] >= 0:
            ref = f32_to_bf16_bits(deq1[lay1["slot"][t * k]])
            assert np.array_equal(out1[t], np.where(ref == 0x8000, 0, ref))
        else:
            assert np.all(out1[t] == 0)
    assert yq.shape == (R, H)


# ---------------------------------------------------------------- combine weight gradient

def test_weight_grad_exact_integers():
    """Integer-valued bf16 gradients and expert outputs: every product and
    partial sum is an exact small integer, so the oracle must equal the dot
    product taken with Python integers over the row that holds each pair,
    found by brute force (the row whose row_src is the pair index)."""
    rng = np.random.default_rng(31)
    for T, E, k, A, H, masked in [(9, 5, 2, 3, 40, 0.0), (30, 8, 3, 1, 64, 0.2), (17, 4, 4, 2, 8, 0.1)]:
        idx = random_routing_table(rng, T, E, k, masked_frac=masked, distinct=False)
        lay = oracle.layout(0, T, E, k, A, 1, 0, idx)
        R = lay["rows_bound"]
        gi = rng.integers(-16, 17, size=(T, H))
        yi = rng.integers(-16, 17, size=(R, H))
        g = f32_to_bf16_bits(gi.astype(np.float32))
        y = f32_to_bf16_bits(yi.astype(np.float32))
        got = oracle.combine_weight_grad(lay, g, y, k)
        for t in range(T):
            for j in range(k):
                rows = [r for r in range(lay["rows"]) if lay["row_src"][r] == t * k + j]
                assert len(rows) == (1 if idx[t, j] >= 0 else 0)
                want = sum(int(a) * int(b) for a, b in zip(gi[t], yi[rows[0]])) if rows else 0
                assert got[t, j] == want, (t, j)


def test_weight_grad_closed_forms():
    """Constant rows give H * a * b exactly; pairs past a FIXED capacity get 0;
    with expert outputs equal to the dispatched x (identity experts) every
    pair of token t gets <g_t, x_t>, checked against math.fsum of the exact
    binary64 products within the binary64 bound of an H-term sum."""
    import math
    T, E, k, H = 12, 4, 2, 384
    rng = np.random.default_rng(32)
    idx = random_routing_table(rng, T, E, k)
    lay = oracle.layout(0, T, E, k, 1, 1, 0, idx)
    g = np.full((T, H), f32_to_bf16_bits(np.array([0.75], np.float32))[0], np.uint16)
    y = np.full((lay["rows_bound"], H), f32_to_bf16_bits(np.array([-1.5], np.float32))[0], np.uint16)
    assert np.all(oracle.combine_weight_grad(lay, g, y, k) == H * 0.75 * -1.5)
    # FIXED capacity 2: the pairs past it are skipped and get 0
    idx_f = np.zeros((T, k), np.int64)
    idx_f[:, 1] = 1
    lay_f = oracle.layout(1, T, E, k, 1, 1, 2, idx_f)
    y_f = np.full((lay_f["rows_bound"], H), y[0, 0], np.uint16)
    got = oracle.combine_weight_grad(lay_f, g, y_f, k)
    assert np.all(got[:2] == H * 0.75 * -1.5) and np.all(got[2:] == 0.0)
    # identity experts
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gr = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    recv = oracle.dispatch_bf16(lay, x, k)
    got = oracle.combine_weight_grad(lay, gr, recv, k)
    x64 = bf16_bits_to_f32(x).astype(np.float64)
    g64 = bf16_bits_to_f32(gr).astype(np.float64)
    for t in range(T):
        terms = [a * b for a, b in zip(g64[t], x64[t])]
        exact = math.fsum(terms)
        bound = H * 2.0 ** -53 * math.fsum(abs(v) for v in terms)
        assert np.all(np.abs(got[t] - exact) <= bound)


def test_combine_backward_fp8_weighted():
    """Weighted FP8 combine_backward: per pair, the codes dequantise to the
    weighted BF16 gradient within the E4M3 bound (checked in binary64 against
    w * g computed from torch's bf16 cast, not the oracle's); the block's
    largest element maps to 448 (0x7E); a zero weight gives zero codes and
    scale 0; pairs of one token with different weights get different scales;
    padding rows are zero."""
    rng = np.random.default_rng(33)
    T, E, k, A, H = 40, 6, 3, 8, 256
    idx = random_routing_table(rng, T, E, k)
    w = rng.random((T, k)).astype(np.float32) + 0.25
    w[0, 1] = 0.0
    g = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = oracle.layout(0, T, E, k, A, 1, 0, idx, w)
    q, s = oracle.combine_backward_fp8(lay, g, k, w)
    vals = torch_e4m3_values()
    g32 = torch.from_numpy(bf16_bits_to_f32(g))
    for t in range(T):
        for j in range(k):
            r = lay["slot"][t * k + j]
            ref = (g32[t] * float(w[t, j])).to(torch.bfloat16).to(torch.float64).numpy()   # bf16(w * g)
            codes = q[r]
            deq = vals[codes & 0x7F] * np.where(codes & 0x80, -1.0, 1.0)
            deq = (deq.reshape(-1, 128) * s[r][:, None].astype(np.float64)).ravel()
            blocks = np.abs(ref).reshape(-1, 128)
            scale = blocks.max(1) / 448.0
            err = np.abs(deq - ref).reshape(-1, 128)
            lim = np.maximum(2.0 ** -4 * np.abs(ref).reshape(-1, 128), 2.0 ** -10 * scale[:, None]) * (1 + 2.0 ** -20)
            assert np.all(err <= lim), (t, j)
            # exact: the pinned block quantiser applied to torch's bf16(w * g)
            ref_bits = f32_to_bf16_bits(ref.astype(np.float32))
            for b in range(H // 128):
                sc, qb = oracle.quantize_block(ref_bits[b * 128:(b + 1) * 128])
                assert np.array_equal(codes[b * 128:(b + 1) * 128], qb) and s[r][b] == sc, (t, j, b)
            if w[t, j] == 0.0:
                assert np.all(codes == 0) and np.all(s[r] == 0.0)
            else:
                assert np.all(np.any((codes.reshape(-1, 128) & 0x7F) == 0x7E, axis=1))
    t = 5
    rows = lay["slot"][t * k: t * k + k]
    assert len({float(s[r][0]) for r in rows}) == k
    R = lay["rows"]
    pad_rows = [r for r in range(R) if lay["row_src"][r] < 0]
    assert pad_rows and np.all(q[pad_rows] == 0) and np.all(s[pad_rows] == 0.0)
