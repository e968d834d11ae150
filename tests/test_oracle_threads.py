"""The oracle's OpenMP timing build returns the same bits as its plain build.

The benchmark times the CPU oracle on several host cores through a second
build of ep_oracle.c (-fopenmp, work-sharing over tokens). That build must be
the same function: every output of every entry point is compared bit for bit
with the plain single-threaded build, at the tiny and mid workload shapes
(all tokens) and on a small FP8 case.
"""
import numpy as np
import pytest

import oracle
from ep_workloads import WORKLOADS, make_inputs, draw_expert_out, _streams


@pytest.fixture(autouse=True)
def _plain_after():
    yield
    oracle.threads(0)


def _run_all(wl, inp, y, g, fp8: bool):
    lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, inp["topk_idx"], inp["topk_w"])
    out = {"slot": lay["slot"].copy()}
    out["recv_bf16"] = oracle.dispatch_bf16(lay, inp["x"], wl.k)
    out["cb_bf16"] = oracle.combine_backward_bf16(lay, g, wl.k, inp["topk_w"])
    out["comb"], _ = oracle.combine(lay, y, wl.k, inp["topk_w"])
    rv = np.arange(y.shape[0], dtype=np.float32)
    out["db"], out["db_vals"] = oracle.dispatch_backward(lay, y, wl.k, rv)
    out["wg"] = oracle.combine_weight_grad(lay, g, y, wl.k)
    if fp8:
        q, s = oracle.dispatch_fp8(lay, inp["x"], wl.k)
        out["fp8_q"], out["fp8_s"] = q, s
        q2, s2 = oracle.dispatch_fp8_prequant(lay, q[: wl.T], s[: wl.T], wl.k)
        out["pre_q"], out["pre_s"] = q2, s2
        q3, s3 = oracle.combine_backward_fp8(lay, g, wl.k, inp["topk_w"])
        out["cbf8_q"], out["cbf8_s"] = q3, s3
    return out


def _same(a: dict, b: dict):
    assert a.keys() == b.keys()
    for key in a:
        x, z = np.asarray(a[key]), np.asarray(b[key])
        assert x.dtype == z.dtype and x.shape == z.shape, key
        # bit patterns (NaN fill values compare equal as bits)
        assert np.array_equal(x.view(np.uint8), z.view(np.uint8)), key


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_threaded_build_same_bits(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl, with_y=False)
    R = oracle.rows_bound(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.C)
    _, _, _, _, sy = _streams(0)
    y = draw_expert_out(wl, sy, R)
    g = draw_expert_out(wl, np.random.default_rng(11), wl.T)
    plain = _run_all(wl, inp, y, g, fp8=wl.H % 128 == 0)
    n = oracle.threads(4)
    assert n == 4
    threaded = _run_all(wl, inp, y, g, fp8=wl.H % 128 == 0)
    _same(plain, threaded)


def test_thread_count_switch():
    assert oracle.threads(0) == 1
    assert oracle.threads(3) == 3
    assert oracle.threads(0) == 1
