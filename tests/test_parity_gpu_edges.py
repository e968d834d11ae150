"""GPU parity at the edges of the launch paths, through the C ABI against
the CPU oracle: FP8 rows wider than one pass of a block, the pre-quantised
passthrough at the 8192 x 7168 x top-8 shape, results independent of the
launch geometry, the handle's topk_idx, and the launch-geometry report."""
import numpy as np
import pytest
import torch

import oracle
from ep_workloads import WORKLOADS, make_inputs, random_routing_table, f32_to_bf16_bits
from gpu_common import log, to_dev, to_dev_bf16, bf16_host, host, cfg_of, compare_layout

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from combine_ep_layout_10_amd import ops
    from test_parity_gpu import _run_small


def test_fp8_rows_wider_than_one_block_pass():
    """H = 16512: 1032 vectors of 16 values per FP8 row, so every lane loop
    over a row (dispatch, the zero-fill, the weighted FP8 backward and its
    DPP amax groups) takes a second pass over the last 8 vectors."""
    _run_small(70, 16512, 24, 6, A=4, D=4, seed=51, dispatch="fp8")
    _run_small(70, 16512, 24, 6, A=4, D=4, seed=52, dispatch="fp8", forward=True, masked=0.1)
    rng = np.random.default_rng(53)
    T, H, E, k, A = 50, 16512, 16, 4, 8
    idx = random_routing_table(rng, T, E, k)
    w = (rng.standard_normal((T, k)) * 2).astype(np.float32)
    g = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = oracle.layout(0, T, E, k, A, 1, 0, idx, w)
    q, s = oracle.combine_backward_fp8(lay, g, k, w)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A)
    h = ops.layout(cfg, to_dev(idx), to_dev(w))
    gq, gs = ops.combine_backward(h, to_dev_bf16(g), ops.FP8_QUANTIZE, to_dev(w))
    rows = np.arange(lay["rows"])
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))


def test_prequant_passthrough_v3_shape():
    """(codes, scales) given as x at 8192 x 7168, 256 experts, top-8,
    alignment 128, 8 destinations: every code byte (NaN patterns included)
    and scale copied bitwise, through ep_dispatch and ep_dispatch_forward."""
    wl = WORKLOADS["v3"]
    inp = make_inputs(wl, with_y=False)
    rng = np.random.default_rng(54)
    xq = rng.integers(0, 256, size=(wl.T, wl.H), dtype=np.uint8)
    xs = rng.standard_normal((wl.T, wl.H // 128)).astype(np.float32)
    lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, inp["topk_idx"], inp["topk_w"])
    q, s = oracle.dispatch_fp8_prequant(lay, xq, xs, wl.k)
    rows = np.arange(lay["rows"])
    cfg = cfg_of(wl)
    dq, ds = to_dev(xq), to_dev(xs)
    log("prequant passthrough v3: ep_dispatch")
    h = ops.layout(cfg, to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
    gq, gs = ops.dispatch(h, dq, ops.FP8_PREQUANT, x_scales=ds)
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))
    log("prequant passthrough v3: ep_dispatch_forward")
    h2, gq2, gs2 = ops.dispatch_forward(cfg, to_dev(inp["topk_idx"]), dq, ops.FP8_PREQUANT,
                                        topk_w=to_dev(inp["topk_w"]), x_scales=ds)
    compare_layout(h2, lay)
    assert np.array_equal(host(gq2)[rows], q[rows])
    assert np.array_equal(host(gs2)[rows].view(np.uint32), s[rows].view(np.uint32))


def _geometry_outputs():
    """Every call whose grid depends on the CU count, on fixed inputs: the
    aligned FP8 dispatch and weighted BF16 combine_backward (zero-fill
    blocks capped per CU), the single-launch decode dispatch (row pieces per
    CU) and a small-batch combine (row pieces per CU)."""
    out = {}
    rng = np.random.default_rng(55)
    T, H, E, k, A, D = 700, 1024, 64, 6, 32, 4
    idx = random_routing_table(rng, T, E, k)
    w = rng.random((T, k)).astype(np.float32)
    x = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, num_dests=D, expert_alignment=A)
    h = ops.layout(cfg, to_dev(idx), to_dev(w))
    rows = int(h.read_counts()[2])          # rows from expert_off[E] on are never written
    q, s = ops.dispatch(h, x, ops.FP8_QUANTIZE)
    out["fp8"], out["fp8_scales"] = host(q)[:rows], host(s)[:rows].view(np.uint32)
    out["cb"] = bf16_host(ops.combine_backward(h, x, ops.BF16, to_dev(w)))[:rows]
    R = cfg.recv_rows_bound()
    y = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32)))
    out["comb"] = bf16_host(ops.combine(h, y, to_dev(w)))
    out["rows"] = rows
    wl = WORKLOADS["decode"]
    inp = make_inputs(wl, with_y=False)
    dcfg = cfg_of(wl)
    hd, dq, dsc = ops.dispatch_forward(dcfg, to_dev(inp["topk_idx"]), to_dev_bf16(inp["x"]), ops.FP8_QUANTIZE,
                                       topk_w=to_dev(inp["topk_w"]))
    lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, inp["topk_idx"], inp["topk_w"])
    drows = np.concatenate([lay["expert_off"][e] + np.arange(lay["pad"][e]) for e in range(wl.E)])
    out["dec"], out["dec_scales"] = host(dq)[drows], host(dsc)[drows].view(np.uint32)
    yd = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((dcfg.recv_rows_bound(), wl.H)).astype(np.float32)))
    out["dec_comb"] = bf16_host(ops.combine(hd, yd, to_dev(inp["topk_w"])))
    return out


def test_results_independent_of_launch_geometry(monkeypatch):
    monkeypatch.delenv("EP_LAUNCH_CUS", raising=False)
    ref = _geometry_outputs()
    for cus in (1, 3, 37, 255, 1024):
        log("launch geometry as for %d CUs" % cus)
        monkeypatch.setenv("EP_LAUNCH_CUS", str(cus))
        got = _geometry_outputs()
        for key in ref:
            assert np.array_equal(np.asarray(got[key]), np.asarray(ref[key])), (cus, key)


def test_handle_topk_idx():
    """The handle keeps the caller's topk_idx (README decode example:
    cached_handle.topk_idx), on every path that builds a layout."""
    cfg = ops.Config(max_tokens=64, hidden=256, num_experts=16, num_topk=2)
    rng = np.random.default_rng(56)
    idx = to_dev(random_routing_table(rng, 64, 16, 2))
    x = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((64, 256)).astype(np.float32)))
    h = ops.layout(cfg, idx)
    assert h.topk_idx is idx and h.c.topk_idx == idx.data_ptr()
    h2, _ = ops.dispatch_forward(cfg, idx, x)
    assert h2.topk_idx is idx and h2.c.topk_idx == idx.data_ptr()
    recv = torch.empty((cfg.recv_rows_bound(), 256), dtype=torch.bfloat16, device="cuda")
    call, h3 = ops.bind_dispatch_forward(cfg, idx, x, ops.BF16, recv)
    call()
    assert h3.topk_idx is idx and h3.c.topk_idx == idx.data_ptr()
    h0 = ops.layout(cfg, idx[:0])
    assert not h0.c.topk_idx
    torch.cuda.synchronize()


def test_buffer_debug_reports_geometry(monkeypatch, capfd):
    """EP_BUFFER_DEBUG=1 prints each launch's geometry; the zero-fill block
    count follows EP_LAUNCH_CUS (at most 8 per CU)."""
    rng = np.random.default_rng(57)
    T, H, E, k, A = 300, 512, 32, 4, 16
    idx = random_routing_table(rng, T, E, k)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A)
    x = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    monkeypatch.setenv("EP_BUFFER_DEBUG", "1")
    monkeypatch.setenv("EP_LAUNCH_CUS", "2")
    h = ops.layout(cfg, to_dev(idx))
    ops.dispatch(h, x)
    y = torch.zeros((cfg.recv_rows_bound(), H), dtype=torch.bfloat16, device="cuda")
    ops.combine(h, y)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("[ep] ")]
    kernels = [l.split()[1] for l in lines]
    assert "k_layout_small" in kernels and "k_dispatch" in kernels and "k_combine<false>" in kernels, err
    disp = [l for l in lines if l.split()[1] == "k_dispatch"][0]
    assert "zero-fill blocks 16 " in disp, disp          # min(pieces, 8 blocks per CU x 2 CUs)
    monkeypatch.setenv("EP_BUFFER_DEBUG", "0")
    ops.dispatch(h, x)
    torch.cuda.synchronize()
    assert "[ep] " not in capfd.readouterr().err
