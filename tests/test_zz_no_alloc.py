"""ep_dispatch_forward_static_scratch (the layout's per-block partials in a
library-held device array, for callers that cannot allocate) against
ep_dispatch_forward, both through the C ABI, on consecutive calls that
share the array: a large batch (multi-block layout, partials in the array),
then a smaller one, then a single-launch batch. Handle arrays, receive rows
and scales must be bit-identical, and the layout equal to the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from ep_workloads import random_routing_table, f32_to_bf16_bits
from gpu_common import log, to_dev, to_dev_bf16, host, compare_layout

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from combine_ep_layout_10_amd import _ffi as F
    from combine_ep_layout_10_amd import ops


def _call(fn_name, cfg, idx, w, x, ws, recv, rs):
    lib = F.lib()
    c = cfg.c()
    hc = F.ep_handle()
    st = getattr(lib, fn_name)(ctypes.byref(c), int(idx.shape[0]), idx.data_ptr(), w.data_ptr(), ws.data_ptr(),
                               ws.numel(), ops.FP8_QUANTIZE, x.data_ptr(), None, recv.data_ptr(), rs.data_ptr(),
                               ctypes.byref(hc), torch.cuda.current_stream().cuda_stream)
    assert st == F.EP_OK, (fn_name, F.status_string(st), F.last_error_message())
    torch.cuda.synchronize()
    return ops.Handle(cfg, hc, ws, idx)


def _case(T, seed, cfg, ws_a, ws_b):
    H, E, k, A, D = cfg.hidden, cfg.num_experts, cfg.num_topk, cfg.expert_alignment, cfg.num_dests
    log("static scratch: T=%d E=%d k=%d A=%d H=%d" % (T, E, k, A, H))
    rng = np.random.default_rng(seed)
    idx_h = random_routing_table(rng, T, E, k)
    w_h = rng.random((T, k)).astype(np.float32)
    x = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    idx, w = to_dev(idx_h), to_dev(w_h)
    R = cfg.recv_rows_bound()
    outs = []
    for fn, ws in (("ep_dispatch_forward", ws_a), ("ep_dispatch_forward_static_scratch", ws_b)):
        recv = torch.full((R, H), 0xEE, dtype=torch.uint8, device="cuda")
        rs = torch.full((R, H // 128), -7.0, dtype=torch.float32, device="cuda")
        outs.append((_call(fn, cfg, idx, w, x, ws, recv, rs), recv, rs))
    (ha, ra, sa), (hb, rb, sb) = outs
    lay = oracle.layout(0, T, E, k, A, D, 0, idx_h, w_h)
    compare_layout(hb, lay)
    rows = int(lay["rows"])
    for key in ("cnt", "pad", "expert_off", "dest_off", "dest_tokens", "slot", "err_flags"):
        assert np.array_equal(host(getattr(ha, key)), host(getattr(hb, key))), key
    assert np.array_equal(host(ha.row_src)[:rows], host(hb.row_src)[:rows])
    assert np.array_equal(host(ha.row_w)[:rows].view(np.uint32), host(hb.row_w)[:rows].view(np.uint32))
    assert np.array_equal(host(ra)[:rows], host(rb)[:rows])
    assert np.array_equal(host(sa)[:rows].view(np.uint32), host(sb)[:rows].view(np.uint32))
    assert np.all(host(rb)[rows:] == 0xEE)


def test_static_scratch_matches_dispatch_forward():
    cfg = ops.Config(max_tokens=3000, hidden=512, num_experts=256, num_topk=8, num_dests=8, expert_alignment=128)
    ws_a = ops.new_workspace(cfg)
    ws_b = ops.new_workspace(cfg)
    _case(3000, 61, cfg, ws_a, ws_b)     # 24,000 pairs: 24 layout blocks, partials in the static array
    _case(1100, 62, cfg, ws_a, ws_b)     # smaller: 9 blocks read only what this call wrote
    _case(300, 63, cfg, ws_a, ws_b)      # 2,400 pairs: the single launch (no partials)
    _case(2000, 64, cfg, ws_a, ws_b)     # larger again after the small ones


def test_static_scratch_graph_replay():
    """The entry point captured in a HIP graph (the use it exists for) at a
    multi-block layout, whose partials live in the static array: three
    replays, with new routing, weights and x copied in and eager calls of
    ep_dispatch_forward between them, each bit-identical to the eager result
    and its slots equal to the oracle's."""
    T, H, E, k, A, D = 3000, 512, 256, 8, 128, 8
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, num_dests=D, expert_alignment=A)
    R = cfg.recv_rows_bound()
    idx_s = torch.zeros((T, k), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    recv_s = torch.empty((R, H), dtype=torch.uint8, device="cuda")
    rs_s = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
    ws_g, ws_e = ops.new_workspace(cfg), ops.new_workspace(cfg)
    c = cfg.c()
    hc = F.ep_handle()

    def launch():
        st = F.lib().ep_dispatch_forward_static_scratch(
            ctypes.byref(c), T, idx_s.data_ptr(), w_s.data_ptr(), ws_g.data_ptr(), ws_g.numel(), ops.FP8_QUANTIZE,
            x_s.data_ptr(), None, recv_s.data_ptr(), rs_s.data_ptr(), ctypes.byref(hc),
            torch.cuda.current_stream().cuda_stream)
        assert st == F.EP_OK, (F.status_string(st), F.last_error_message())

    rng = np.random.default_rng(65)
    idx_s.copy_(to_dev(random_routing_table(rng, T, E, k)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    hg = ops.Handle(cfg, hc, ws_g, idx_s)
    for rep in range(3):
        log("static scratch graph replay %d" % rep)
        idx_h = random_routing_table(rng, T, E, k)
        w_h = rng.random((T, k)).astype(np.float32)
        x_h = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        idx_s.copy_(to_dev(idx_h))
        w_s.copy_(to_dev(w_h))
        x_s.copy_(to_dev_bf16(x_h))
        recv_s.fill_(0xEE)
        g.replay()
        torch.cuda.synchronize()
        lay = oracle.layout(0, T, E, k, A, D, 0, idx_h, w_h)
        compare_layout(hg, lay)
        rows = int(lay["rows"])
        recv_e = torch.full((R, H), 0xEE, dtype=torch.uint8, device="cuda")
        rs_e = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
        he = _call("ep_dispatch_forward", cfg, idx_s, w_s, x_s, ws_e, recv_e, rs_e)
        for key in ("cnt", "pad", "expert_off", "dest_off", "dest_tokens", "slot", "err_flags"):
            assert np.array_equal(host(getattr(hg, key)), host(getattr(he, key))), (rep, key)
        assert np.array_equal(host(recv_s)[:rows], host(recv_e)[:rows]), rep
        assert np.array_equal(host(rs_s)[:rows].view(np.uint32), host(rs_e)[:rows].view(np.uint32)), rep
        assert np.all(host(recv_s)[rows:] == 0xEE), rep
