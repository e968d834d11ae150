"""The compiled torch binding's argument checks: a tensor on the wrong
device, of the wrong dtype or shape, or not contiguous is refused with
ValueError before any C call, so nothing is enqueued and the caller's
buffers keep their contents; C-level errors surface as RuntimeError with
the library's message."""
import numpy as np
import pytest
import torch

from ep_workloads import random_routing_table, f32_to_bf16_bits
from gpu_common import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from combine_ep_layout_10_amd import ops


def _setup():
    T, H, E, k = 96, 256, 16, 4
    rng = np.random.default_rng(71)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=8)
    idx = to_dev(random_routing_table(rng, T, E, k))
    w = to_dev(rng.random((T, k)).astype(np.float32))
    x = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    return cfg, idx, w, x


def test_dispatch_arguments_refused_before_any_work():
    cfg, idx, w, x = _setup()
    T, H = x.shape
    h = ops.layout(cfg, idx, w)
    R = cfg.recv_rows_bound()
    recv = torch.full((R, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    bad_x = [x.float(),                                          # dtype
             x[:, :H - 8].contiguous(),                          # shape
             torch.cat([x, x], 1)[:, ::2],                       # not contiguous
             x.cpu()]                                            # device
    for bx in bad_x:
        with pytest.raises(ValueError):
            ops.dispatch(h, bx, ops.BF16, recv=recv)
    with pytest.raises(ValueError):
        ops.dispatch(h, x, ops.BF16, recv=recv[:R - 1])          # receive buffer one row short
    with pytest.raises(ValueError):
        ops.dispatch(h, x, ops.FP8_QUANTIZE, recv=torch.empty((R, H), dtype=torch.uint8, device="cuda"),
                     recv_scales=torch.empty((R, H // 128 + 1), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((recv.view(torch.int16) == -1).all())           # nothing was written


def test_combine_and_backward_arguments_refused():
    cfg, idx, w, x = _setup()
    T, H = x.shape
    h = ops.layout(cfg, idx, w)
    R = cfg.recv_rows_bound()
    y = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    with pytest.raises(ValueError):
        ops.combine(h, y[:R - 1], w, out=out)                    # y one row short
    with pytest.raises(ValueError):
        ops.combine(h, y, w[:, :2].contiguous(), out=out)        # weights [T, 2] for top-4
    with pytest.raises(ValueError):
        ops.combine(h, y, w.double(), out=out)                   # weights not binary32
    with pytest.raises(ValueError):
        ops.combine_backward(h, x[:T - 1].contiguous(), ops.BF16, w)
    with pytest.raises(ValueError):
        ops.dispatch_backward(h, y.float())
    torch.cuda.synchronize()
    assert bool((out.view(torch.int16) == -1).all())


def test_library_errors_are_runtime_errors():
    cfg, idx, w, x = _setup()
    h = ops.layout(cfg, idx, w)
    codes = torch.zeros(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.ones((x.shape[0], x.shape[1] // 128), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="weighted combine_backward"):
        ops.combine_backward(h, codes, ops.FP8_PREQUANT, w, grad_out_scales=scales)
    with pytest.raises(RuntimeError, match="grad_out_scales"):
        ops.combine_backward(h, codes, ops.FP8_PREQUANT)
