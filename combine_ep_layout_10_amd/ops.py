"""Torch-facing calls over the C ABI: PyTorch supplies device memory and the
stream, every step runs in the HIP kernels behind include/ep.h.

Mapping to the DeepEP README ("Interfaces and examples"):
  layout + dispatch            -> dispatch_forward (recv_x, handle)
  dispatch_forward             -> the same in one call (one launch for small batches)
  Handle.row_src / row_w       -> recv_topk_idx / recv_topk_weights (per row)
  Handle.pad (read_counts)     -> handle.num_recv_tokens_per_expert_list
  combine                      -> combine_forward
  dispatch_backward            -> dispatch_backward (a combine)
  combine_backward             -> combine_backward (a dispatch on the handle)
  combine_weight_grad          -> the weight gradient of the weighted combine
  grouped_gemm_fp8             -> the expert GEMM the layout is built for
  dispatch with an old Handle  -> decode_dispatch with cached_handle
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

from . import _ffi as F

_TORCH_EXT = __import__("os").path.join(__import__("os").path.dirname(__file__), "_ep_torch.so")


def _load_binding():
    """The compiled binding (_ep_torch.so, built beside libep.so): the tensor
    checks and the C calls of the hot entry points. Raises if it has not
    been built; there is no other path."""
    import importlib.util
    import os
    if not os.path.exists(_TORCH_EXT):
        raise ImportError("_ep_torch.so not found at %s: build it with `python -m combine_ep_layout_10_amd.build`"
                          % _TORCH_EXT)
    F.lib()  # libep.so first, through ctypes: the binding links the same file
    spec = importlib.util.spec_from_file_location(__package__ + "._ep_torch", _TORCH_EXT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_B = _load_binding()

MODE_COMPACT = F.EP_MODE_COMPACT
MODE_FIXED = F.EP_MODE_FIXED
BF16 = F.EP_BF16
FP8_QUANTIZE = F.EP_FP8_QUANTIZE
FP8_PREQUANT = F.EP_FP8_PREQUANT
FLAG_NO_ZERO_PAD = F.EP_FLAG_NO_ZERO_PAD


@dataclasses.dataclass(frozen=True)
class Config:
    max_tokens: int
    hidden: int
    num_experts: int
    num_topk: int
    num_dests: int = 1
    expert_alignment: int = 1
    capacity: int = 0
    mode: int = MODE_COMPACT
    idx_bits: int = 64
    flags: int = 0

    def c(self) -> F.ep_config:
        """The C struct, built once per Config (cached on the instance)."""
        c = self.__dict__.get("_c_struct")
        if c is None:
            c = F.ep_config(self.max_tokens, self.hidden, self.num_experts, self.num_topk, self.num_dests,
                            self.expert_alignment, self.capacity, self.mode, self.idx_bits, self.flags)
            object.__setattr__(self, "_c_struct", c)
            object.__setattr__(self, "_c_addr", ctypes.addressof(c))
        return c

    def c_addr(self) -> int:
        """Address of the cached C struct (the compiled binding reads it)."""
        a = self.__dict__.get("_c_addr")
        if a is None:
            self.c()
            a = self.__dict__["_c_addr"]
        return a

    def workspace_bytes(self) -> int:
        n = F.ep_workspace_bytes(self.c())
        if n == 0:
            raise F.EPError(F.EP_ERR_INVALID_ARG, "ep_workspace_bytes", F.last_error_message())
        return n

    def recv_rows_bound(self) -> int:
        n = self.__dict__.get("_rows_bound")
        if n is None:
            n = F.ep_recv_rows_bound(self.c())
            if n < 0:
                raise F.EPError(F.EP_ERR_INVALID_ARG, "ep_recv_rows_bound", F.last_error_message())
            object.__setattr__(self, "_rows_bound", n)
        return n


_current_device = torch.cuda.current_device
_raw_stream = torch._C._cuda_getCurrentRawStream


def _stream(cur: Optional[int] = None) -> int:
    return _raw_stream(_current_device() if cur is None else cur)


def _bad_tensor(t, name: str, dtype, cur: int) -> ValueError:
    """The error for a tensor _dev refused (built only on failure)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        return ValueError("%s must be a device tensor" % name)
    if t.get_device() != cur:
        # kernels run on the current device's stream
        return ValueError("%s is on %s, not on the current device cuda:%d" % (name, t.device, cur))
    if not t.is_contiguous():
        return ValueError("%s must be contiguous" % name)
    return ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _dev(t: torch.Tensor, name: str, dtype=None, cur: Optional[int] = None) -> int:
    """Device pointer of a contiguous tensor on the current device (cur: that
    device's index, when the caller already has it), of the given dtype (one
    dtype, or a tuple of them; torch dtypes are singletons, so identity
    decides)."""
    if cur is None:
        cur = _current_device()
    try:
        dt = t.dtype
        ok = (dtype is None or dt is dtype or (type(dtype) is tuple and dt in dtype)) and \
            t.get_device() == cur and t.is_contiguous()
    except AttributeError:
        ok = False
    if not ok:
        raise _bad_tensor(t, name, dtype, cur)
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor], name: str, dtype=None, cur: Optional[int] = None):
    return None if t is None else _dev(t, name, dtype, cur)


def _need(t: Optional[torch.Tensor], shape, name: str) -> None:
    """The kernels index these buffers by the handle's sizes: check them here."""
    if t is not None and t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class Handle:
    """An ep_handle plus the workspace tensor it points into and the topk_idx
    tensor the layout was built from (README "Example use in inference
    decoding": a cached handle hands back its topk_idx)."""

    __slots__ = ("cfg", "c", "workspace", "_topk_idx")

    def __init__(self, cfg: Config, h: F.ep_handle, workspace: torch.Tensor,
                 topk_idx: Optional[torch.Tensor] = None):
        self.cfg = cfg
        self.c = h
        self.workspace = workspace
        self._topk_idx = topk_idx

    @property
    def topk_idx(self) -> Optional[torch.Tensor]:
        """The [T, k] routing tensor of this layout (the caller's tensor, not
        a copy; ep_handle.topk_idx points at it)."""
        return self._topk_idx

    @property
    def num_tokens(self) -> int:
        return int(self.c.num_tokens)

    def _view(self, ptr: int, n: int, dtype) -> torch.Tensor:
        off = ptr - self.workspace.data_ptr()
        itemsize = torch.empty((), dtype=dtype).element_size()
        return self.workspace[off: off + n * itemsize].view(dtype)

    @property
    def cnt(self):
        return self._view(self.c.cnt, self.cfg.num_experts, torch.int32)

    @property
    def pad(self):
        return self._view(self.c.pad, self.cfg.num_experts, torch.int32)

    @property
    def expert_off(self):
        return self._view(self.c.expert_off, self.cfg.num_experts + 1, torch.int32)

    @property
    def dest_off(self):
        return self._view(self.c.dest_off, self.cfg.num_dests + 1, torch.int32)

    @property
    def dest_tokens(self):
        return self._view(self.c.dest_tokens, self.cfg.num_dests, torch.int32)

    @property
    def slot(self):
        return self._view(self.c.slot, self.num_tokens * self.cfg.num_topk, torch.int32)

    @property
    def row_src(self):
        return self._view(self.c.row_src, self.cfg.recv_rows_bound(), torch.int32)

    @property
    def row_w(self):
        return self._view(self.c.row_w, self.cfg.recv_rows_bound(), torch.float32)

    @property
    def err_flags(self):
        return self._view(self.c.err_flags, 1, torch.int32)

    def read_counts(self) -> Tuple[np.ndarray, np.ndarray, int]:
        """cnt, pad and the row total on the host (synchronises the stream)."""
        E = self.cfg.num_experts
        cnt = np.zeros(E, np.int32)
        pad = np.zeros(E, np.int32)
        rows = np.zeros(1, np.int64)
        F.ep_handle_read_counts(self.c, cnt.ctypes.data, pad.ctypes.data, rows.ctypes.data, _stream())
        return cnt, pad, int(rows[0])

    def check(self) -> int:
        """EP_ERRFLAG_* bits of the layout (synchronises the stream)."""
        return F.ep_handle_check(self.c, _stream())


def _c_config(cfg: Config) -> F.ep_config:
    return cfg.c()


def new_workspace(cfg: Config, device="cuda") -> torch.Tensor:
    return torch.empty(cfg.workspace_bytes(), dtype=torch.uint8, device=device)


def layout(cfg: Config, topk_idx: torch.Tensor, topk_w: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> Handle:
    cur = _current_device()
    if workspace is None:
        workspace = new_workspace(cfg, topk_idx.device)
    h = F.ep_handle()
    _B.layout(cfg.c_addr(), topk_idx, topk_w, workspace, ctypes.addressof(h), _raw_stream(cur), cur)
    return Handle(cfg, h, workspace, topk_idx)


def _recv_buffers(h: Handle, dtype: int, device, recv, recv_scales):
    R, H = h.cfg.recv_rows_bound(), h.cfg.hidden
    fp8 = dtype != BF16
    if recv is None:
        recv = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=device)
    if fp8 and recv_scales is None:
        recv_scales = torch.empty((R, H // 128), dtype=torch.float32, device=device)
    return recv, recv_scales


def dispatch(h: Handle, x: torch.Tensor, dtype: int = BF16, x_scales: Optional[torch.Tensor] = None,
             recv: Optional[torch.Tensor] = None, recv_scales: Optional[torch.Tensor] = None):
    """Returns recv (and recv_scales for the FP8 types)."""
    cur = _current_device()
    recv, recv_scales = _recv_buffers(h, dtype, x.device, recv, recv_scales)
    _B.dispatch(ctypes.addressof(h.c), dtype, x, x_scales, recv, recv_scales, _raw_stream(cur), cur)
    return (recv, recv_scales) if dtype != BF16 else recv


def dispatch_forward(cfg: Config, topk_idx: torch.Tensor, x: torch.Tensor, dtype: int = BF16,
                     topk_w: Optional[torch.Tensor] = None, x_scales: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, recv: Optional[torch.Tensor] = None,
                     recv_scales: Optional[torch.Tensor] = None):
    """Layout + dispatch in one call (README dispatch_forward). Returns
    (handle, recv) or (handle, recv, recv_scales) for the FP8 types."""
    cur = _current_device()
    if workspace is None:
        workspace = new_workspace(cfg, topk_idx.device)
    fp8 = dtype != BF16
    if recv is None:
        recv = torch.empty((cfg.recv_rows_bound(), cfg.hidden), dtype=torch.uint8 if fp8 else torch.bfloat16,
                           device=x.device)
    if fp8 and recv_scales is None:
        recv_scales = torch.empty((cfg.recv_rows_bound(), cfg.hidden // 128), dtype=torch.float32, device=x.device)
    c = F.ep_handle()
    _B.dispatch_forward(cfg.c_addr(), topk_idx, topk_w, workspace, dtype, x, x_scales, recv, recv_scales,
                        ctypes.addressof(c), _raw_stream(cur), cur)
    h = Handle(cfg, c, workspace, topk_idx)
    return (h, recv, recv_scales) if fp8 else (h, recv)


def combine(h: Handle, y: torch.Tensor, topk_w: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            row_vals: Optional[torch.Tensor] = None):
    """Returns out [T, H] bf16 (and out_vals [T, k] when row_vals is given)."""
    cur = _current_device()
    if out is None:
        out = torch.empty((h.c.num_tokens, h.cfg.hidden), dtype=torch.bfloat16, device=y.device)
    out_vals = None if row_vals is None else torch.empty((h.c.num_tokens, h.cfg.num_topk), dtype=torch.float32,
                                                         device=y.device)
    _B.combine(ctypes.addressof(h.c), y, topk_w, out, row_vals, out_vals, _raw_stream(cur), cur)
    return out if row_vals is None else (out, out_vals)


def dispatch_backward(h: Handle, grad_recv: torch.Tensor, grad_row_w: Optional[torch.Tensor] = None,
                      grad_x: Optional[torch.Tensor] = None, grad_topk_w: Optional[torch.Tensor] = None):
    """README dispatch_backward: returns grad_x (and grad_topk_w when
    grad_row_w is given), into the given buffers or new ones."""
    cur = _current_device()
    T, H, k = h.c.num_tokens, h.cfg.hidden, h.cfg.num_topk
    gx = grad_x if grad_x is not None else torch.empty((T, H), dtype=torch.bfloat16, device=grad_recv.device)
    gw = None
    if grad_row_w is not None:
        gw = grad_topk_w if grad_topk_w is not None else torch.empty((T, k), dtype=torch.float32,
                                                                     device=grad_recv.device)
    _B.dispatch_backward(ctypes.addressof(h.c), grad_recv, grad_row_w, gx, gw, _raw_stream(cur), cur)
    return gx if gw is None else (gx, gw)


def combine_backward(h: Handle, grad_out: torch.Tensor, dtype: int = BF16, topk_w: Optional[torch.Tensor] = None,
                     grad_y: Optional[torch.Tensor] = None, grad_y_scales: Optional[torch.Tensor] = None,
                     grad_out_scales: Optional[torch.Tensor] = None):
    """README combine_backward: a dispatch of grad_out on the handle
    (FP8_PREQUANT: grad_out holds E4M3 codes and grad_out_scales their 1x128
    scales, the README's (data, scale_factors) input)."""
    cur = _current_device()
    grad_y, grad_y_scales = _recv_buffers(h, dtype, grad_out.device, grad_y, grad_y_scales)
    _B.combine_backward(ctypes.addressof(h.c), dtype, grad_out, grad_out_scales, topk_w, grad_y, grad_y_scales,
                        _raw_stream(cur), cur)
    return (grad_y, grad_y_scales) if dtype != BF16 else grad_y


def combine_weight_grad(h: Handle, grad_out: torch.Tensor, y: torch.Tensor,
                        grad_topk_w: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the weighted combine with respect to topk_w: [T, k] float32,
    grad_topk_w[t, j] = <grad_out[t], y[slot[t, j]]> (0 for skipped pairs)."""
    T, H, k = h.num_tokens, h.cfg.hidden, h.cfg.num_topk
    _need(grad_out, (T, H), "grad_out")
    _need(y, (h.cfg.recv_rows_bound(), H), "y")
    if grad_topk_w is None:
        grad_topk_w = torch.empty((T, k), dtype=torch.float32, device=grad_out.device)
    _need(grad_topk_w, (T, k), "grad_topk_w")
    F.ep_combine_weight_grad(h.c, _dev(grad_out, "grad_out", torch.bfloat16), _dev(y, "y", torch.bfloat16),
                             _dev(grad_topk_w, "grad_topk_w", torch.float32), _stream())
    return grad_topk_w



def grouped_gemm_fp8(h: Handle, a: torch.Tensor, a_scales: torch.Tensor, b: torch.Tensor, b_scales: torch.Tensor,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FP8 grouped GEMM over the receive layout: out [rows bound, n] bf16,
    rows of expert e times b[e] [n, hidden] (E4M3FN) with 1x128 row scales
    and 128x128 weight scales."""
    R, H, E = h.cfg.recv_rows_bound(), h.cfg.hidden, h.cfg.num_experts
    if b.dim() != 3 or b.shape[0] != E or b.shape[2] != H:
        raise ValueError("b must be [E, n, hidden]")
    n = int(b.shape[1])
    _need(a, (R, H), "a")
    _need(a_scales, (R, H // 128), "a_scales")
    _need(b_scales, (E, n // 128, H // 128), "b_scales")
    if out is None:
        out = torch.empty((R, n), dtype=torch.bfloat16, device=a.device)
    _need(out, (R, n), "out")
    F.ep_grouped_gemm_fp8(h.c, _dev(a, "a", torch.uint8), _dev(a_scales, "a_scales", torch.float32),
                          _dev(b, "b", torch.uint8), _dev(b_scales, "b_scales", torch.float32), n,
                          _dev(out, "out", torch.bfloat16), _stream())
    return out

# ---------------------------------------------------------------- bound calls

class BoundCall:
    """One entry point with every argument converted once. Each call
    re-issues the same C function on the same buffers and stream (their
    contents are read when the kernels run), so it costs one foreign call:
    the low-latency form of the README's cached-handle decode loop, for
    callers that reuse their buffers from step to step. The tensors stay
    referenced for the object's lifetime."""

    def __init__(self, fn, args, name: str, keep):
        self._fn = fn
        self._args = args
        self._name = name
        self._keep = keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != F.EP_OK:
            raise F.EPError(st, self._name, F.last_error_message())


def bind_dispatch_forward(cfg: Config, topk_idx: torch.Tensor, x: torch.Tensor, dtype: int, recv: torch.Tensor,
                          recv_scales: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                          x_scales: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Bound ep_dispatch_forward on fixed buffers. Returns (call, handle):
    every call() rebuilds the layout from topk_idx's current contents and
    dispatches x into recv; `handle` (shared by all calls) describes it."""
    import ctypes
    T, H, R = int(topk_idx.shape[0]), cfg.hidden, cfg.recv_rows_bound()
    idx_dtype = torch.int64 if cfg.idx_bits == 64 else torch.int32
    if topk_idx.dim() != 2 or topk_idx.shape[1] != cfg.num_topk:
        raise ValueError("topk_idx must be [T, %d]" % cfg.num_topk)
    _need(topk_w, tuple(topk_idx.shape), "topk_w")
    _need(x, (T, H), "x")
    _need(recv, (R, H), "recv")
    fp8 = dtype != BF16
    if fp8:
        _need(recv_scales, (R, H // 128), "recv_scales")
    if dtype == FP8_PREQUANT:
        _need(x_scales, (T, H // 128), "x_scales")
    if workspace is None:
        workspace = new_workspace(cfg, topk_idx.device)
    c = _c_config(cfg)
    hc = F.ep_handle()
    xdt = torch.uint8 if dtype == FP8_PREQUANT else torch.bfloat16
    vp = ctypes.c_void_p
    args = (ctypes.byref(c), ctypes.c_int32(T), vp(_dev(topk_idx, "topk_idx", idx_dtype)),
            vp(_opt(topk_w, "topk_w", torch.float32)), vp(_dev(workspace, "workspace", torch.uint8)),
            ctypes.c_size_t(workspace.numel()), ctypes.c_int(dtype), vp(_dev(x, "x", xdt)),
            vp(_opt(x_scales, "x_scales", torch.float32)),
            vp(_dev(recv, "recv", torch.uint8 if fp8 else torch.bfloat16)),
            vp(_opt(recv_scales, "recv_scales", torch.float32)), ctypes.byref(hc), vp(_stream()))
    call = BoundCall(F.lib().ep_dispatch_forward, args, "ep_dispatch_forward",
                     (cfg, c, hc, topk_idx, topk_w, x, x_scales, recv, recv_scales, workspace))
    call()
    return call, Handle(cfg, hc, workspace, topk_idx)


def bind_combine(h: Handle, y: torch.Tensor, out: torch.Tensor, topk_w: Optional[torch.Tensor] = None):
    """Bound ep_combine on fixed buffers and on h's handle structure (which a
    bound dispatch_forward rewrites in place), issued with call()."""
    import ctypes
    T, H = h.num_tokens, h.cfg.hidden
    _need(y, (h.cfg.recv_rows_bound(), H), "y")
    _need(topk_w, (T, h.cfg.num_topk), "topk_w")
    _need(out, (T, H), "out")
    vp = ctypes.c_void_p
    args = (ctypes.byref(h.c), vp(_dev(y, "y", torch.bfloat16)), vp(_opt(topk_w, "topk_w", torch.float32)),
            vp(_dev(out, "out", torch.bfloat16)), None, None, vp(_stream()))
    return BoundCall(F.lib().ep_combine, args, "ep_combine", (h, y, out, topk_w))
