"""ctypes binding of include/ep.h: same names, argument marshalling only.

Loads the in-tree libep.so built for gfx950. There is no fallback: if the
library is missing this module raises, so nothing can run on another path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

EP_OK = 0
EP_ERR_INVALID_ARG = 1
EP_ERR_UNSUPPORTED = 2
EP_ERR_HIP = 3
EP_ERR_WORKSPACE = 4

EP_MODE_COMPACT = 0
EP_MODE_FIXED = 1

EP_BF16 = 0
EP_FP8_QUANTIZE = 1
EP_FP8_PREQUANT = 2

EP_FLAG_NO_ZERO_PAD = 1
EP_ERRFLAG_BAD_ID = 1
EP_ERRFLAG_OVERFLOW = 2


class ep_config(ctypes.Structure):
    _fields_ = [
        ("max_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("num_dests", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("idx_bits", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class ep_handle(ctypes.Structure):
    _fields_ = [
        ("cfg", ep_config),
        ("num_tokens", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("cnt", ctypes.c_void_p),
        ("pad", ctypes.c_void_p),
        ("expert_off", ctypes.c_void_p),
        ("dest_off", ctypes.c_void_p),
        ("dest_tokens", ctypes.c_void_p),
        ("slot", ctypes.c_void_p),
        ("row_src", ctypes.c_void_p),
        ("row_w", ctypes.c_void_p),
        ("err_flags", ctypes.c_void_p),
        ("internal", ctypes.c_void_p),
        ("topk_idx", ctypes.c_void_p),
    ]


class EPError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__("%s failed: %s: %s" % (where, status_string(status), message))
        self.status = status


_lib = None

# name -> (restype, argtypes)
_P = ctypes.c_void_p
_SIGNATURES = {
    "ep_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ep_config)]),
    "ep_recv_rows_bound": (ctypes.c_int64, [ctypes.POINTER(ep_config)]),
    "ep_layout": (ctypes.c_int, [ctypes.POINTER(ep_config), ctypes.c_int32, _P, _P, _P, ctypes.c_size_t,
                                 ctypes.POINTER(ep_handle), _P]),
    "ep_dispatch_forward": (ctypes.c_int, [ctypes.POINTER(ep_config), ctypes.c_int32, _P, _P, _P, ctypes.c_size_t,
                                           ctypes.c_int32, _P, _P, _P, _P, ctypes.POINTER(ep_handle), _P]),
    "ep_dispatch_forward_static_scratch": (ctypes.c_int, [ctypes.POINTER(ep_config), ctypes.c_int32, _P, _P, _P,
                                                          ctypes.c_size_t, ctypes.c_int32, _P, _P, _P, _P,
                                                          ctypes.POINTER(ep_handle), _P]),
    "ep_dispatch": (ctypes.c_int, [ctypes.POINTER(ep_handle), ctypes.c_int32, _P, _P, _P, _P, _P]),
    "ep_combine": (ctypes.c_int, [ctypes.POINTER(ep_handle), _P, _P, _P, _P, _P, _P]),
    "ep_dispatch_backward": (ctypes.c_int, [ctypes.POINTER(ep_handle), _P, _P, _P, _P, _P]),
    "ep_combine_backward": (ctypes.c_int, [ctypes.POINTER(ep_handle), ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "ep_combine_weight_grad": (ctypes.c_int, [ctypes.POINTER(ep_handle), _P, _P, _P, _P]),
    "ep_grouped_gemm_fp8": (ctypes.c_int, [ctypes.POINTER(ep_handle), _P, _P, _P, _P, ctypes.c_int32, _P, _P]),
    "ep_handle_read_counts": (ctypes.c_int, [ctypes.POINTER(ep_handle), _P, _P, _P, _P]),
    "ep_handle_check": (ctypes.c_int, [ctypes.POINTER(ep_handle), _P, _P]),
    "ep_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "ep_last_error_message": (ctypes.c_char_p, []),
}


def lib():
    """The loaded libep.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libep.so not found at %s: build it with "
                              "`python -m combine_ep_layout_10_amd.build` (hipcc, gfx950)" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(s: int) -> str:
    return lib().ep_status_string(int(s)).decode()


def last_error_message() -> str:
    return lib().ep_last_error_message().decode()


def _check(status: int, where: str) -> None:
    if status != EP_OK:
        raise EPError(status, where, last_error_message())


# ---------------------------------------------------------------- same names

def ep_workspace_bytes(cfg: ep_config) -> int:
    return int(lib().ep_workspace_bytes(ctypes.byref(cfg)))


def ep_recv_rows_bound(cfg: ep_config) -> int:
    return int(lib().ep_recv_rows_bound(ctypes.byref(cfg)))


def ep_layout(cfg: ep_config, num_tokens: int, topk_idx: int, topk_w, workspace: int,
              workspace_bytes: int, stream: int) -> ep_handle:
    h = ep_handle()
    _check(lib().ep_layout(ctypes.byref(cfg), int(num_tokens), topk_idx, topk_w, workspace,
                           int(workspace_bytes), ctypes.byref(h), stream), "ep_layout")
    return h


def ep_dispatch_forward(cfg: ep_config, num_tokens: int, topk_idx: int, topk_w, workspace: int,
                        workspace_bytes: int, dtype: int, x: int, x_scales, recv: int, recv_scales,
                        stream: int) -> ep_handle:
    h = ep_handle()
    st = (_lib or lib()).ep_dispatch_forward(ctypes.byref(cfg), num_tokens, topk_idx, topk_w, workspace,
                                             workspace_bytes, dtype, x, x_scales, recv, recv_scales,
                                             ctypes.byref(h), stream)
    if st != EP_OK:
        _check(st, "ep_dispatch_forward")
    return h


def ep_dispatch(h: ep_handle, dtype: int, x: int, x_scales, recv: int, recv_scales, stream: int) -> None:
    _check(lib().ep_dispatch(ctypes.byref(h), int(dtype), x, x_scales, recv, recv_scales, stream), "ep_dispatch")


def ep_combine(h: ep_handle, y: int, topk_w, out: int, row_vals, out_vals, stream: int) -> None:
    st = (_lib or lib()).ep_combine(ctypes.byref(h), y, topk_w, out, row_vals, out_vals, stream)
    if st != EP_OK:
        _check(st, "ep_combine")


def ep_dispatch_backward(h: ep_handle, grad_recv: int, grad_row_w, grad_x: int, grad_topk_w, stream: int) -> None:
    _check(lib().ep_dispatch_backward(ctypes.byref(h), grad_recv, grad_row_w, grad_x, grad_topk_w, stream),
           "ep_dispatch_backward")


def ep_combine_backward(h: ep_handle, dtype: int, grad_out: int, grad_out_scales, topk_w, grad_y: int,
                        grad_y_scales, stream: int) -> None:
    _check(lib().ep_combine_backward(ctypes.byref(h), int(dtype), grad_out, grad_out_scales, topk_w, grad_y,
                                     grad_y_scales, stream), "ep_combine_backward")


def ep_combine_weight_grad(h: ep_handle, grad_out: int, y: int, grad_topk_w: int, stream: int) -> None:
    _check(lib().ep_combine_weight_grad(ctypes.byref(h), grad_out, y, grad_topk_w, stream),
           "ep_combine_weight_grad")


def ep_grouped_gemm_fp8(h: ep_handle, a: int, a_scales: int, b: int, b_scales: int, n: int, out: int,
                        stream: int) -> None:
    _check(lib().ep_grouped_gemm_fp8(ctypes.byref(h), a, a_scales, b, b_scales, int(n), out, stream),
           "ep_grouped_gemm_fp8")


def ep_handle_read_counts(h: ep_handle, cnt, pad, rows, stream: int) -> None:
    _check(lib().ep_handle_read_counts(ctypes.byref(h), cnt, pad, rows, stream), "ep_handle_read_counts")


def ep_handle_check(h: ep_handle, stream: int) -> int:
    f = ctypes.c_uint32(0)
    _check(lib().ep_handle_check(ctypes.byref(h), ctypes.byref(f), stream), "ep_handle_check")
    return int(f.value)


def ep_status_string(s: int) -> str:
    return status_string(s)


def ep_last_error_message() -> str:
    return last_error_message()
