"""CPU oracle for MoE dispatch / combine — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its binding)
never imports it and shares no code with it.

The arithmetic lives in ``ep_oracle.c`` (plain single-threaded C, built with
gcc -O2 -ffp-contract=off). This module compiles it on first use when the
shared object is missing or older than the source, and marshals numpy arrays
through ctypes. Every function here states the reading it follows; the C
file cites the page passages. A second build of the same file with -fopenmp
spreads the per-token loops over host threads (``threads(n)`` selects it for
the calls that follow); it exists to time the oracle on several cores and
returns the same bits as the plain build.

Parity pins: every function is pinned by tests under ``tests/`` against
closed forms, library special cases, brute force and hand-derived fixtures;
none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")
_LIB_OMP = os.path.join(_HERE, "libep_oracle_omp.so")

MODE_COMPACT = 0
MODE_FIXED = 1
FLAG_BAD_ID = 1
FLAG_OVERFLOW = 2

_libs = {}
_use_omp = False


def _build_one(out: str, omp: bool, force: bool) -> str:
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-Wextra", "-shared", "-fPIC"]
        cmd += ["-fopenmp"] if omp else ["-Wno-unknown-pragmas"]
        cmd += ["-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction): the plain
    build and the OpenMP timing build of the same source."""
    _build_one(_LIB_OMP, True, force)
    return _build_one(_LIB, False, force)


def threads(n: int) -> int:
    """Route the calls that follow through the OpenMP build with n threads
    (n >= 1), or back to the plain build (n = 0). Returns the threads the
    loops use (1 for the plain build)."""
    global _use_omp
    _use_omp = n > 0
    return int(_load().ora_threads(n))


def _load():
    key = "omp" if _use_omp else "plain"
    lib = _libs.get(key)
    if lib is not None:
        return lib
    path = _build_one(_LIB_OMP, True, False) if _use_omp else build()
    lib = ctypes.CDLL(path)
    lib.ora_threads.restype = ctypes.c_int
    lib.ora_threads.argtypes = [ctypes.c_int]
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.ora_layout.restype = ctypes.c_uint32
    lib.ora_layout.argtypes = [i32] * 8 + [P] * 10
    lib.ora_dispatch_bf16.restype = None
    lib.ora_dispatch_bf16.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, i32, P]
    lib.ora_dispatch_fp8.restype = None
    lib.ora_dispatch_fp8.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i32, P, P]
    lib.ora_dispatch_fp8_prequant.restype = None
    lib.ora_dispatch_fp8_prequant.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, i32, P, P]
    lib.ora_combine.restype = None
    lib.ora_combine.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.ora_combine_backward_fp8.restype = None
    lib.ora_combine_backward_fp8.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, i32, P, P]
    lib.ora_grouped_gemm_fp8.restype = None
    lib.ora_grouped_gemm_fp8.argtypes = [i32, i32, i32, P, P, P, P, P, P, P]
    lib.ora_grouped_gemm_fp8_at.restype = None
    lib.ora_grouped_gemm_fp8_at.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, ctypes.c_int64, P]
    lib.ora_combine_weight_grad.restype = None
    lib.ora_combine_weight_grad.argtypes = [i32, i32, i32, P, P, P, P]
    lib.ora_e4m3_encode_many.restype = None
    lib.ora_e4m3_encode_many.argtypes = [P, ctypes.c_int64, P]
    lib.ora_bf16_rne_many.restype = None
    lib.ora_bf16_rne_many.argtypes = [P, ctypes.c_int64, P]
    lib.ora_e4m3_code_value.restype = ctypes.c_double
    lib.ora_e4m3_code_value.argtypes = [i32]
    lib.ora_quantize_block.restype = ctypes.c_float
    lib.ora_quantize_block.argtypes = [P, i32, P]
    _libs[key] = lib
    return lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def rows_bound(mode: int, T: int, E: int, k: int, A: int, C: int) -> int:
    return E * C if mode == MODE_FIXED else T * k + E * (A - 1)


def check_args(mode: int, T: int, E: int, k: int, A: int, D: int, C: int) -> None:
    if mode not in (MODE_COMPACT, MODE_FIXED):
        raise ValueError("mode")
    if T < 0 or k < 1 or E < 1 or E > 4096 or D < 1 or E % D != 0:
        raise ValueError("bad shape T=%d E=%d k=%d D=%d" % (T, E, k, D))
    if mode == MODE_COMPACT and A < 1:
        raise ValueError("expert_alignment must be >= 1")
    if mode == MODE_FIXED and (C < 1 or A != 1):
        raise ValueError("fixed mode needs capacity >= 1 and alignment 1")


def layout(mode: int, T: int, E: int, k: int, A: int, D: int, C: int,
           topk_idx: np.ndarray, topk_w: Optional[np.ndarray] = None) -> dict:
    """Counts, padded counts, offsets, stable slots (see ora_layout).

    ``topk_idx`` is int64 or int32 [T, k]; rows of ``row_src``/``row_w`` that
    the layout does not define keep the fill values -2 / NaN."""
    check_args(mode, T, E, k, A, D, C)
    lib = _load()
    idx = np.ascontiguousarray(topk_idx)
    if idx.dtype not in (np.int64, np.int32) or idx.shape != (T, k):
        raise ValueError("topk_idx must be int64/int32 [T, k]")
    bits = 64 if idx.dtype == np.int64 else 32
    w = None if topk_w is None else _c(topk_w, np.float32)
    R = rows_bound(mode, T, E, k, A, C)
    out = {
        "cnt": np.zeros(E, np.int32), "pad": np.zeros(E, np.int32),
        "expert_off": np.zeros(E + 1, np.int32), "dest_off": np.zeros(D + 1, np.int32),
        "dest_tokens": np.zeros(D, np.int32), "slot": np.zeros(T * k, np.int32),
        "row_src": np.full(max(R, 1), -2, np.int32),
        "row_w": np.full(max(R, 1), np.nan, np.float32),
    }
    flags = lib.ora_layout(mode, T, E, k, A, D, C, bits, _p(idx), _p(w),
                           _p(out["cnt"]), _p(out["pad"]), _p(out["expert_off"]),
                           _p(out["dest_off"]), _p(out["dest_tokens"]), _p(out["slot"]),
                           _p(out["row_src"]), _p(out["row_w"]))
    out["row_src"] = out["row_src"][:R]
    out["row_w"] = out["row_w"][:R]
    out["flags"] = int(flags)
    out["rows"] = int(out["expert_off"][E]) if mode == MODE_COMPACT else E * C
    out["rows_bound"] = R
    out["mode"] = mode
    return out


def dispatch_bf16(lay: dict, x: np.ndarray, k: int, pair_w: Optional[np.ndarray] = None,
                  zero_pad: bool = True, recv: Optional[np.ndarray] = None) -> np.ndarray:
    """BF16 dispatch into ``recv`` [rows_bound, H] (uint16 bit patterns).
    Rows the dispatch does not write keep their previous content (0xFFFF
    when ``recv`` is created here)."""
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    E = lay["cnt"].shape[0]
    if recv is None:
        recv = np.full((lay["rows_bound"], H), 0xFFFF, np.uint16)
    w = None if pair_w is None else _c(pair_w, np.float32)
    lib.ora_dispatch_bf16(T, H, k, E, _p(x), _p(lay["slot"]), _p(w), _p(lay["cnt"]),
                          _p(lay["pad"]), _p(lay["expert_off"]), int(bool(zero_pad)), _p(recv))
    return recv


def dispatch_fp8(lay: dict, x: np.ndarray, k: int, zero_pad: bool = True,
                 recv: Optional[np.ndarray] = None, recv_scales: Optional[np.ndarray] = None):
    """FP8 (E4M3FN) quantise + dispatch; returns (codes [R, H] u8, scales [R, H/128] f32)."""
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    if H % 128:
        raise ValueError("FP8 needs hidden % 128 == 0")
    E = lay["cnt"].shape[0]
    R = lay["rows_bound"]
    if recv is None:
        recv = np.full((R, H), 0xFF, np.uint8)
    if recv_scales is None:
        recv_scales = np.full((R, H // 128), np.nan, np.float32)
    lib.ora_dispatch_fp8(T, H, k, E, _p(x), _p(lay["slot"]), _p(lay["cnt"]), _p(lay["pad"]),
                         _p(lay["expert_off"]), int(bool(zero_pad)), _p(recv), _p(recv_scales))
    return recv, recv_scales


def dispatch_fp8_prequant(lay: dict, xq: np.ndarray, xs: np.ndarray, k: int, zero_pad: bool = True,
                          recv: Optional[np.ndarray] = None, recv_scales: Optional[np.ndarray] = None):
    lib = _load()
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.float32)
    T, H = xq.shape
    if H % 128 or xs.shape != (T, H // 128):
        raise ValueError("pre-quantised input needs [T, H] codes and [T, H/128] scales")
    E = lay["cnt"].shape[0]
    R = lay["rows_bound"]
    if recv is None:
        recv = np.full((R, H), 0xFF, np.uint8)
    if recv_scales is None:
        recv_scales = np.full((R, H // 128), np.nan, np.float32)
    lib.ora_dispatch_fp8_prequant(T, H, k, E, _p(xq), _p(xs), _p(lay["slot"]), _p(lay["cnt"]),
                                  _p(lay["pad"]), _p(lay["expert_off"]), int(bool(zero_pad)),
                                  _p(recv), _p(recv_scales))
    return recv, recv_scales


def combine(lay: dict, y: np.ndarray, k: int, topk_w: Optional[np.ndarray] = None,
            row_vals: Optional[np.ndarray] = None, T: Optional[int] = None):
    """Weighted (or plain) combine; returns out [T, H] (uint16) and, when
    ``row_vals`` is given, out_vals [T, k] (float32)."""
    lib = _load()
    y = _c(y, np.uint16)
    H = y.shape[1]
    slot = lay["slot"]
    T = slot.shape[0] // k if T is None else T
    out = np.empty((T, H), np.uint16)
    w = None if topk_w is None else _c(topk_w, np.float32)
    rv = None if row_vals is None else _c(row_vals, np.float32)
    ov = None if row_vals is None else np.empty((T, k), np.float32)
    lib.ora_combine(T, H, k, _p(y), _p(slot), _p(w), _p(out), _p(rv), _p(ov))
    return out, ov


def dispatch_backward(lay: dict, grad_recv: np.ndarray, k: int,
                      grad_row_w: Optional[np.ndarray] = None):
    """README dispatch_backward: a combine without weights, plus the gather
    of per-row weight gradients back to [T, k]."""
    return combine(lay, grad_recv, k, None, grad_row_w)


def combine_backward_bf16(lay: dict, grad_out: np.ndarray, k: int,
                          topk_w: Optional[np.ndarray] = None, zero_pad: bool = True):
    """README combine_backward: a dispatch on the same layout; with weights,
    each copy is scaled by its pair weight (gradient of a weighted combine)."""
    return dispatch_bf16(lay, grad_out, k, pair_w=topk_w, zero_pad=zero_pad)


def combine_weight_grad(lay: dict, grad_out: np.ndarray, y: np.ndarray, k: int) -> np.ndarray:
    """Gradient of the weighted combine with respect to topk_w: [T, k]
    float64, grad_w[t, j] = sum_h grad_out[t, h] * y[slot[t, j], h] (0 for
    skipped pairs), exact products summed in binary64 in channel order."""
    lib = _load()
    g = _c(grad_out, np.uint16)
    y = _c(y, np.uint16)
    T, H = g.shape
    if y.shape[1] != H or lay["slot"].shape[0] != T * k:
        raise ValueError("grad_out [T, H], y [rows, H] and the layout must agree")
    out = np.empty((T, k), np.float64)
    lib.ora_combine_weight_grad(T, H, k, _p(g), _p(y), _p(lay["slot"]), _p(out))
    return out


def combine_backward_fp8(lay: dict, grad_out: np.ndarray, k: int, topk_w: np.ndarray, zero_pad: bool = True):
    """Weighted combine_backward with FP8 output: each pair's row is
    bf16_rne(w * g) quantised per 1x128 block (its own scales). Returns
    (codes [R, H] u8, scales [R, H/128] f32); rows not written keep 0xFF / NaN."""
    lib = _load()
    g = _c(grad_out, np.uint16)
    T, H = g.shape
    if H % 128:
        raise ValueError("FP8 needs hidden % 128 == 0")
    w = _c(topk_w, np.float32)
    E = lay["cnt"].shape[0]
    R = lay["rows_bound"]
    recv = np.full((R, H), 0xFF, np.uint8)
    scales = np.full((R, H // 128), np.nan, np.float32)
    lib.ora_combine_backward_fp8(T, H, k, E, _p(g), _p(w), _p(lay["slot"]), _p(lay["cnt"]), _p(lay["pad"]),
                                 _p(lay["expert_off"]), int(bool(zero_pad)), _p(recv), _p(scales))
    return recv, scales


def grouped_gemm_fp8(row_begin: np.ndarray, row_end: np.ndarray, a: np.ndarray, sa: np.ndarray,
                     b: np.ndarray, sb: np.ndarray, pairs: Optional[np.ndarray] = None) -> np.ndarray:
    """FP8 grouped GEMM over expert row ranges (see ora_grouped_gemm_fp8).
    a [rows, K] u8, sa [rows, K/128] f32, b [E, N, K] u8, sb [E, N/128, K/128]
    f32. Returns C [rows, N] bf16 bits (rows outside every range 0xFFFF), or,
    with pairs [n, 2] int64 (r, n), the bf16 bits of those outputs."""
    lib = _load()
    a = _c(a, np.uint8)
    sa = _c(sa, np.float32)
    b = _c(b, np.uint8)
    sb = _c(sb, np.float32)
    rb = _c(row_begin, np.int32)
    re_ = _c(row_end, np.int32)
    E, N, K = b.shape
    if K % 128 or N % 128 or a.shape[1] != K or sa.shape != (a.shape[0], K // 128) or sb.shape != (E, N // 128, K // 128):
        raise ValueError("grouped GEMM shapes disagree")
    if pairs is None:
        C = np.full((a.shape[0], N), 0xFFFF, np.uint16)
        lib.ora_grouped_gemm_fp8(E, K, N, _p(rb), _p(re_), _p(a), _p(sa), _p(b), _p(sb), _p(C))
        return C
    pr = _c(pairs, np.int64)
    out = np.empty(pr.shape[0], np.uint16)
    lib.ora_grouped_gemm_fp8_at(E, K, N, _p(rb), _p(re_), _p(a), _p(sa), _p(b), _p(sb), _p(pr), pr.shape[0],
                                _p(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = _c(v, np.float32).ravel()
    q = np.empty(v.shape, np.uint8)
    lib.ora_e4m3_encode_many(_p(v), v.size, _p(q))
    return q


def bf16_rne(v: np.ndarray) -> np.ndarray:
    lib = _load()
    v = _c(v, np.float32).ravel()
    q = np.empty(v.shape, np.uint16)
    lib.ora_bf16_rne_many(_p(v), v.size, _p(q))
    return q


def e4m3_code_value(code: int) -> float:
    return float(_load().ora_e4m3_code_value(int(code)))


def quantize_block(xb: np.ndarray):
    """One 1x128 (or any length) block: returns (scale, codes)."""
    lib = _load()
    xb = _c(xb, np.uint16).ravel()
    q = np.empty(xb.shape, np.uint8)
    s = lib.ora_quantize_block(_p(xb), xb.size, _p(q))
    return float(np.float32(s)), q
