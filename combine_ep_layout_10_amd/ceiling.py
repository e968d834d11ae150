"""ctypes binding of libep_ceiling.so: access-pattern reference kernels that
the benchmark times beside the path (no part of the dispatch/combine API).

Each kernel moves bytes in one of the path's access patterns with no
arithmetic, so its rate is what the memory system gives that pattern on the
machine at hand; a path kernel's rate over the reference's is how much of
that it reaches. Sizes are bytes; pointers are device addresses; `stream` is
a hipStream_t (0: the null stream). Each call raises on bad arguments or a
launch error.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_ceiling.so")

_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "ep_ceiling_write_rows": [_P, _I64, _I32, _P],
    "ep_ceiling_read_rows": [_P, _I64, _I32, _P, _P],
    "ep_ceiling_copy": [_P, _P, _I64, _P],
    "ep_ceiling_broadcast": [_P, _I64, _I32, _P, _I32, _P, _I32, _P],
    "ep_ceiling_gather": [_P, _I32, _P, _I32, _I64, _P, _P],
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        # torch first: torch ships its own HIP runtime under the same soname
        # (libamdhip64.so.7), and whichever copy loads first serves the whole
        # process; the kernels must launch on the runtime torch's device
        # memory and streams belong to.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError("libep_ceiling.so not found at %s: build it with "
                              "`python -m combine_ep_layout_10_amd.build`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = ctypes.c_int
            f.argtypes = args
        _lib = l
    return _lib


def _ok(rc: int, where: str) -> None:
    if rc != 0:
        raise RuntimeError("%s failed (code %d)" % (where, rc))


def write_rows(dst: int, rows: int, row_bytes: int, stream: int = 0) -> None:
    """rows x row_bytes of streaming row stores, one block per row."""
    _ok(lib().ep_ceiling_write_rows(dst, rows, row_bytes, stream), "ep_ceiling_write_rows")


def read_rows(src: int, rows: int, row_bytes: int, sink: int, stream: int = 0) -> None:
    """rows x row_bytes of streaming loads, one block per row; sink: a
    device int32 the kernel never writes for non-degenerate data."""
    _ok(lib().ep_ceiling_read_rows(src, rows, row_bytes, sink, stream), "ep_ceiling_read_rows")


def copy(src: int, dst: int, nbytes: int, stream: int = 0) -> None:
    """A plain copy, 4 KiB per block, one 16-byte load and store per lane."""
    _ok(lib().ep_ceiling_copy(src, dst, nbytes, stream), "ep_ceiling_copy")


def broadcast(src: int, tokens: int, src_row_bytes: int, dst: int, dst_row_bytes: int, rows: int, k: int,
              stream: int = 0) -> None:
    """Row t of src to the rows rows[t*k + j] of dst (int32, -1 skipped);
    src_row_bytes is dst_row_bytes or twice it (a bf16 row into an FP8
    row). Every row named must lie inside dst."""
    _ok(lib().ep_ceiling_broadcast(src, tokens, src_row_bytes, dst, dst_row_bytes, rows, k, stream),
        "ep_ceiling_broadcast")


def gather(src: int, row_bytes: int, rows: int, k: int, tokens: int, dst: int, stream: int = 0) -> None:
    """Rows rows[t*k + j] of src (int32, -1 skipped) read, one row written
    to dst[t]. Every row named must lie inside src."""
    _ok(lib().ep_ceiling_gather(src, row_bytes, rows, k, tokens, dst, stream), "ep_ceiling_gather")
