"""The C-ABI library on the CPU: it loads, exports every entry point that
include/ep.h declares, sizes workspaces and rejects bad arguments before
touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from combine_ep_layout_10_amd import _ffi as F
from ep_workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "ep.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 11, names
    lib = F.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in F._SIGNATURES, n


def cfg(**kw):
    base = dict(max_tokens=64, hidden=256, num_experts=16, num_topk=2, num_dests=1, expert_alignment=1,
                capacity=0, mode=F.EP_MODE_COMPACT, idx_bits=64, flags=0)
    base.update(kw)
    return F.ep_config(**base)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_rows_bound_and_workspace(name):
    wl = WORKLOADS[name]
    c = cfg(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.k, num_dests=wl.D,
            expert_alignment=wl.A, capacity=wl.C, mode=wl.mode)
    assert F.ep_recv_rows_bound(c) == wl.recv_rows_bound
    ws = F.ep_workspace_bytes(c)
    # at least slot + row_src + row_w + counts
    assert ws >= 4 * (wl.T * wl.k + 2 * wl.recv_rows_bound + 2 * wl.E)
    assert ws % 256 == 0


@pytest.mark.parametrize("bad", [
    dict(num_experts=0), dict(num_experts=1025), dict(num_topk=0), dict(num_topk=33),
    dict(num_dests=3), dict(hidden=100), dict(hidden=0), dict(hidden=(1 << 24) + 8), dict(idx_bits=16),
    dict(expert_alignment=0), dict(mode=2), dict(mode=F.EP_MODE_FIXED, capacity=0),
    dict(mode=F.EP_MODE_FIXED, capacity=4, expert_alignment=2), dict(flags=8), dict(max_tokens=-1),
    dict(max_tokens=1 << 30, num_topk=4),
])
def test_invalid_configs(bad):
    c = cfg(**bad)
    assert F.ep_workspace_bytes(c) == 0
    assert F.ep_recv_rows_bound(c) == -1
    assert F.last_error_message() != ""
    h = F.ep_handle()
    st = F.lib().ep_layout(ctypes.byref(c), 1, ctypes.c_void_p(256), None, ctypes.c_void_p(256), 1 << 30,
                           ctypes.byref(h), None)
    assert st == F.EP_ERR_INVALID_ARG


def test_layout_argument_errors():
    c = cfg()
    lib = F.lib()
    h = F.ep_handle()
    need = F.ep_workspace_bytes(c)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks first
    assert lib.ep_layout(None, 1, fake, None, fake, need, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_layout(ctypes.byref(c), 65, fake, None, fake, need, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_layout(ctypes.byref(c), -1, fake, None, fake, need, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_layout(ctypes.byref(c), 4, None, None, fake, need, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_layout(ctypes.byref(c), 4, fake, None, None, need, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_layout(ctypes.byref(c), 4, fake, None, ctypes.c_void_p((1 << 20) + 8), need,
                         ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG     # misaligned workspace
    assert lib.ep_layout(ctypes.byref(c), 4, fake, None, fake, need - 1, ctypes.byref(h), None) == F.EP_ERR_WORKSPACE
    assert "needs" in F.last_error_message()
    assert lib.ep_layout(ctypes.byref(c), 4, fake, None, fake, need, None, None) == F.EP_ERR_INVALID_ARG


def fake_handle(**kw):
    h = F.ep_handle()
    h.cfg = cfg(**kw)
    h.num_tokens = 4
    for f in ("cnt", "pad", "expert_off", "dest_off", "dest_tokens", "slot", "row_src", "row_w", "err_flags"):
        setattr(h, f, 1 << 20)
    return h


def test_dispatch_combine_argument_errors():
    lib = F.lib()
    fake = ctypes.c_void_p(1 << 20)
    h = fake_handle()
    assert lib.ep_dispatch(None, F.EP_BF16, fake, None, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(h), 7, fake, None, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(h), F.EP_BF16, None, None, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(h), F.EP_BF16, ctypes.c_void_p((1 << 20) + 2), None, fake, None,
                           None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(h), F.EP_FP8_QUANTIZE, fake, None, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_dispatch(ctypes.byref(h), F.EP_FP8_PREQUANT, fake, None, fake, fake, None) == F.EP_ERR_INVALID_ARG
    h2 = fake_handle(hidden=200)
    assert lib.ep_dispatch(ctypes.byref(h2), F.EP_FP8_QUANTIZE, fake, None, fake, fake, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_combine(ctypes.byref(h), None, None, fake, None, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_combine(ctypes.byref(h), fake, None, fake, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_combine_backward(ctypes.byref(h), F.EP_FP8_PREQUANT, fake, fake, fake, fake, fake,
                                   None) == F.EP_ERR_UNSUPPORTED                # weights with FP8 input
    assert lib.ep_combine_backward(ctypes.byref(h), F.EP_FP8_QUANTIZE, fake, None, fake, fake, None,
                                   None) == F.EP_ERR_INVALID_ARG                # output scales missing
    assert lib.ep_combine_backward(ctypes.byref(h), F.EP_FP8_PREQUANT, fake, None, None, fake, fake,
                                   None) == F.EP_ERR_INVALID_ARG                # input scales missing
    assert lib.ep_combine_weight_grad(ctypes.byref(h), None, fake, fake, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_combine_weight_grad(ctypes.byref(h), fake, None, fake, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_combine_weight_grad(ctypes.byref(h), fake, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_combine_weight_grad(None, fake, fake, fake, None) == F.EP_ERR_INVALID_ARG
    h3 = fake_handle()
    h3.num_tokens = 65
    assert lib.ep_combine(ctypes.byref(h3), fake, None, fake, None, None, None) == F.EP_ERR_INVALID_ARG
    h4 = fake_handle()
    h4.slot = None
    assert lib.ep_dispatch(ctypes.byref(h4), F.EP_BF16, fake, None, fake, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_handle_check(None, None, None) == F.EP_ERR_INVALID_ARG
    assert lib.ep_handle_check(ctypes.byref(h), None, None) == F.EP_ERR_INVALID_ARG


def test_status_strings():
    for s, n in ((0, "EP_OK"), (1, "EP_ERR_INVALID_ARG"), (2, "EP_ERR_UNSUPPORTED"), (3, "EP_ERR_HIP"),
                 (4, "EP_ERR_WORKSPACE"), (99, "EP_ERR_UNKNOWN")):
        assert F.status_string(s) == n


def test_struct_sizes_match_header():
    # ep_config: 10 x 4 bytes; ep_handle: config + 2 ints + 11 pointers
    assert ctypes.sizeof(F.ep_config) == 40
    assert ctypes.sizeof(F.ep_handle) == 40 + 8 + 11 * 8


def test_struct_layout_matches_c_compiler(tmp_path):
    """Every field offset and the size of the ctypes structs equal what a C
    compiler gives for include/ep.h."""
    import subprocess
    lines = []
    for st in (F.ep_config, F.ep_handle):
        name = st.__name__
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (name, name))
        for f, _ in st._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (name, f, name, f))
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "ep.h"\nint main(void) {\n%s\nreturn 0;\n}\n'
                   % "\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {k: int(v) for k, v in (line.split() for line in out if line)}
    for st in (F.ep_config, F.ep_handle):
        name = st.__name__
        assert got[name] == ctypes.sizeof(st), name
        for f, _ in st._fields_:
            assert got[name + "." + f] == getattr(st, f).offset, (name, f)


def test_dispatch_forward_argument_errors():
    """Layout and dispatch arguments are all checked before anything is
    enqueued (every call below fails a check; no pointer is dereferenced)."""
    c = cfg()
    lib = F.lib()
    h = F.ep_handle()
    need = F.ep_workspace_bytes(c)
    fake = ctypes.c_void_p(1 << 20)
    f = lib.ep_dispatch_forward
    assert f(None, 4, fake, None, fake, need, F.EP_BF16, fake, None, fake, None, ctypes.byref(h), None) \
        == F.EP_ERR_INVALID_ARG
    assert f(ctypes.byref(c), 65, fake, None, fake, need, F.EP_BF16, fake, None, fake, None, ctypes.byref(h),
             None) == F.EP_ERR_INVALID_ARG
    assert f(ctypes.byref(c), 4, fake, None, fake, need - 256, F.EP_BF16, fake, None, fake, None,
             ctypes.byref(h), None) == F.EP_ERR_WORKSPACE
    assert f(ctypes.byref(c), 4, fake, None, fake, need, 7, fake, None, fake, None, ctypes.byref(h),
             None) == F.EP_ERR_INVALID_ARG
    assert f(ctypes.byref(c), 4, fake, None, fake, need, F.EP_BF16, None, None, fake, None, ctypes.byref(h),
             None) == F.EP_ERR_INVALID_ARG                                     # x NULL
    assert f(ctypes.byref(c), 4, fake, None, fake, need, F.EP_BF16, fake, None, None, None, ctypes.byref(h),
             None) == F.EP_ERR_INVALID_ARG                                     # recv NULL
    assert f(ctypes.byref(c), 4, fake, None, fake, need, F.EP_FP8_QUANTIZE, fake, None, fake, None,
             ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG                    # recv_scales NULL
    assert f(ctypes.byref(c), 4, fake, None, fake, need, F.EP_FP8_PREQUANT, fake, None, fake, fake,
             ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG                    # x_scales NULL
    assert f(ctypes.byref(c), 4, fake, None, fake, need, F.EP_BF16, fake, None, fake, None, None,
             None) == F.EP_ERR_INVALID_ARG                                     # out NULL
    assert "out handle" in F.last_error_message()


def test_grouped_gemm_argument_errors():
    """Every shape and pointer rule of ep_grouped_gemm_fp8 is checked on the
    host before the launch (no call below reaches the GPU)."""
    lib = F.lib()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)                          # 8-byte, not 16-byte, aligned
    g = lib.ep_grouped_gemm_fp8
    h = fake_handle(expert_alignment=128)
    assert g(None, fake, fake, fake, fake, 256, fake, None) == F.EP_ERR_INVALID_ARG
    for n in (0, -128, 64, 200):
        assert g(ctypes.byref(h), fake, fake, fake, fake, n, fake, None) == F.EP_ERR_INVALID_ARG, n
    assert g(ctypes.byref(fake_handle(hidden=200, expert_alignment=128)), fake, fake, fake, fake, 256, fake,
             None) == F.EP_ERR_UNSUPPORTED                                  # hidden % 128
    assert g(ctypes.byref(fake_handle(expert_alignment=64)), fake, fake, fake, fake, 256, fake,
             None) == F.EP_ERR_UNSUPPORTED                                  # a tile would span two experts
    assert g(ctypes.byref(fake_handle(mode=F.EP_MODE_FIXED, capacity=96)), fake, fake, fake, fake, 256, fake,
             None) == F.EP_ERR_UNSUPPORTED
    for args in ((None, fake, fake, fake), (odd, fake, fake, fake), (fake, None, fake, fake),
                 (fake, ctypes.c_void_p((1 << 20) + 2), fake, fake), (fake, fake, None, fake),
                 (fake, fake, odd, fake), (fake, fake, fake, None)):
        assert g(ctypes.byref(h), *args, 256, fake, None) == F.EP_ERR_INVALID_ARG, args
    assert g(ctypes.byref(h), fake, fake, fake, fake, 256, None, None) == F.EP_ERR_INVALID_ARG
    assert g(ctypes.byref(h), fake, fake, fake, fake, 256, odd, None) == F.EP_ERR_INVALID_ARG
    assert "16-byte" in F.last_error_message()


def test_static_scratch_rejects_layouts_beyond_its_array():
    """ep_dispatch_forward_static_scratch: a layout whose per-block partials
    exceed the 1 MiB static array is refused before any device work (the
    check precedes the array's lookup, so it runs without a GPU)."""
    lib = F.lib()
    # 1024 experts, 1024 destinations, 2^20 pairs: 1024 blocks x (1024 + 1024 + 1) ints
    c = cfg(max_tokens=1 << 17, hidden=128, num_experts=1024, num_topk=8, num_dests=1024, expert_alignment=1)
    h = F.ep_handle()
    st = lib.ep_dispatch_forward_static_scratch(ctypes.byref(c), 1 << 17, None, None, None, 0, F.EP_BF16, None,
                                                None, None, None, ctypes.byref(h), None)
    assert st == F.EP_ERR_WORKSPACE
    assert "static scratch" in F.last_error_message()
    # invalid configs and token counts are rejected as by ep_dispatch_forward
    bad = cfg(num_experts=0)
    assert lib.ep_dispatch_forward_static_scratch(ctypes.byref(bad), 1, None, None, None, 0, F.EP_BF16, None,
                                                  None, None, None, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
    c = cfg()
    assert lib.ep_dispatch_forward_static_scratch(ctypes.byref(c), 65, None, None, None, 0, F.EP_BF16, None,
                                                  None, None, None, ctypes.byref(h), None) == F.EP_ERR_INVALID_ARG
