"""Benchmark: MoE layout -> dispatch -> combine (and the backward duals) on one MI355X.

One step = one pass of the whole path over one batch: ep_dispatch_forward
(the layout — counts, offsets, stable slots — and the dispatch — FP8 E4M3
1x128 quantise + copy for the V3 shape — in one call), ep_combine (weighted
BF16 reduction of the expert outputs), and, for the training-shaped
workloads (aligned COMPACT layout), the backward duals on the cached
handle: ep_combine_backward (a dispatch of the output gradient, each copy
scaled by its pair weight, BF16) and ep_dispatch_backward (a combine of the
receive-row gradients plus the gather of per-row weight gradients). The
decode workload (FIXED capacity) is inference: forward only; so are
--step forward, --graph and --bound. The expert computation between
dispatch and combine is not part of this path; combine and the backward
calls read seeded synthetic tensors of the receive layout.

Inputs are seeded synthetic data resident in HBM before the timed region.
Throughput is algorithmic bytes (the minimum each kernel must read and
write) over time; `roofline` reports the kernel that moves the most bytes
against the MI355X HBM peak, timed with HIP events recorded around it
inside the timed region, on the stream the kernels run on (--graph replays a
captured step instead; the per-kernel times then come from an evented eager
pass); `roofline.pattern_reference` is the simplest kernel with the dominant
call's access pattern and no arithmetic (libep_ceiling.so), timed in the same
run on the same rows, which tells how much of that pattern's rate on this
memory system the kernel reaches (`kernels.pattern_reference` holds the same
for every call of the step). `cpu_baseline` times the CPU oracle on the
same inputs and the same work: its OpenMP build on the host's cores (the value) and its plain build on
one core (`single_core`).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3] [--step path|forward] [--graph | --bound]
    python bench.py --step gemm [--gemm-n 4096]   # the FP8 grouped GEMM on the receive layout
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch/combine effective GB/s + % of HBM peak, 8K tok×7168 top-8"
HBM_PEAK_GBPS = 8000.0
# the sources each step's kernels are built from (a profile taken with one
# hash stays valid while those files are unchanged)
KERNEL_SOURCES = {
    "path": ["ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_fused.hip", "ep_internal.h",
             "ep_device.h", "ep_layout_dev.h", "ep_dispatch_dev.h"],
    "gemm": ["ep_gemm.hip", "ep_internal.h", "ep_device.h"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="v3")
    p.add_argument("--step", default="path", choices=["path", "forward", "gemm", "weight_grad", "fp8_backward"],
                   help="path: layout + dispatch + combine, plus the backward duals for COMPACT workloads "
                        "(the headline); forward: without the backward duals; gemm: the FP8 grouped GEMM consumer; "
                        "weight_grad / fp8_backward: one training call on the cached layout (the routing-weight "
                        "gradient, the weighted FP8 combine_backward)")
    p.add_argument("--gemm-n", type=int, default=4096, help="output channels per expert for --step gemm")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (for rocprofv3 counter scaling)")
    p.add_argument("--graph", action="store_true",
                   help="capture one step in a HIP graph and time K replays (launch-bound shapes)")
    p.add_argument("--bound", action="store_true",
                   help="time steps issued through bound calls (arguments converted once)")
    p.add_argument("--rotate", type=int, default=4,
                   help="copies of x and grad_out the eager steps cycle through (each step reads inputs no cache "
                        "holds: 4 copies of x and grad_out are 0.94 GB at the V3 shape, against a 256 MB MALL); "
                        "1 = the same inputs every step")
    p.add_argument("--no-warm", action="store_true",
                   help="skip the reference pass on one unrotated copy of the inputs (so that every call of the "
                        "run reads rotated inputs, as a profiled run should)")
    p.add_argument("--no-flush", action="store_true",
                   help="skip the per-kernel pass with L2 and MALL flushed before each kernel")
    p.add_argument("--no-copy-ceiling", action="store_true",
                   help="skip the reference kernels: 1 GiB copies and fill, and each call's access pattern with no "
                        "arithmetic (libep_ceiling.so)")
    return p.parse_args()


def kernel_hash(step: str = "path") -> str:
    h = hashlib.sha256()
    for s in KERNEL_SOURCES[step]:
        with open(os.path.join(ROOT, "combine_ep_layout_10_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, R: int, P: int, dispatch: str, train: bool = False) -> dict:
    """Minimum bytes each kernel must move (MB = 1e6 B in reports)."""
    T, H, k = wl.T, wl.H, wl.k
    nb = H // 128
    if dispatch == "fp8":
        row_out = H + 4 * nb            # codes + 1x128 scales
    else:
        row_out = 2 * H
    pad_rows = max(R - P, 0) if wl.mode == 0 else 0
    layout = T * k * 8 + T * k * 4 + T * k * 4 + 2 * 4 * (R if wl.mode == 0 else P)
    dispatch_b = T * H * 2 + T * k * 4 + P * row_out + pad_rows * row_out
    combine = P * H * 2 + T * k * 4 + T * k * 4 + T * H * 2
    out = {"layout": layout, "dispatch": dispatch_b, "combine": combine,
           "padding_rows": pad_rows, "pairs": P, "rows": R}
    if train:
        # combine_backward: grad_out, slots and pair weights in; every pair's
        # weighted BF16 copy and the zero padding rows out
        out["combine_backward"] = T * H * 2 + T * k * 4 + T * k * 4 + (P + pad_rows) * 2 * H
        # dispatch_backward: the pairs' gradient rows and slots in, grad_x
        # out, plus the per-row weight gradients gathered to [T, k]
        out["dispatch_backward"] = P * H * 2 + T * k * 4 + T * H * 2 + P * 4 + T * k * 4
    return out


def calib_copy(dev) -> None:
    """Three plain 1 GiB device-to-device copies, the reference that
    profile_summary scales FETCH_SIZE / WRITE_SIZE by."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def load_traffic(kernel: str, khash: str, workload: str, path: str = None):
    """HBM bytes per launch of `kernel` (name with template arguments, e.g.
    k_dispatch<2>) from committed rocprofv3 counter runs, if they were taken
    on the current kernel sources and on the same workload (the bytes of a
    launch depend on its shape), else None."""
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(workload, {}).get(kernel)
    if not ent or ent.get("kernel_hash") != khash or ent.get("workload") != workload:
        return None
    return ent.get("bytes_per_launch")


def median_event_ms(fn, stream, n: int = 5) -> float:
    """Median of n launches of fn(i) (i = 1..n, after one untimed fn(0)),
    each timed with HIP events on `stream`, in ms."""
    import numpy as np
    import torch
    fn(0)
    torch.cuda.synchronize()
    ts = []
    for i in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(i + 1)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def host_threads() -> int:
    """Host threads for the oracle's OpenMP leg: the cores this process may
    run on, capped by OMP_NUM_THREADS when the environment sets it."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def time_oracle(run, budget_s: float, max_runs: int = 50):
    """Median wall time of run() over at least one and at most max_runs
    calls, stopping once budget_s has passed; returns (seconds, runs)."""
    import numpy as np
    times = []
    end = time.perf_counter() + budget_s
    while not times or (len(times) < max_runs and time.perf_counter() < end):
        c0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - c0)
        print("[bench] oracle run %.2f s" % times[-1], file=sys.stderr, flush=True)
    return float(np.median(times)), len(times)


def oracle_baseline(run, nbytes: float, unit_scale: float, unit: str, budget_s: float, what: str) -> dict:
    """The oracle timed twice on the same work: the OpenMP build on this
    host's cores (the reported value) and the plain build on one core. The
    layout inside `run` stays serial in both."""
    import oracle
    n = oracle.threads(host_threads())
    t_mt, k_mt = time_oracle(run, budget_s / 3)
    oracle.threads(0)
    t_1, k_1 = time_oracle(run, budget_s * 2 / 3)
    return {"value": round(nbytes / t_mt / unit_scale, 6 if unit == "TFLOP/s" else 3), "unit": unit, "cores": n,
            "kind": "oracle",
            "sample": "%s; C oracle, OpenMP over tokens on %d host threads (layout serial): median of %d runs of "
                      "%.3f s; single-threaded: median of %d runs of %.2f s" % (what, n, k_mt, t_mt, k_1, t_1),
            "single_core": {"value": round(nbytes / t_1 / unit_scale, 6 if unit == "TFLOP/s" else 3),
                            "unit": unit, "cores": 1}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library computes one GPU's share and has no multi-GPU path "
              "(--gpus %d requested). Run with --gpus 1." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from ep_workloads import WORKLOADS, make_inputs, draw_routing, draw_weights, draw_hidden, _streams
    from combine_ep_layout_10_amd import ops

    if args.step == "gemm":
        return bench_gemm(args)
    if args.step in ("weight_grad", "fp8_backward"):
        return bench_call(args)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print("[bench] workload %s: generating inputs" % wl.name, file=sys.stderr, flush=True)
    sx, sr, sl, so, sy = _streams(0)
    x_h = draw_hidden(wl, sx, so)
    idx_h = draw_routing(wl, sr)
    w_h = draw_weights(wl, sl)
    cfg = ops.Config(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.k, num_dests=wl.D,
                     expert_alignment=wl.A, capacity=wl.C, mode=wl.mode, idx_bits=64)
    R_cap = cfg.recv_rows_bound()
    x = torch.from_numpy(x_h.view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(idx_h).to(dev)
    w = torch.from_numpy(w_h).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    y = torch.randn((R_cap, wl.H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ws = ops.new_workspace(cfg, dev)
    fp8 = wl.dispatch == "fp8"
    dtype = ops.FP8_QUANTIZE if fp8 else ops.BF16
    recv = torch.empty((R_cap, wl.H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    rs = torch.empty((R_cap, wl.H // 128), dtype=torch.float32, device=dev) if fp8 else None
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # training-shaped workloads also run the backward duals on the cached
    # handle; decode (FIXED capacity) is inference, forward only
    train = args.step == "path" and wl.mode == ops.MODE_COMPACT and not (args.graph or args.bound)
    if train:
        gen.manual_seed(5)
        grad_out = torch.randn((wl.T, wl.H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        grad_recv = torch.randn((R_cap, wl.H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        grad_row_w = torch.randn((R_cap,), generator=gen, device=dev, dtype=torch.float32)
        grad_y = torch.empty((R_cap, wl.H), dtype=torch.bfloat16, device=dev)
        grad_x = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        grad_w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)

    # The eager steps cycle through `rotate` copies of the inputs read with
    # plain loads (x, grad_out; identical contents), so that each step reads
    # them from HBM as a step of a real model would after other work, not
    # from the caches the previous step left them in. The expert-output
    # inputs (y, grad_recv: 1.4 GB each) are read with non-temporal loads and
    # never fit the caches anyway.
    nrot = max(1, args.rotate) if not (args.graph or args.bound) else 1
    xs = [x] + [x.clone() for _ in range(nrot - 1)]
    gos = ([grad_out] + [grad_out.clone() for _ in range(nrot - 1)]) if train else None
    cur = [0]                  # the step's copy index

    def do_dispatch(h):
        xi = xs[cur[0] % nrot]
        if fp8:
            ops.dispatch(h, xi, dtype, recv=recv, recv_scales=rs)
        else:
            ops.dispatch(h, xi, dtype, recv=recv)

    # the calls after the layout, in step order, and the kernel each runs
    calls = {"dispatch": do_dispatch, "combine": lambda h: ops.combine(h, y, w, out=out)}
    kname = {"dispatch": "k_dispatch<2>" if fp8 else "k_dispatch<0>", "combine": "k_combine<true>"}
    if train:
        calls["combine_backward"] = lambda h: ops.combine_backward(h, gos[cur[0] % nrot], ops.BF16, w,
                                                                   grad_y=grad_y)
        calls["dispatch_backward"] = lambda h: ops.dispatch_backward(h, grad_recv, grad_row_w, grad_x=grad_x,
                                                                     grad_topk_w=grad_w)
        kname["combine_backward"] = "k_dispatch<1>"
        kname["dispatch_backward"] = "k_combine<false>"
    names = list(calls)
    after = names[1:]          # what follows the layout + dispatch call

    def forward_head():
        xi = xs[cur[0] % nrot]
        if fp8:
            return ops.dispatch_forward(cfg, idx, xi, dtype, topk_w=w, workspace=ws, recv=recv, recv_scales=rs)[0]
        return ops.dispatch_forward(cfg, idx, xi, dtype, topk_w=w, workspace=ws, recv=recv)[0]

    def step():
        h = forward_head()
        for n in after:
            calls[n](h)
        return h

    def step_split(evs):
        """The same work as separate layout / dispatch / ... calls, with an
        event between them."""
        evs[0].record(stream)
        h = ops.layout(cfg, idx, w, workspace=ws)
        evs[1].record(stream)
        for i, n in enumerate(names):
            calls[n](h)
            evs[i + 2].record(stream)

    h = step()
    cnt, pad, R = h.read_counts()
    flags = h.check()
    if flags:
        raise RuntimeError("layout raised error flags %d on a valid workload" % flags)
    P = int(cnt.sum()) if wl.mode == 0 else int(pad.sum())
    nbytes = algorithmic_bytes(wl, R, P, wl.dispatch, train)
    step_bytes = nbytes["layout"] + sum(nbytes[n] for n in names)
    dominant = max(names, key=lambda n: nbytes[n])

    if args.calib_copy:
        calib_copy(dev)

    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    bound = None
    if args.bound:
        fwd_call, hb = ops.bind_dispatch_forward(cfg, idx, x, dtype, recv, rs, topk_w=w, workspace=ws)
        bound = (fwd_call, ops.bind_combine(hb, y, out, topk_w=w))

    def run_step():
        if graph is not None:
            graph.replay()
        elif bound is not None:
            bound[0]()
            bound[1]()
        else:
            step()

    print("[bench] warmup %d steps" % args.warmup, file=sys.stderr, flush=True)
    for i in range(args.warmup):
        cur[0] = i
        run_step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps. Eager steps carry one event pair around
    # the dominant kernel (recorded on the kernels' stream); graph replays
    # and bound calls carry none. Recording an event costs the host a few
    # microseconds, as much as a whole launch-bound step (under 100 MB moved),
    # so there only every 8th step carries the pair.
    ev_every = 8 if step_bytes < 100e6 else 1
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(0, args.steps, ev_every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
            continue
        if bound is not None:
            bound[0]()
            bound[1]()
            continue
        cur[0] = args.warmup + i
        ev = dom_ev[i // ev_every] if i % ev_every == 0 else None
        if dominant == "dispatch":
            h = ops.layout(cfg, idx, w, workspace=ws)
            if ev:
                ev[0].record(stream)
            do_dispatch(h)
            if ev:
                ev[1].record(stream)
            for n in after:
                calls[n](h)
        else:
            h = forward_head()
            for n in after:
                if n == dominant and ev:
                    ev[0].record(stream)
                    calls[n](h)
                    ev[1].record(stream)
                else:
                    calls[n](h)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    live = graph is None and bound is None
    dom_live_ms = float(np.mean([a.elapsed_time(b) for a, b in dom_ev])) if live else None
    # Per-kernel durations: K more steps as separate layout / dispatch / ...
    # calls with events between them (not part of the timed region).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 2)] for _ in range(args.steps)]
    for i in range(args.steps):
        cur[0] = i
        step_split(evs[i])
    torch.cuda.synchronize()
    lay_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    k_ms = {n: float(np.mean([e[i + 1].elapsed_time(e[i + 2]) for e in evs])) for i, n in enumerate(names)}
    gpu_ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    warm = None
    if nrot > 1 and not args.no_warm:
        # the same calls on the same inputs every step (x and grad_out stay
        # in the MALL between steps): for reference only
        wev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 2)] for _ in range(args.steps)]
        cur[0] = 0
        for i in range(args.steps):
            step_split(wev[i])
        torch.cuda.synchronize()
        warm = {n + "_us": round(float(np.mean([e[i + 1].elapsed_time(e[i + 2]) for e in wev])) * 1e3, 2)
                for i, n in enumerate(names)}
        warm["stat"] = "mean of %d steps on one copy of the inputs" % args.steps
    # the step with dispatch_forward as one unit (one launch for small batches)
    fw = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(fw):
        cur[0] = i
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_ev_ms = float(np.mean([a.elapsed_time(b) for a, b in fw]))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    khash = kernel_hash()
    gbps = {n: nbytes[n] / (k_ms[n] * 1e-3) / 1e9 for n in names}
    dom_ms = dom_live_ms if dom_live_ms is not None else k_ms[dominant]
    dom_gbps = nbytes[dominant] / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": load_traffic(kname[dominant], khash, wl.name),
                "kernel": kname[dominant], "call": dominant,
                "algorithmic_bytes_per_launch": nbytes[dominant],
                "avg_launch_us": round(dom_ms * 1e3, 2),
                "timed": ("events in the timed region" + (" (every %d-th step)" % ev_every if ev_every > 1 else ""))
                         if dom_live_ms is not None else "evented eager pass",
                "inputs": ("x and grad_out cycled through %d copies (read from HBM, not from the caches)" % nrot
                           if nrot > 1 else "the same inputs every step")}

    flushed = None
    if not args.no_flush and graph is None and bound is None:
        # Cold-cache per-kernel times (not the timed region): before the
        # layout and before each later call, a 512 MB buffer (larger than L2,
        # 4 MB per XCD, plus the 256 MB MALL) is written and then read, so
        # the caches hold only clean, unrelated lines (after a write alone
        # the next kernel would also pay for writing back its dirty lines);
        # medians over K steps.
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        sink = torch.empty((), dtype=torch.int64, device=dev)

        def flush(v):
            scratch.fill_(v)
            torch.sum(scratch.view(torch.int32), dim=0, out=sink)

        fl = []
        cur[0] = 0
        for i in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * (len(names) + 1))]
            flush(i & 0x7F)
            e[0].record(stream)
            hf = ops.layout(cfg, idx, w, workspace=ws)
            e[1].record(stream)
            for j, n in enumerate(names):
                flush((i + j + 1) & 0x7F)
                e[2 * j + 2].record(stream)
                calls[n](hf)
                e[2 * j + 3].record(stream)
            fl.append(e)
        torch.cuda.synchronize()
        med = [float(np.median([e[2 * j].elapsed_time(e[2 * j + 1]) for e in fl])) for j in range(len(names) + 1)]
        flushed = {"layout_us": round(med[0] * 1e3, 2)}
        for j, n in enumerate(names):
            flushed[n + "_us"] = round(med[j + 1] * 1e3, 2)
            flushed[n + "_frac"] = round(nbytes[n] / (med[j + 1] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        flushed["stat"] = "median of %d; 512 MB written and read before each kernel" % args.steps
        del scratch, sink

    copy_ceiling = fill_ceiling = None
    pattern = None
    # (the reference kernels move a row with one block pass: rows up to 16 KiB)
    if not args.no_copy_ceiling and graph is None and bound is None and 2 * wl.H <= 16384:
        def med_ms(fn):
            return median_event_ms(fn, stream)

        # Reference only, torch's own kernels on 1 GiB: a device-to-device copy
        # (read + write) and a fill (a pure write stream).
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        copy_ceiling = round(2 * (1 << 30) / (med_ms(lambda i: b.copy_(a)) * 1e-3) / 1e9, 1)
        fill_ceiling = round((1 << 30) / (med_ms(lambda i: b.fill_(0)) * 1e-3) / 1e9, 1)
        # Each call's own access pattern with no arithmetic (the
        # reference kernels of libep_ceiling.so), on the same rows, slots and
        # rotated sources: what the memory system gives that pattern here.
        from combine_ep_layout_10_amd import ceiling
        sp = stream.cuda_stream
        own_copy = round(2 * (1 << 30) / (med_ms(lambda i: ceiling.copy(a.data_ptr(), b.data_ptr(), 1 << 30, sp))
                                          * 1e-3) / 1e9, 1)
        del a, b
        hr = ops.layout(cfg, idx, w, workspace=ws)
        slots = hr.slot
        nvalid = int((slots >= 0).sum().item())
        smax = int(slots.max().item())
        H2 = 2 * wl.H

        def reference(n):
            """The plain kernel with call n's access pattern on its own rows:
            (kernel, pattern, bytes, median ms, destination, row bytes, rows)."""
            if n in ("dispatch", "combine_backward"):
                srcs = xs if n == "dispatch" else gos
                dst = recv if n == "dispatch" else grad_y
                drow = wl.H if (n == "dispatch" and fp8) else H2
                assert smax < dst.shape[0] and all(t.shape[0] == wl.T for t in srcs)
                ms = med_ms(lambda i: ceiling.broadcast(srcs[i % len(srcs)].data_ptr(), wl.T, H2, dst.data_ptr(),
                                                        drow, slots.data_ptr(), wl.k, sp))
                return ("k_broadcast<%d>" % (H2 // drow),
                        "each token's %d-byte row read (plain loads, rotated copies as in the steps) and stored to "
                        "its %d receive rows of %d bytes (row stores as the path's)" % (H2, wl.k, drow),
                        wl.T * H2 + nvalid * drow, ms, dst, drow, R)
            src = y if n == "combine" else grad_recv
            dst = out if n == "combine" else grad_x
            assert smax < src.shape[0] and dst.shape[0] == wl.T
            ms = med_ms(lambda i: ceiling.gather(src.data_ptr(), H2, slots.data_ptr(), wl.k, wl.T, dst.data_ptr(),
                                                 sp))
            return ("k_gather", "each token's %d receive rows of %d bytes read (streaming loads) and one row "
                    "written" % (wl.k, H2), nvalid * H2 + wl.T * H2, ms, dst, H2, wl.T)

        pattern = {}
        for n in names:
            ref_kernel, what, ref_bytes, ref_ms, dst, drow, wrows = reference(n)
            ref_gbps = ref_bytes / (ref_ms * 1e-3) / 1e9
            kern_gbps = dom_gbps if n == dominant else gbps[n]
            pattern[n] = {"kernel": ref_kernel, "pattern": what, "bytes": ref_bytes, "us": round(ref_ms * 1e3, 2),
                          "GBps": round(ref_gbps, 1), "frac_of_peak": round(ref_gbps / HBM_PEAK_GBPS, 4),
                          "call_frac_of_reference": round(kern_gbps / ref_gbps, 4)}
            if n == dominant:
                assert dst.numel() * dst.element_size() >= wrows * drow
                rw_ms = med_ms(lambda i: ceiling.write_rows(dst.data_ptr(), wrows, drow, sp))
                pattern[n]["row_writes_GBps"] = round(wrows * drow / (rw_ms * 1e-3) / 1e9, 1)
                pattern[n]["row_writes_bytes"] = wrows * drow
        pattern["copy_4KiB_blocks_1GiB_GBps"] = own_copy
        pattern["stat"] = ("median of 5 launches after one untimed; call_frac_of_reference: the call's rate (the "
                           "dominant's from the timed region, the others' from the evented pass) over the reference's")
        del hr, slots

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        y_h = y.view(torch.int16).cpu().numpy().view(np.uint16)
        if train:
            go_h = grad_out.view(torch.int16).cpu().numpy().view(np.uint16)
            gr_h = grad_recv.view(torch.int16).cpu().numpy().view(np.uint16)
            grw_h = grad_row_w.cpu().numpy()
        def run():
            lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, idx_h, w_h)
            if fp8:
                oracle.dispatch_fp8(lay, x_h, wl.k)
            else:
                oracle.dispatch_bf16(lay, x_h, wl.k)
            oracle.combine(lay, y_h, wl.k, w_h)
            if train:
                oracle.combine_backward_bf16(lay, go_h, wl.k, w_h)
                oracle.dispatch_backward(lay, gr_h, wl.k, grw_h)

        cpu = oracle_baseline(run, step_bytes, 1e9, "GB/s", args.cpu_budget_s,
                              "the full %s step (layout + %s dispatch + combine%s) on the same inputs"
                              % (wl.name, wl.dispatch, " + combine_backward + dispatch_backward" if train else ""))

    kernels = {"layout_us": round(lay_ms * 1e3, 2)}
    for n in names:
        kernels[n + "_us"] = round(k_ms[n] * 1e3, 2)
    kernels.update({"gpu_step_us": round(gpu_ms * 1e3, 2), "step_with_dispatch_forward_us": round(step_ev_ms * 1e3, 2),
                    "graph": bool(args.graph), "bound": bool(args.bound)})
    for n in names:
        kernels[n + "_GBps"] = round(gbps[n], 1)
        kernels[n + "_frac"] = round(gbps[n] / HBM_PEAK_GBPS, 4)
    kernels.update({"bytes": nbytes, "kernel_bytes": {kname[n]: nbytes[n] for n in names}, "kernel_hash": khash,
                    "cold_cache": flushed, "warm": warm, "copy_1GiB_GBps": copy_ceiling,
                    "fill_1GiB_GBps": fill_ceiling, "pattern_reference": pattern})
    # the dominant kernel against the rates measured in this run (a device
    # copy: half reads, half writes; a fill: writes only)
    for key, ceil in (("copy", copy_ceiling), ("fill", fill_ceiling)):
        kernels["dominant_frac_of_" + key] = round(dom_gbps / ceil, 4) if ceil else None
    if pattern is not None:
        # the dominant kernel against the simplest kernel with its access
        # pattern, timed in this run on the same rows
        roofline["pattern_reference"] = {k_: pattern[dominant][k_] for k_ in ("kernel", "GBps", "frac_of_peak",
                                                                              "call_frac_of_reference")}
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "step": "forward+backward" if train else "forward",
                   "launch": "graph" if args.graph else ("bound" if args.bound else "eager"), "tokens": wl.T,
                   "hidden": wl.H, "experts": wl.E, "topk": wl.k,
                   "expert_alignment": wl.A, "dests": wl.D, "mode": "fixed" if wl.mode else "compact",
                   "dispatch": "fp8_e4m3_1x128" if fp8 else "bf16", "combine": "bf16",
                   "backward": "bf16 weighted combine_backward, dispatch_backward with weight-grad gather"
                               if train else None, "routing": wl.routing},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


def bench_call(args):
    """One training call on the cached layout of a workload, K launches:
    ep_combine_weight_grad (grad_topk_w[t, j] = <grad_out[t], y[slot]>) or
    ep_combine_backward with FP8 output and pair weights (each pair's copy
    bf16(w * grad_out) quantised 1x128 with its own scales). Algorithmic
    bytes as for the path's calls; roofline against the HBM peak."""
    import numpy as np
    import torch
    from ep_workloads import WORKLOADS, draw_routing, draw_weights, _streams
    from combine_ep_layout_10_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]
    if wl.mode != ops.MODE_COMPACT or wl.H % 128:
        print("--step %s needs a COMPACT workload with hidden %% 128 == 0" % args.step, file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    sx, sr, sl, so, sy = _streams(0)
    idx_h = draw_routing(wl, sr)
    w_h = draw_weights(wl, sl)
    cfg = ops.Config(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.k, num_dests=wl.D,
                     expert_alignment=wl.A, capacity=wl.C, mode=wl.mode, idx_bits=64)
    R_cap = cfg.recv_rows_bound()
    idx = torch.from_numpy(idx_h).to(dev)
    w = torch.from_numpy(w_h).to(dev)
    h = ops.layout(cfg, idx, w)
    cnt, pad, R = h.read_counts()
    P = int(cnt.sum())
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    grad_out = torch.randn((wl.T, wl.H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    # grad_out (read with plain loads) cycles through copies, as in the path's
    # steps, so each call reads it from HBM
    nrot = max(1, args.rotate)
    gos = [grad_out] + [grad_out.clone() for _ in range(nrot - 1)]
    cur = [0]
    T, H, k = wl.T, wl.H, wl.k
    if args.step == "weight_grad":
        y = torch.randn((R_cap, H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        gw = torch.empty((T, k), dtype=torch.float32, device=dev)

        def call():
            ops.combine_weight_grad(h, gos[cur[0] % nrot], y, gw)
        # grad_out and the pairs' rows of y in, slots in, one float per pair out
        nbytes = T * H * 2 + P * H * 2 + T * k * 4 + T * k * 4
        kname, what = "k_weight_grad", "ep_combine_weight_grad"
    else:
        gq = torch.empty((R_cap, H), dtype=torch.uint8, device=dev)
        gs = torch.empty((R_cap, H // 128), dtype=torch.float32, device=dev)

        def call():
            ops.combine_backward(h, gos[cur[0] % nrot], ops.FP8_QUANTIZE, w, grad_y=gq, grad_y_scales=gs)
        # grad_out, slots and weights in; every row (pairs and zero padding)
        # with its 1x128 scales out
        nbytes = T * H * 2 + T * k * 4 + T * k * 4 + R * (H + 4 * (H // 128))
        kname, what = "k_dispatch<4>", "ep_combine_backward (FP8, weighted)"
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        calib_copy(dev)
    for i in range(args.warmup):
        cur[0] = i
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (e0, e1) in enumerate(ev):
        cur[0] = args.warmup + i
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    khash = kernel_hash()
    pattern = None
    if not args.no_copy_ceiling and 2 * H <= 16384:
        # the call's access pattern with no arithmetic (libep_ceiling.so), on
        # the same rows: FP8 backward, each grad_out row (rotated copies)
        # stored to its pairs' rows at FP8 width; weight_grad, the rows it
        # reads as plain streams (y's receive rows and grad_out's rows)
        from combine_ep_layout_10_amd import ceiling
        sp = stream.cuda_stream
        slots = h.slot
        assert int(slots.max().item()) < R_cap
        if args.step == "fp8_backward":
            ref_ms = median_event_ms(lambda i: ceiling.broadcast(gos[i % nrot].data_ptr(), T, 2 * H, gq.data_ptr(), H,
                                                                 slots.data_ptr(), k, sp), stream)
            ref_bytes = T * 2 * H + P * H
            ref_kernel, ref_what = "k_broadcast<2>", ("each grad_out row (%d bytes) read and stored to its %d pairs' "
                                                      "rows of %d bytes" % (2 * H, k, H))
        else:
            sink = torch.zeros((1,), dtype=torch.int32, device=dev)
            ref_ms = median_event_ms(lambda i: (ceiling.read_rows(y.data_ptr(), R, 2 * H, sink.data_ptr(), sp),
                                                ceiling.read_rows(gos[i % nrot].data_ptr(), T, 2 * H, sink.data_ptr(),
                                                                  sp)), stream)
            ref_bytes = (R + T) * 2 * H
            ref_kernel, ref_what = "k_read_rows", ("the %d receive rows of y and the %d rows of grad_out read "
                                                   "in order (streaming loads)" % (R, T))
        ref_gbps = ref_bytes / (ref_ms * 1e-3) / 1e9
        pattern = {"kernel": ref_kernel, "pattern": ref_what, "bytes": ref_bytes, "us": round(ref_ms * 1e3, 2),
                   "GBps": round(ref_gbps, 1), "frac_of_peak": round(ref_gbps / HBM_PEAK_GBPS, 4),
                   "call_frac_of_reference": round(achieved / ref_gbps, 4),
                   "stat": "median of 5 launches after one untimed"}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, idx_h, w_h)
        go_h = grad_out.view(torch.int16).cpu().numpy().view(np.uint16)
        if args.step == "weight_grad":
            y_h = y.view(torch.int16).cpu().numpy().view(np.uint16)
            run = lambda: oracle.combine_weight_grad(lay, go_h, y_h, wl.k)
        else:
            run = lambda: oracle.combine_backward_fp8(lay, go_h, wl.k, w_h)
        cpu = oracle_baseline(run, nbytes, 1e9, "GB/s", args.cpu_budget_s,
                              "the same %s call on the same inputs" % what)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name + "_" + args.step, "call": what, "tokens": T, "hidden": H,
                   "experts": wl.E, "topk": k, "expert_alignment": wl.A, "routing": wl.routing},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(kname, khash, wl.name + "_" + args.step),
                     "kernel": kname, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(launch_ms * 1e3, 2), "timed": "events in the timed region",
                     "inputs": "grad_out cycled through %d copies" % nrot, "pattern_reference": pattern},
        "cpu_baseline": cpu,
        "kernels": {"kernel_bytes": {kname: nbytes}, "kernel_hash": khash, "pairs": P, "rows": R},
    }
    print(json.dumps(res), flush=True)


def bench_gemm(args):
    """The FP8 grouped GEMM over the receive layout of a workload: its FP8
    dispatch output [rows, H] (1x128 scales) times a seeded random E4M3 weight
    matrix [N, H] per expert (128x128 scales). One step = one GEMM launch.
    Algorithmic flops = 2 * pairs * N * H (the routed rows; padding rows of
    the aligned layout are computed too and reported separately)."""
    import numpy as np
    import torch
    from ep_workloads import WORKLOADS, draw_routing, draw_weights, draw_hidden, _streams
    from combine_ep_layout_10_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]
    if wl.dispatch != "fp8":
        print("--step gemm needs an FP8 workload (v3, skewed_v3, skewed_v3_s06, decode)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    N, H = args.gemm_n, wl.H
    sx, sr, sl, so, sy = _streams(0)
    x_h = draw_hidden(wl, sx, so)
    idx_h = draw_routing(wl, sr)
    cfg = ops.Config(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.k, num_dests=wl.D,
                     expert_alignment=wl.A, capacity=wl.C, mode=wl.mode, idx_bits=64)
    x = torch.from_numpy(x_h.view(np.int16)).view(torch.bfloat16).to(dev)
    h, q, s = ops.dispatch_forward(cfg, torch.from_numpy(idx_h).to(dev), x, ops.FP8_QUANTIZE)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    c = torch.randint(0, 254, (wl.E, N, H), dtype=torch.uint8, device=dev, generator=gen)
    b = torch.where(c >= 0x7F, c + 1, c)          # every E4M3FN code but the NaN patterns
    del c
    sb = torch.rand((wl.E, N // 128, H // 128), device=dev, generator=gen) * 1e-2 + 1e-3
    out = torch.empty((cfg.recv_rows_bound(), N), dtype=torch.bfloat16, device=dev)
    cnt, pad, R = h.read_counts()
    pairs = int(cnt.sum()) if wl.mode == 0 else int(pad.sum())
    rows = R if wl.mode == 0 else int(sum(-(-p // 128) * 128 for p in pad))
    flops = 2.0 * pairs * N * H
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        calib_copy(dev)
    for _ in range(args.warmup):
        ops.grouped_gemm_fp8(h, q, s, b, sb, out=out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        ops.grouped_gemm_fp8(h, q, s, b, sb, out=out)
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = float(np.mean([a.elapsed_time(b_) for a, b_ in ev]))
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        qh, sh = q.cpu().numpy(), s.cpu().numpy()
        off = h.expert_off.cpu().numpy()
        rng = np.random.default_rng(0)
        # 64 random routed rows, each with one random 128-channel piece of its
        # expert's weights, packed as a grouped GEMM of 64 one-row experts
        # (inputs copied to the host before the timed runs)
        ns = 64
        a1 = np.zeros((ns, H), np.uint8)
        s1 = np.zeros((ns, H // 128), np.float32)
        b1 = np.zeros((ns, 128, H), np.uint8)
        sb1 = np.zeros((ns, 1, H // 128), np.float32)
        for i in range(ns):
            r = int(rng.integers(0, int(off[-1])))
            n0 = int(rng.integers(0, N // 128)) * 128
            e = int(np.searchsorted(off, r, side="right") - 1)
            a1[i], s1[i] = qh[r], sh[r]
            b1[i] = b[e, n0:n0 + 128].cpu().numpy()
            sb1[i, 0] = sb[e, n0 // 128].cpu().numpy()
        rb = np.arange(ns, dtype=np.int32)
        re_ = rb + 1
        pairs_ = np.stack([np.repeat(np.arange(ns), 128), np.tile(np.arange(128), ns)], axis=1).astype(np.int64)

        def run():
            oracle.grouped_gemm_fp8(rb, re_, a1, s1, b1, sb1, pairs=pairs_)

        cpu = oracle_baseline(run, 2.0 * len(pairs_) * H, 1e12, "TFLOP/s", args.cpu_budget_s,
                              "%d outputs (128-channel pieces of %d random routed rows) of the same GEMM in "
                              "binary64" % (len(pairs_), ns))
    kname = "k_grouped_gemm_fp8_dma" if N % 256 == 0 and H // 128 <= 256 else "k_grouped_gemm_fp8"
    # the least HBM traffic of one launch: weights and A rows (with scales)
    # read once, the output rows written once
    floor_bytes = wl.E * N * H + wl.E * (N // 128) * (H // 128) * 4 + rows * (H + 4 * H // 128) + rows * N * 2
    khash = kernel_hash("gemm")
    res = {
        "metric": "FP8 grouped GEMM TFLOP/s on the receive layout", "value": round(tflops, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 x fp8_e4m3 -> f32",
        "data": "synthetic",
        "config": {"workload": wl.name + "_gemm", "tokens": wl.T, "hidden": H, "experts": wl.E, "topk": wl.k,
                   "n": N, "pairs": pairs, "rows_computed": rows, "expert_alignment": wl.A},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": 5000.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 5000.0, 4), "traffic": load_traffic(kname, khash, wl.name + "_gemm"),
                     "kernel": kname,
                     "algorithmic_flops_per_launch": flops, "avg_launch_us": round(launch_ms * 1e3, 1),
                     "timed": "events in the timed region"},
        "cpu_baseline": cpu,
        "kernels": {"computed_rows_TFLOPs": round(2.0 * rows * N * H / (launch_ms * 1e-3) / 1e12, 1),
                    "weight_bytes": wl.E * N * H, "kernel_bytes": {kname: floor_bytes},
                    "hbm_floor_us": round(floor_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6, 1),
                    "kernel_hash": khash},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
