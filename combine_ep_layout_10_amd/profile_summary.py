"""Summaries of rocprofv3 output for the kernels of this library.

Two reports, both written as short text under profiles/:

  trace    per-kernel call count and average / min / max duration from a
           `rocprofv3 --kernel-trace --stats` run (its *_kernel_stats.csv);
  traffic  HBM bytes per launch from two `rocprofv3 --pmc` runs, one with
           FETCH_SIZE and one with WRITE_SIZE (their *_counter_collection.csv).
           Both counters are in KiB per dispatch. They are calibrated on the
           1 GiB device-to-device copy that `bench.py --calib-copy` runs
           (the largest `__amd_rocclr_copyBuffer` dispatches, 2^30 bytes read
           and written): scale = 2^30 B / counter bytes for that copy. The
           scaled bytes of each kernel are set against the algorithmic bytes
           `bench.py` reports for the same workload (for the grouped GEMM:
           its HBM floor, weights and A read once, output written once), and
           also stored in
           profiles/traffic.json (by workload, then kernel), which
           `bench.py` reads for `roofline.traffic` while the kernel sources
           are unchanged.

    python -m combine_ep_layout_10_amd.profile_summary trace STATS_CSV --workload v3 \\
        --command "..." --bench-json BENCH.json --out profiles/NAME.md
    python -m combine_ep_layout_10_amd.profile_summary traffic --fetch FETCH_CSV --write WRITE_CSV \\
        --workload v3 --command-fetch "..." --command-write "..." --bench-json BENCH.json \\
        --out profiles/NAME.md --json profiles/traffic.json
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re

COPY_KERNEL = "__amd_rocclr_copyBuffer"
REF_NS = "ep_ceiling::"
GIB = 1 << 30


def short_name(full: str) -> str:
    """`void ep::k_combine<true>(ep::CombineArgs)` -> `ep::k_combine<true>`."""
    n = re.sub(r"^void ", "", full.strip())
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def kernel_key(name: str) -> str:
    """Key in traffic.json: the kernel name without the namespace, template
    arguments kept (`ep::k_dispatch<2>` -> `k_dispatch<2>`): one kernel
    template serves several calls (the FP8 dispatch and the weighted BF16
    combine_backward are both k_dispatch)."""
    n = short_name(name)
    return n[len("ep::"):] if n.startswith("ep::") else n


def read_stats(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return rows


def read_counter(path: str, counter: str):
    """Per kernel name: list of (grid size, value in KiB) per dispatch."""
    out = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out[short_name(r["Kernel_Name"])].append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def copy_scale(per_kernel) -> tuple:
    """Scale factor from the 1 GiB copies: the copyBuffer dispatches with the
    largest counter value. (Other copies of the run, such as the benchmark's
    copies of its inputs, use the same grid but move far fewer bytes, so the
    grid size does not single out the 1 GiB copies.) Every copy within 1 % of
    the largest value is one of them."""
    copies = per_kernel.get(COPY_KERNEL, [])
    if not copies:
        raise SystemExit("no %s dispatch found: run bench.py with --calib-copy" % COPY_KERNEL)
    top = max(v for _, v in copies)
    vals = [v for _, v in copies if v >= 0.99 * top]
    kib = sum(vals) / len(vals)
    return GIB / (kib * 1024.0), kib


def load_bench(path: str) -> dict:
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)
    raise SystemExit("no JSON line in %s" % path)


def cmd_trace(a) -> None:
    rows = read_stats(a.stats)
    bench = load_bench(a.bench_json) if a.bench_json else None
    lines = ["# Kernel trace: %s" % a.workload, "",
             "Command (run from the repository root, MI355X, ROCm 7.2):", "", "    " + a.command, ""]
    if bench:
        lines += ["Kernel sources hash (as bench.py reports it): `%s`" % bench["kernels"]["kernel_hash"], ""]
    lines += ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, avg, mn, mx in sorted(rows, key=lambda r: -r[1] * r[2]):
        if not (name.startswith("ep::") or name.startswith(REF_NS)) and not a.all:
            continue
        lines.append("| %s | %d | %.2f | %.2f | %.2f |" % (name, calls, avg, mn, mx))
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a) -> None:
    fetch = read_counter(a.fetch, "FETCH_SIZE")
    write = read_counter(a.write, "WRITE_SIZE")
    fs, fcopy = copy_scale(fetch)
    ws, wcopy = copy_scale(write)
    bench = load_bench(a.bench_json)
    khash = bench["kernels"]["kernel_hash"]
    # algorithmic (or least) bytes per launch of each kernel the bench line
    # measures: the path's calls, or the grouped GEMM's HBM floor
    alg = dict(bench["kernels"].get("kernel_bytes", {}))
    stored = set(alg)
    # the access-pattern reference kernels the bench line timed beside the
    # path (libep_ceiling.so), against the bytes it credits them with
    ref = bench["kernels"].get("pattern_reference") or {}
    for v in ref.values():
        if isinstance(v, dict):
            alg.setdefault(REF_NS + v["kernel"], v["bytes"])
            if "row_writes_bytes" in v:
                alg[REF_NS + "k_write_rows"] = v["row_writes_bytes"]
    if ref:
        alg[REF_NS + "k_copy"] = 2 * GIB
    table = {}
    for name in sorted(set(fetch) | set(write)):
        if not name.startswith("ep::") and kernel_key(name) not in alg:
            continue
        fk = [v for _, v in fetch.get(name, [])]
        wk = [v for _, v in write.get(name, [])]
        if not fk or not wk:
            continue
        f_kib = sum(fk) / len(fk)
        w_kib = sum(wk) / len(wk)
        table[name] = (f_kib, w_kib, int(round(f_kib * 1024 * fs + w_kib * 1024 * ws)))
    lines = ["# HBM traffic per launch: %s" % a.workload, "",
             "Commands (one counter per run, from the repository root):", "",
             "    " + a.command_fetch, "    " + a.command_write, "",
             "Kernel sources hash: `%s`" % khash, "",
             "Calibration: `--calib-copy` runs a plain 1 GiB device-to-device copy (`%s`, "
             "1,073,741,824 B read and written)." % COPY_KERNEL,
             "FETCH_SIZE reads %.1f KiB and WRITE_SIZE %.1f KiB for it, so the scale factors are "
             "%.3f (fetch) and %.3f (write)." % (fcopy, wcopy, fs, ws), "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|"]
    out_json = {}
    if a.json and os.path.exists(a.json):
        with open(a.json) as f:
            out_json = json.load(f)
    for name, (f_kib, w_kib, nbytes) in table.items():
        key = kernel_key(name)
        al = alg.get(key)
        ratio = "%.3f" % (nbytes / al) if al else "-"
        lines.append("| %s | %.1f | %.1f | %d | %s | %s |" % (name, f_kib, w_kib, nbytes, al if al else "-", ratio))
        if key not in stored:
            continue  # set-up and reference kernels of this run: listed, not stored
        # by workload, then kernel: one kernel runs in several workloads' steps
        out_json.setdefault(a.workload, {})[key] = {
            "bytes_per_launch": nbytes, "fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "kernel_hash": khash, "workload": a.workload}
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if a.json:
        with open(a.json, "w") as f:
            json.dump(out_json, f, indent=1, sort_keys=True)
    print("\n".join(lines))


def main(argv=None) -> None:
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = p.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--bench-json")
    t.add_argument("--all", action="store_true", help="also list kernels outside this library")
    t.add_argument("--out", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--command-fetch", required=True)
    r.add_argument("--command-write", required=True)
    r.add_argument("--bench-json", required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--json")
    a = p.parse_args(argv)
    if a.what == "trace":
        cmd_trace(a)
    else:
        cmd_traffic(a)


if __name__ == "__main__":
    main()
