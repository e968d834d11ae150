"""Host-side measurement logic (no GPU): the algorithmic byte counts the
benchmark divides by, and the rocprofv3 summaries (kernel-name parsing,
copy-calibrated traffic scaling, which kernels traffic.json records)."""
import csv
import json
import os

import pytest

import bench
from combine_ep_layout_10_amd import profile_summary as ps
from ep_workloads import WORKLOADS


def test_v3_algorithmic_bytes_by_hand():
    """V3: 8192 tokens x 7168, top-8, 65,536 pairs, 80,768 aligned rows
    (15,232 of padding); every term written out by hand."""
    wl = WORKLOADS["v3"]
    T, H, k, P, R = 8192, 7168, 8, 65536, 80768
    b = bench.algorithmic_bytes(wl, R, P, "fp8", train=True)
    row_fp8 = H + 4 * (H // 128)                              # codes + 56 scales
    assert b["dispatch"] == T * H * 2 + T * k * 4 + R * row_fp8
    assert b["dispatch"] == 714_739_712
    assert b["combine"] == P * H * 2 + 2 * T * k * 4 + T * H * 2 == 1_057_488_896
    assert b["combine_backward"] == T * H * 2 + 2 * T * k * 4 + R * 2 * H == 1_275_854_848
    assert b["dispatch_backward"] == P * H * 2 + T * k * 4 + T * H * 2 + P * 4 + T * k * 4
    assert b["padding_rows"] == R - P == 15_232
    fwd = bench.algorithmic_bytes(wl, R, P, "fp8")
    assert "combine_backward" not in fwd and fwd["combine"] == b["combine"]


def test_fixed_mode_has_no_padding_bytes():
    wl = WORKLOADS["decode"]
    b = bench.algorithmic_bytes(wl, 256 * 128, 1024, "fp8")
    assert b["padding_rows"] == 0
    assert b["dispatch"] == 128 * 7168 * 2 + 128 * 8 * 4 + 1024 * (7168 + 4 * 56)


def test_kernel_names():
    full = "void ep::k_combine<true>(ep::CombineArgs)"
    assert ps.short_name(full) == "ep::k_combine<true>"
    assert ps.kernel_key(full) == "k_combine<true>"
    assert ps.kernel_key("void ep::k_layout_dispatch_small<1, 2>(ep::LayoutArgs, ep::DispatchArgs)") == \
        "k_layout_dispatch_small<1, 2>"
    assert ps.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for name, grid, val in rows:
            w.writerow([name, grid, counter, val])


def test_traffic_scaling_and_recorded_kernels(tmp_path):
    """The 1 GiB copy fixes the scale (FETCH reads half the bytes here, WRITE
    all of them); only kernels the bench line names are stored, under
    their template-qualified names and the bench's source hash."""
    copy = "__amd_rocclr_copyBuffer"
    disp = "void ep::k_dispatch<1>(ep::DispatchArgs)"
    setup = "void ep::k_layout_count(ep::LayoutArgs)"
    gib_kib = (1 << 30) / 1024
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 4096, 1.0), (copy, 1 << 20, gib_kib / 2),
                                                     (disp, 99, 1000.0), (disp, 99, 1002.0), (setup, 8, 3.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1 << 20, gib_kib), (disp, 99, 5000.0), (setup, 8, 1.0)])
    line = {"kernels": {"kernel_hash": "abc", "kernel_bytes": {"k_dispatch<1>": 7_000_000}}}
    (tmp_path / "b.log").write_text("[bench] noise\n" + json.dumps(line) + "\n")
    out_json = tmp_path / "traffic.json"
    out_json.write_text(json.dumps({"w": {"k_combine<true>": {"bytes_per_launch": 1, "kernel_hash": "old"}},
                                    "v": {"k_dispatch<1>": {"bytes_per_launch": 2, "kernel_hash": "abc"}}}))
    ps.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
             "--workload", "w", "--command-fetch", "cf", "--command-write", "cw",
             "--bench-json", str(tmp_path / "b.log"), "--out", str(tmp_path / "t.md"), "--json", str(out_json)])
    t = json.loads(out_json.read_text())
    assert set(t["w"]) == {"k_combine<true>", "k_dispatch<1>"}   # set-up kernel listed in the table, not stored
    e = t["w"]["k_dispatch<1>"]
    assert e["kernel_hash"] == "abc" and e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["bytes_per_launch"] == round((1001.0 * 2 + 5000.0) * 1024)
    assert t["w"]["k_combine<true>"]["kernel_hash"] == "old"     # other entries are kept
    assert t["v"]["k_dispatch<1>"]["bytes_per_launch"] == 2       # the same kernel in another workload too
    md = (tmp_path / "t.md").read_text()
    assert "ep::k_layout_count" in md and "| 7000000 |" in md


def test_copy_scale_ignores_smaller_copies_on_the_same_grid(tmp_path):
    """The benchmark's copies of its inputs run as copyBuffer dispatches with
    the same grid as the 1 GiB calibration copy; only the largest counter
    values (the 1 GiB copies) set the scale."""
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = (1 << 30) / 1024
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 131072, 114688.0)] * 6 +
                 [(copy, 512, 1.0), (copy, 131072, gib_kib), (copy, 131072, gib_kib * 1.001)])
    scale, kib = ps.copy_scale(ps.read_counter(str(tmp_path / "w.csv"), "WRITE_SIZE"))
    assert abs(kib - gib_kib * 1.0005) < 1e-6 * gib_kib
    assert abs(scale - 1 / 1.0005) < 1e-9


def test_traffic_needs_the_copy(tmp_path):
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("void ep::k_combine<true>(ep::CombineArgs)", 1, 1.0)])
    with pytest.raises(SystemExit):
        ps.copy_scale(ps.read_counter(str(tmp_path / "f.csv"), "FETCH_SIZE"))


def test_trace_summary(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void ep::k_combine<true>(ep::CombineArgs)", 4, 800000, 200000.0, 50, 190000, 210000, 1])
        w.writerow(["void at::native::fill(int)", 9, 90, 10.0, 1, 9, 11, 0])
    rows = ps.read_stats(str(p))
    assert rows[0] == ("ep::k_combine<true>", 4, 200.0, 190.0, 210.0)
    ps.main(["trace", str(p), "--workload", "w", "--command", "c", "--out", str(tmp_path / "o.md")])
    md = (tmp_path / "o.md").read_text()
    assert "| ep::k_combine<true> | 4 | 200.00 | 190.00 | 210.00 |" in md
    assert "at::native" not in md                               # only this library's kernels


def test_kernel_hash_tracks_step_sources():
    assert bench.kernel_hash("path") != bench.kernel_hash("gemm")
    for step, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(bench.ROOT, "combine_ep_layout_10_amd", "csrc", f)), (step, f)


def test_traffic_lists_reference_kernels(tmp_path):
    """The access-pattern reference kernels of the bench line are listed
    against the bytes the line credits them with, and never stored."""
    copy = "__amd_rocclr_copyBuffer"
    bc = "void ep_ceiling::k_broadcast<1>(char const*, int, char*, int, int const*, int)"
    wr = "void ep_ceiling::k_write_rows(char*, int)"
    gib_kib = (1 << 30) / 1024
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 1 << 20, gib_kib / 2), (bc, 9, 500.0), (wr, 9, 0.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1 << 20, gib_kib), (bc, 9, 4000.0), (wr, 9, 2000.0)])
    ref = {"combine_backward": {"kernel": "k_broadcast<1>", "bytes": 5000 * 1024, "row_writes_bytes": 2000 * 1024},
           "stat": "x"}
    line = {"kernels": {"kernel_hash": "abc", "kernel_bytes": {"k_dispatch<1>": 7}, "pattern_reference": ref}}
    (tmp_path / "b.log").write_text(json.dumps(line) + "\n")
    out_json = tmp_path / "traffic.json"
    ps.main(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
             "--workload", "w", "--command-fetch", "cf", "--command-write", "cw",
             "--bench-json", str(tmp_path / "b.log"), "--out", str(tmp_path / "t.md"), "--json", str(out_json)])
    md = (tmp_path / "t.md").read_text()
    assert "| ep_ceiling::k_broadcast<1> | 500.0 | 4000.0 | %d | %d | 1.000 |" % (5000 * 1024, 5000 * 1024) in md
    assert "| ep_ceiling::k_write_rows | 0.0 | 2000.0 |" in md
    assert json.loads(out_json.read_text()) == {}


def test_traffic_only_for_the_measured_workload_and_sources(tmp_path):
    """Counter bytes are reported only for the workload and kernel sources
    they were taken on: a launch's bytes depend on its shape."""
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"v3": {"k_combine<true>": {"bytes_per_launch": 123, "kernel_hash": "abc",
                                                        "workload": "v3"}},
                             "mid": {"k_combine<true>": {"bytes_per_launch": 45, "kernel_hash": "abc",
                                                         "workload": "mid"}}}))
    assert bench.load_traffic("k_combine<true>", "abc", "v3", str(p)) == 123
    assert bench.load_traffic("k_combine<true>", "abc", "mid", str(p)) == 45
    assert bench.load_traffic("k_combine<true>", "abc", "decode", str(p)) is None
    assert bench.load_traffic("k_combine<true>", "abd", "v3", str(p)) is None
    assert bench.load_traffic("k_combine<false>", "abc", "v3", str(p)) is None
    assert bench.load_traffic("k_combine<true>", "abc", "v3", str(tmp_path / "missing.json")) is None


def test_host_threads_respects_affinity_and_cap(monkeypatch):
    n_aff = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.host_threads() == n_aff
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    assert bench.host_threads() == min(2, n_aff)
    monkeypatch.setenv("OMP_NUM_THREADS", "junk")
    assert bench.host_threads() == n_aff


def test_oracle_baseline_reports_threads_and_single_core(monkeypatch):
    """Both legs run the same work; `cores` is the thread count the OpenMP
    build reports, the plain build's figure sits under single_core."""
    import numpy as np
    import oracle
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    wl = WORKLOADS["tiny"]
    from ep_workloads import make_inputs
    inp = make_inputs(wl)
    lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, inp["topk_idx"], inp["topk_w"])
    seen = []

    def run():
        seen.append(oracle.combine(lay, inp["y"], wl.k, inp["topk_w"])[0])

    res = bench.oracle_baseline(run, 1e6, 1e9, "GB/s", 0.2, "tiny combine")
    assert res["cores"] == min(2, len(os.sched_getaffinity(0)))
    assert res["single_core"]["cores"] == 1
    assert res["value"] > 0 and res["single_core"]["value"] > 0
    assert all(np.array_equal(seen[0], s) for s in seen)
    assert oracle.threads(0) == 1
