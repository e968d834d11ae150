"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: layout, slots, copies, FP8 codes and scales bit-exact; combine within
1 bf16 ulp (bit-exact expected: both sides sum in binary32 with fused
multiply-add in k order). All five workloads run at their full sizes, in the
launch configuration the benchmark uses."""
import numpy as np
import pytest
import torch

import oracle
from ep_workloads import WORKLOADS, make_inputs, random_routing_table, f32_to_bf16_bits, bf16_bits_to_f32
from gpu_common import (log, to_dev, to_dev_bf16, bf16_host, host, cfg_of, workload_case, written_rows,
                        bf16_ulp_distance, compare_layout)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from combine_ep_layout_10_amd import ops


def _run_small(T, H, E, k, A=1, D=1, C=0, mode=0, seed=0, masked=0.0, bad=0.0, distinct=True,
               idx_bits=64, flags=0, dispatch="bf16", weights=True, forward=False, table=None):
    """Random small case through every stage, checked against the oracle.
    forward=True builds the layout and dispatches with one ep_dispatch_forward
    call instead of ep_layout + ep_dispatch; table: a given routing table
    instead of a random one."""
    log("case T=%d H=%d E=%d k=%d A=%d D=%d C=%d mode=%d idx_bits=%d dispatch=%s seed=%d forward=%d table=%s"
        % (T, H, E, k, A, D, C, mode, idx_bits, dispatch, seed, forward, table is not None))
    rng = np.random.default_rng(seed)
    if table is None:
        idx = random_routing_table(rng, T, E, k, masked_frac=masked, bad_frac=bad, distinct=distinct)
    else:
        idx = np.ascontiguousarray(table, dtype=np.int64)
        assert idx.shape == (T, k)
    if idx_bits == 32:
        idx = idx.astype(np.int32)
    w = rng.random((T, k)).astype(np.float32) if weights else None
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = oracle.layout(mode, T, E, k, A, D, C, idx, w)
    cfg = ops.Config(max_tokens=max(T, 1), hidden=H, num_experts=E, num_topk=k, num_dests=D,
                     expert_alignment=A, capacity=C, mode=mode, idx_bits=idx_bits, flags=flags)
    R = cfg.recv_rows_bound()
    dev_w = None if w is None else to_dev(w)
    if dispatch == "bf16":
        recv = torch.full((R, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        rs = None
    else:
        recv = torch.full((R, H), 0xEE, dtype=torch.uint8, device="cuda")
        rs = torch.full((R, H // 128), -7.0, dtype=torch.float32, device="cuda")
    dt = ops.BF16 if dispatch == "bf16" else ops.FP8_QUANTIZE
    if forward:
        h = ops.dispatch_forward(cfg, to_dev(idx), to_dev_bf16(x), dt, topk_w=dev_w, recv=recv, recv_scales=rs)[0]
    else:
        h = ops.layout(cfg, to_dev(idx), dev_w)
    compare_layout(h, lay, weights=w is not None)
    rows = written_rows(lay)
    zero_pad = not (flags & ops.FLAG_NO_ZERO_PAD)
    if mode == oracle.MODE_COMPACT and not zero_pad:
        rows = rows[lay["row_src"][rows] >= 0]
    if dispatch == "bf16":
        ref = oracle.dispatch_bf16(lay, x, k, zero_pad=zero_pad)
        if not forward:
            ops.dispatch(h, to_dev_bf16(x), ops.BF16, recv=recv)
        got = bf16_host(recv)
        assert np.array_equal(got[rows], ref[rows])
        untouched = np.setdiff1d(np.arange(R), rows)
        assert np.all(got[untouched] == 0xFFFF)
    else:
        q, s = oracle.dispatch_fp8(lay, x, k, zero_pad=zero_pad)
        if not forward:
            ops.dispatch(h, to_dev_bf16(x), ops.FP8_QUANTIZE, recv=recv, recv_scales=rs)
        assert np.array_equal(host(recv)[rows], q[rows])
        assert np.array_equal(host(rs)[rows].view(np.uint32), s[rows].view(np.uint32))
        untouched = np.setdiff1d(np.arange(R), rows)
        assert np.all(host(recv)[untouched] == 0xEE)
    # combine over random expert outputs
    y = f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    out_ref, vals_ref = oracle.combine(lay, y, k, w, row_vals=lay["row_w"] if w is not None else None)
    res = ops.combine(h, to_dev_bf16(y), None if w is None else to_dev(w),
                      row_vals=h.row_w if w is not None else None)
    out = res[0] if w is not None else res
    got = bf16_host(out)
    assert bf16_ulp_distance(got, out_ref).max(initial=0) <= 1
    assert np.array_equal(got, out_ref), "combine differs from the oracle (within 1 ulp)"
    if w is not None:
        assert np.array_equal(host(res[1]).view(np.uint32), vals_ref.view(np.uint32))
    return h, lay


# ---------------------------------------------------------------- small cases

def test_tiny_hand_example():
    _run_small(3, 256, 4, 2, A=2, D=2, seed=1)


@pytest.mark.parametrize("T,E,k,A,D", [
    (1, 16, 2, 1, 1), (37, 8, 3, 4, 2), (128, 16, 2, 1, 1), (300, 24, 5, 7, 3),
    (819, 64, 5, 128, 4),        # P = 4095: single-block path
    (820, 64, 5, 128, 4),        # P = 4100: multi-block path
    (2049, 600, 2, 8, 6),        # E > 512: multi-block path with few pairs
    (5000, 1024, 7, 3, 32),      # largest E; per-block count matrix too big to re-read: 3 kernels
    (16384, 256, 8, 128, 8),     # 128 count blocks x 256 experts: the largest matrix reduced inline
    (16400, 256, 8, 128, 8),     # 129 count blocks: one-block scan launch
    (40000, 256, 4, 16, 8),      # many count blocks, 3 kernels
    (50, 4, 2, 1000, 2),         # alignment 1000: 250 zero-fill blocks per expert, most rows padding
])
def test_random_layouts(T, E, k, A, D):
    _run_small(T, 64, E, k, A=A, D=D, seed=T + E)


def _layout_every_table(mode, T, E, k, A, D, C, tables, forward=False):
    """One ep_layout launch per routing table, each into its own slice of one
    workspace, one synchronisation, then every table's layout against the
    oracle (which equals the O(P^2) brute-force definition on these same
    tables: tests/test_oracle_layout.py). forward=True builds each layout with
    ep_dispatch_forward (BF16) instead and also checks every table's receive
    rows: the token's row where the layout puts a pair, untouched elsewhere."""
    n = len(tables)
    log("every table: mode=%d T=%d E=%d k=%d A=%d D=%d C=%d forward=%d, %d tables"
        % (mode, T, E, k, A, D, C, forward, n))
    cfg = ops.Config(max_tokens=T, hidden=128, num_experts=E, num_topk=k, num_dests=D,
                     expert_alignment=A, capacity=C, mode=mode)
    ws = -(-cfg.workspace_bytes() // 256) * 256
    big = torch.empty(n * ws, dtype=torch.uint8, device="cuda")
    idx_all = to_dev(np.ascontiguousarray(np.asarray(tables, np.int64)))
    w = ((np.arange(T * k, dtype=np.float32) + 1) / 8).reshape(T, k)
    w_dev = to_dev(w)
    Rb = cfg.recv_rows_bound()
    if forward:
        x = f32_to_bf16_bits(np.random.default_rng(T * 100 + C).standard_normal((T, 128)).astype(np.float32))
        x_dev = to_dev_bf16(x)
        recv_all = torch.full((n, Rb, 128), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        handles = [ops.dispatch_forward(cfg, idx_all[i], x_dev, ops.BF16, topk_w=w_dev,
                                        workspace=big[i * ws:(i + 1) * ws], recv=recv_all[i])[0] for i in range(n)]
    else:
        handles = [ops.layout(cfg, idx_all[i], w_dev, workspace=big[i * ws:(i + 1) * ws]) for i in range(n)]
    torch.cuda.synchronize()
    recv_host = bf16_host(recv_all) if forward else None
    whole = big.cpu().numpy()
    base = big.data_ptr()

    def field(ptr, count, dt):
        off = ptr - base
        return whole[off: off + count * np.dtype(dt).itemsize].view(dt)

    for i, (h, tab) in enumerate(zip(handles, tables)):
        lay = oracle.layout(mode, T, E, k, A, D, C, np.asarray(tab, np.int64), w)
        c = h.c
        got = {"cnt": field(c.cnt, E, np.int32), "pad": field(c.pad, E, np.int32),
               "expert_off": field(c.expert_off, E + 1, np.int32), "dest_off": field(c.dest_off, D + 1, np.int32),
               "dest_tokens": field(c.dest_tokens, D, np.int32), "slot": field(c.slot, T * k, np.int32)}
        for key, val in got.items():
            assert np.array_equal(val, lay[key]), (i, tab, key)
        assert int(field(c.err_flags, 1, np.int32)[0]) == lay["flags"], (i, tab)
        rows = written_rows(lay)
        assert np.array_equal(field(c.row_src, Rb, np.int32)[rows], lay["row_src"][rows]), (i, tab)
        assert np.array_equal(field(c.row_w, Rb, np.float32)[rows].view(np.uint32),
                              lay["row_w"][rows].view(np.uint32)), (i, tab)
        if forward:
            ref = oracle.dispatch_bf16(lay, x, k)
            assert np.array_equal(recv_host[i][rows], ref[rows]), (i, tab)
            assert np.all(recv_host[i][np.setdiff1d(np.arange(Rb), rows)] == 0xFFFF), (i, tab)


def test_every_tiny_routing_table():
    """Every routing table with 4 tokens, 4 experts, top-2 distinct (12^4 =
    20,736 tables; alignment 2, two destinations), bit-exact."""
    import itertools
    rows = list(itertools.permutations(range(4), 2))
    _layout_every_table(oracle.MODE_COMPACT, 4, 4, 2, 2, 2, 0, list(itertools.product(rows, repeat=4)))


def test_every_tiny_routing_table_single_launch():
    """Every 4-token, 4-expert top-2 distinct table (20,736), alignment 1,
    two destinations, through ep_dispatch_forward: its single launch builds
    alignment-1 layouts from per-token counts (rows = pairs with a smaller
    expert id + earlier pairs of the same expert); handle arrays, flags and
    receive rows. Then every 3-token, 3-expert top-2 table with repeated
    experts (9^3)."""
    import itertools
    rows = list(itertools.permutations(range(4), 2))
    _layout_every_table(oracle.MODE_COMPACT, 4, 4, 2, 1, 2, 0, list(itertools.product(rows, repeat=4)),
                        forward=True)
    rows = list(itertools.product(range(3), repeat=2))
    _layout_every_table(oracle.MODE_COMPACT, 3, 3, 2, 1, 1, 0, list(itertools.product(rows, repeat=3)),
                        forward=True)


def test_every_tiny_fixed_table():
    """FIXED capacity 1 and 2: every table of 3 tokens, 3 experts, top-2 with
    repeats allowed (9^3 tables), overflow flags included."""
    import itertools
    rows = list(itertools.product(range(3), repeat=2))
    for C in (1, 2):
        _layout_every_table(oracle.MODE_FIXED, 3, 3, 2, 1, 1, C, list(itertools.product(rows, repeat=3)))


def test_every_tiny_fixed_table_single_launch():
    """The same tables through ep_dispatch_forward, whose single launch
    builds FIXED layouts from per-token rank counts (no block builds the
    whole layout): handle arrays, flags and receive rows."""
    import itertools
    rows = list(itertools.product(range(3), repeat=2))
    for C in (1, 2):
        _layout_every_table(oracle.MODE_FIXED, 3, 3, 2, 1, 1, C, list(itertools.product(rows, repeat=3)),
                            forward=True)


@pytest.mark.parametrize("T,H,E,k,A,D,dispatch", [
    (64, 16384, 1024, 32, 2, 8, "fp8"),     # largest top-k and E; FP8 rows of exactly 1024 lanes x 16 values
    (40, 8200, 96, 32, 1, 4, "bf16"),       # 1025 vectors per row: every loop over a row wraps; 8200 % 128 != 0
    (33, 8, 40, 32, 3, 5, "bf16"),          # one vector per row, k = 32 of 40 experts
    (600, 8200, 64, 4, 8, 4, "bf16"),       # >= 512 tokens: combine rows in 9 pieces of 114 vectors, the last 113
    (520, 1032, 16, 2, 1, 1, "bf16"),       # >= 512 tokens, 129 vectors: combine pieces of 65 and 64
])
def test_largest_topk_and_ragged_rows(T, H, E, k, A, D, dispatch):
    _run_small(T, H, E, k, A=A, D=D, seed=T + H, dispatch=dispatch)
    _run_small(T, H, E, k, A=A, D=D, seed=T + H + 1, dispatch=dispatch, forward=True, masked=0.2, bad=0.05,
               distinct=False)


@pytest.mark.parametrize("seed", range(16))
def test_random_config_sweep(seed):
    """Seeded random configurations through the whole path against the
    oracle: batch size, hidden size (FP8 needs a multiple of 128), expert
    count, top-k (duplicates allowed in odd seeds), alignment, destination
    count, COMPACT or FIXED capacity, BF16 or FP8, two-call or one-call
    dispatch, masked and bad ids."""
    rng = np.random.default_rng(900 + seed)
    dispatch = "fp8" if rng.random() < 0.5 else "bf16"
    H = int(rng.choice([128, 256, 384, 640, 1024, 2048]) if dispatch == "fp8"
            else rng.choice([8, 72, 136, 256, 1000, 2056]))
    E = int(rng.choice([1, 4, 8, 32, 64, 256]))
    k = int(rng.integers(1, min(E, 9) + 1))
    D = int(rng.choice([d for d in (1, 2, 4, 8) if E % d == 0]))
    T = int(rng.integers(1, max(2, min(3000, 4_000_000 // H))))
    mode = int(rng.random() < 0.3)
    A = 1 if mode else int(rng.choice([1, 2, 16, 128]))
    C = int(rng.choice([16, 64, 256])) if mode else 0
    forward = bool(rng.random() < 0.5)
    masked = float(rng.choice([0.0, 0.05]))
    bad = float(rng.choice([0.0, 0.02]))
    _run_small(T, H, E, k, A=A, D=D, C=C, mode=mode, seed=seed, masked=masked, bad=bad,
               distinct=(seed % 2 == 0), dispatch=dispatch, forward=forward)


def test_widest_rows():
    """The largest hidden size the configuration accepts (2^24 channels:
    32 MiB BF16 rows, 16 MiB FP8 rows with 131,072 scales each) and a 2^20
    one: every loop over a row runs thousands of passes and every in-row
    byte offset exceeds 2^24; both dispatch kinds, two-call and one-call."""
    _run_small(3, 1 << 24, 2, 1, A=2, seed=91)
    _run_small(3, 1 << 24, 2, 1, A=2, seed=92, dispatch="fp8", forward=True)
    _run_small(5, 1 << 20, 4, 2, A=2, D=2, seed=93, dispatch="fp8")
    _run_small(5, 1 << 20, 4, 2, A=2, D=2, seed=94, forward=True, masked=0.2)


def test_largest_batch():
    """A million tokens at top-8 (8,388,608 pairs, 8,192 layout blocks: the
    count matrix of 8,192 x 256 takes the separate scan kernel) with narrow
    rows, FP8-free so the rows stay small: layout, dispatch and combine
    against the oracle."""
    _run_small(1 << 20, 8, 256, 8, A=128, D=8, seed=95, masked=0.01)


def test_hot_experts():
    """Degenerate routing at sizes that take the multi-block layout: every
    token to the same k experts (one expert's count is T, the others 0),
    to the last destination's experts, and half of the batch to one hot
    set; the single launch with every token on the same experts; FIXED
    capacity with every token on the same experts (all but C pairs of each
    dropped)."""
    T, E, k = 5000, 256, 8
    same = np.tile(np.arange(k), (T, 1))
    _run_small(T, 256, E, k, A=128, D=8, seed=81, table=same)
    _run_small(T, 256, E, k, A=128, D=8, seed=82, table=same[:, ::-1] + (E - k), dispatch="fp8")
    rng = np.random.default_rng(83)
    half = random_routing_table(rng, T, E, k)
    half[::2] = np.arange(100, 100 + k)
    _run_small(T, 256, E, k, A=128, D=8, seed=84, table=half, dispatch="fp8")
    _run_small(300, 512, E, k, A=1, seed=85, table=same[:300], forward=True, dispatch="fp8")
    _run_small(T, 256, E, k, mode=oracle.MODE_FIXED, C=128, seed=86, table=same)


def test_masked_and_bad_ids():
    h, lay = _run_small(500, 128, 12, 4, A=3, D=4, seed=3, masked=0.2, bad=0.05, distinct=False)
    assert lay["flags"] == oracle.FLAG_BAD_ID and h.check() == oracle.FLAG_BAD_ID
    h, lay = _run_small(6000, 64, 40, 3, A=16, D=2, seed=4, masked=0.1, bad=0.01, distinct=False)
    assert h.check() == oracle.FLAG_BAD_ID


def test_int32_indices_and_fp8():
    _run_small(700, 256, 32, 4, A=32, D=4, seed=5, idx_bits=32, dispatch="fp8")
    _run_small(3000, 384, 96, 6, A=64, D=8, seed=6, idx_bits=32, dispatch="fp8")


def test_fixed_capacity_and_overflow():
    h, lay = _run_small(128, 256, 16, 4, mode=1, C=64, seed=7, dispatch="fp8")
    assert h.check() == 0
    h, lay = _run_small(200, 128, 8, 3, mode=1, C=20, seed=8)       # overflow
    assert lay["flags"] == oracle.FLAG_OVERFLOW and h.check() == oracle.FLAG_OVERFLOW
    h, lay = _run_small(3000, 128, 8, 3, mode=1, C=500, seed=9)     # multi-block, overflow
    assert h.check() == oracle.FLAG_OVERFLOW
    h, lay = _run_small(12000, 64, 1024, 4, mode=1, C=40, seed=16)  # 3-kernel layout, overflow
    assert lay["flags"] == oracle.FLAG_OVERFLOW and h.check() == oracle.FLAG_OVERFLOW
    h, lay = _run_small(9000, 64, 1000, 5, A=4, D=8, seed=17, masked=0.1, bad=0.01, distinct=False)
    assert h.check() == oracle.FLAG_BAD_ID                             # 3-kernel layout, bad ids


def test_no_zero_pad_flag():
    _run_small(333, 128, 16, 3, A=16, D=2, seed=10, flags=ops.FLAG_NO_ZERO_PAD)
    _run_small(333, 256, 16, 3, A=16, D=2, seed=11, flags=ops.FLAG_NO_ZERO_PAD, dispatch="fp8")


def test_unweighted_and_k1():
    _run_small(99, 64, 5, 1, A=4, seed=12)
    _run_small(99, 64, 5, 3, A=4, seed=13, weights=False)


def test_empty_batch():
    cfg = ops.Config(max_tokens=16, hidden=128, num_experts=8, num_topk=2, expert_alignment=4)
    idx = torch.zeros((0, 2), dtype=torch.int64, device="cuda")
    h = ops.layout(cfg, idx)
    cnt, pad, R = h.read_counts()
    assert R == 0 and cnt.sum() == 0 and h.check() == 0
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    ops.dispatch(h, x)
    y = torch.zeros((cfg.recv_rows_bound(), 128), dtype=torch.bfloat16, device="cuda")
    out = ops.combine(h, y)
    assert out.shape == (0, 128)
    torch.cuda.synchronize()


def test_argument_errors_enqueue_nothing():
    cfg = ops.Config(max_tokens=4, hidden=100, num_experts=8, num_topk=2)
    with pytest.raises(Exception):
        ops.new_workspace(cfg)
    cfg = ops.Config(max_tokens=4, hidden=128, num_experts=8, num_topk=2)
    idx = torch.zeros((5, 2), dtype=torch.int64, device="cuda")
    with pytest.raises(Exception):
        ops.layout(cfg, idx)                                # T > max_tokens
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(Exception):
        ops.layout(cfg, idx[:4], workspace=ws)              # workspace too small


# ---------------------------------------------------------------- one-call dispatch_forward

@pytest.mark.parametrize("T,E,k,A,D,C,mode,dispatch,masked,bad", [
    (128, 16, 2, 1, 1, 0, 0, "bf16", 0.0, 0.0),          # tiny shape, single launch
    (300, 40, 4, 1, 4, 0, 0, "bf16", 0.1, 0.02),         # alignment 1, P = 1200 (four groups per wave), masked/bad ids
    (512, 512, 8, 1, 8, 0, 0, "fp8", 0.05, 0.01),        # alignment 1, P = 4096, E = 512, repeated experts
    (128, 256, 8, 1, 1, 128, 1, "fp8", 0.0, 0.0),        # decode shape (FIXED), single launch
    (100, 64, 8, 16, 4, 0, 0, "fp8", 0.0, 0.0),          # padding rows cleared by the same launch
    (128, 64, 8, 1, 1, 12, 1, "bf16", 0.0, 0.0),         # FIXED overflow
    (200, 64, 6, 1, 4, 20, 1, "fp8", 0.1, 0.02),         # FIXED, P = 1200 (four groups per wave), D = 4, masked/bad ids
    (512, 512, 8, 1, 8, 16, 1, "bf16", 0.1, 0.02),       # FIXED, P = 4096, E = 512, overflow, repeated experts
    (1, 4, 3, 1, 2, 1, 1, "bf16", 0.0, 0.0),             # FIXED, one token
    (129, 64, 8, 32, 2, 0, 0, "bf16", 0.0, 0.0),         # P = 1032: four groups per wave
    (512, 512, 8, 8, 8, 0, 0, "fp8", 0.1, 0.02),         # P = 4096, E = 512: largest single launch
    (513, 512, 8, 8, 8, 0, 0, "bf16", 0.0, 0.0),         # P = 4104: layout + dispatch launches
    (300, 513, 2, 4, 3, 0, 0, "bf16", 0.0, 0.0),         # E = 513: layout + dispatch launches
    (1, 16, 4, 4, 2, 0, 0, "fp8", 0.0, 0.0),             # one token
    (16, 256, 8, 128, 8, 0, 0, "fp8", 0.0, 0.0),         # 2,048 zero-fill pieces: layout + dispatch launches
    (40, 64, 6, 128, 4, 0, 0, "bf16", 0.0, 0.0),         # 512 zero-fill pieces + 40 tokens: two launches
])
def test_dispatch_forward(T, E, k, A, D, C, mode, dispatch, masked, bad):
    H = 7168 if (T, E) == (128, 256) else 256
    h, lay = _run_small(T, H, E, k, A=A, D=D, C=C, mode=mode, seed=T * 7 + E, masked=masked, bad=bad,
                        distinct=masked == 0.0, dispatch=dispatch, forward=True)
    assert h.check() == lay["flags"]


def test_dispatch_forward_prequant_and_empty():
    rng = np.random.default_rng(21)
    T, H, E, k, A = 200, 256, 32, 4, 8
    idx = random_routing_table(rng, T, E, k)
    lay = oracle.layout(0, T, E, k, A, 1, 0, idx)
    xq = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    xs = rng.standard_normal((T, H // 128)).astype(np.float32)
    q, s = oracle.dispatch_fp8_prequant(lay, xq, xs, k)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A)
    h, gq, gs = ops.dispatch_forward(cfg, to_dev(idx), to_dev(xq), ops.FP8_PREQUANT, x_scales=to_dev(xs))
    compare_layout(h, lay, weights=False)
    rows = np.arange(lay["rows"])
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))
    # empty batch: zero counts, nothing copied
    cfg = ops.Config(max_tokens=16, hidden=128, num_experts=8, num_topk=2, expert_alignment=4)
    idx = torch.zeros((0, 2), dtype=torch.int64, device="cuda")
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    h, recv = ops.dispatch_forward(cfg, idx, x)
    cnt, pad, R = h.read_counts()
    assert R == 0 and cnt.sum() == 0 and h.check() == 0


def test_dispatch_forward_graph_replay():
    """The decode step (one-call layout + dispatch, then combine) captured in
    a HIP graph: every replay, with new routing copied in between, matches
    the eager calls."""
    wl = WORKLOADS["decode"]
    cfg = cfg_of(wl)
    R = cfg.recv_rows_bound()
    rng = np.random.default_rng(22)
    idx_s = torch.zeros((wl.T, wl.k), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((wl.T, wl.k), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    y = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((R, wl.H)).astype(np.float32)))
    ws = ops.new_workspace(cfg)
    recv = torch.empty((R, wl.H), dtype=torch.uint8, device="cuda")
    rs = torch.empty((R, wl.H // 128), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    def step():
        h = ops.dispatch_forward(cfg, idx_s, x_s, ops.FP8_QUANTIZE, topk_w=w_s, workspace=ws, recv=recv,
                                 recv_scales=rs)[0]
        ops.combine(h, y, w_s, out=out)
        return h

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = step()
    for rep in range(3):
        idx = np.stack([rng.permutation(wl.E)[:wl.k] for _ in range(wl.T)]).astype(np.int64)
        w = rng.random((wl.T, wl.k)).astype(np.float32)
        x = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H)).astype(np.float32))
        idx_s.copy_(to_dev(idx))
        w_s.copy_(to_dev(w))
        x_s.copy_(to_dev_bf16(x))
        g.replay()
        torch.cuda.synchronize()
        got = (host(h.slot).copy(), host(recv).copy(), host(rs).copy(), bf16_host(out).copy())
        step()                                     # eager, same inputs
        torch.cuda.synchronize()
        ref = (host(h.slot), host(recv), host(rs), bf16_host(out))
        lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, idx, w)
        assert np.array_equal(got[0], lay["slot"]), rep
        rows = written_rows(lay)
        assert np.array_equal(got[1][rows], ref[1][rows]), rep
        assert np.array_equal(got[2][rows].view(np.uint32), ref[2][rows].view(np.uint32)), rep
        assert np.array_equal(got[3], ref[3]), rep


def test_bound_calls_match_eager():
    """Bound dispatch_forward + combine (arguments converted once) on fixed
    buffers: three steps with new routing, weights and x copied in between,
    each equal to the eager calls and the oracle's slots."""
    wl = WORKLOADS["decode"]
    cfg = cfg_of(wl)
    R = cfg.recv_rows_bound()
    rng = np.random.default_rng(23)
    idx_s = torch.zeros((wl.T, wl.k), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((wl.T, wl.k), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    y = to_dev_bf16(f32_to_bf16_bits(rng.standard_normal((R, wl.H)).astype(np.float32)))
    recv = torch.empty((R, wl.H), dtype=torch.uint8, device="cuda")
    rs = torch.empty((R, wl.H // 128), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    fwd, h = ops.bind_dispatch_forward(cfg, idx_s, x_s, ops.FP8_QUANTIZE, recv, rs, topk_w=w_s)
    comb = ops.bind_combine(h, y, out, topk_w=w_s)
    for rep in range(3):
        idx = np.stack([rng.permutation(wl.E)[:wl.k] for _ in range(wl.T)]).astype(np.int64)
        w = rng.random((wl.T, wl.k)).astype(np.float32)
        x = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H)).astype(np.float32))
        idx_s.copy_(to_dev(idx))
        w_s.copy_(to_dev(w))
        x_s.copy_(to_dev_bf16(x))
        fwd()
        comb()
        torch.cuda.synchronize()
        got = (host(h.slot).copy(), host(recv).copy(), host(rs).copy(), bf16_host(out).copy())
        he, re_, se = ops.dispatch_forward(cfg, idx_s, x_s, ops.FP8_QUANTIZE, topk_w=w_s)
        oe = ops.combine(he, y, w_s)
        lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, idx, w)
        rows = written_rows(lay)
        assert np.array_equal(got[0], lay["slot"]), rep
        assert np.array_equal(got[1][rows], host(re_)[rows]), rep
        assert np.array_equal(got[2][rows].view(np.uint32), host(se)[rows].view(np.uint32)), rep
        assert np.array_equal(got[3], bf16_host(oe)), rep


# ---------------------------------------------------------------- duals

def test_backward_duals():
    rng = np.random.default_rng(14)
    T, H, E, k, A = 400, 256, 16, 4, 8
    idx = random_routing_table(rng, T, E, k, masked_frac=0.05)
    w = rng.random((T, k)).astype(np.float32)
    lay = oracle.layout(0, T, E, k, A, 1, 0, idx, w)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A)
    h = ops.layout(cfg, to_dev(idx), to_dev(w))
    R = cfg.recv_rows_bound()
    # dispatch_backward = unweighted combine + gather of row grads
    g = f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    grow = rng.standard_normal(R).astype(np.float32)
    ref_x, ref_w = oracle.dispatch_backward(lay, g, k, grow)
    gx, gw = ops.dispatch_backward(h, to_dev_bf16(g), to_dev(grow))
    assert np.array_equal(bf16_host(gx), ref_x)
    assert np.array_equal(host(gw).view(np.uint32), ref_w.view(np.uint32))
    # combine_backward = dispatch of grad_out, weighted per pair (BF16)
    go = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ref = oracle.combine_backward_bf16(lay, go, k, w)
    gy = ops.combine_backward(h, to_dev_bf16(go), ops.BF16, to_dev(w))
    rows = np.arange(lay["rows"])
    assert np.array_equal(bf16_host(gy)[rows], ref[rows])
    # unweighted and FP8 combine_backward
    ref = oracle.combine_backward_bf16(lay, go, k, None)
    gy = ops.combine_backward(h, to_dev_bf16(go), ops.BF16)
    assert np.array_equal(bf16_host(gy)[rows], ref[rows])
    q, s = oracle.dispatch_fp8(lay, go, k)
    gq, gs = ops.combine_backward(h, to_dev_bf16(go), ops.FP8_QUANTIZE)
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))
    # weighted FP8: each pair's bf16(w * g) quantised with its own scales
    q, s = oracle.combine_backward_fp8(lay, go, k, w)
    gq, gs = ops.combine_backward(h, to_dev_bf16(go), ops.FP8_QUANTIZE, to_dev(w))
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))
    with pytest.raises(Exception):
        ops.combine_backward(h, to_dev(np.zeros((T, H), np.uint8)), ops.FP8_PREQUANT, to_dev(w))
    # an FP8 (codes, scales) gradient, unweighted: every code byte (NaN
    # patterns included) and scale lands in its pairs' rows bitwise
    gq8 = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    gs8 = rng.standard_normal((T, H // 128)).astype(np.float32)
    q, s = oracle.dispatch_fp8_prequant(lay, gq8, gs8, k)
    gq, gs = ops.combine_backward(h, to_dev(gq8), ops.FP8_PREQUANT, grad_out_scales=to_dev(gs8))
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))
    with pytest.raises(Exception):
        ops.combine_backward(h, to_dev(gq8), ops.FP8_PREQUANT)          # scales missing


def _weight_grad_bound(H, g, y, slot):
    """Error bound of the GPU sum: each product passes through at most
    d = 8 * ceil(vectors / threads) + 6 + (waves - 1) binary32 additions
    (lane, wave butterfly, waves in order), so |got - exact| <=
    gamma_d * sum |g * y| with gamma_d = d u / (1 - d u), u = 2^-24."""
    nvec = H // 8
    threads = min(1024, -(-nvec // 64) * 64)
    d = 8 * -(-nvec // threads) + 6 + (threads // 64 - 1)
    u = 2.0 ** -24
    T, k = slot.shape
    mag = np.empty((T, k))
    ga = np.abs(g)
    for j in range(k):
        mag[:, j] = (ga * np.abs(y[np.maximum(slot[:, j], 0)])).sum(-1)
    return d * u / (1 - d * u) * mag


def _check_weight_grad(h, lay, g_bits, y_bits, k):
    ref = oracle.combine_weight_grad(lay, g_bits, y_bits, k)
    got = ops.combine_weight_grad(h, to_dev_bf16(g_bits), to_dev_bf16(y_bits))
    got2 = ops.combine_weight_grad(h, to_dev_bf16(g_bits), to_dev_bf16(y_bits))
    got, got2 = host(got).astype(np.float64), host(got2)
    assert np.array_equal(got.astype(np.float32).view(np.uint32), got2.view(np.uint32))   # deterministic
    T, H = g_bits.shape
    slot = lay["slot"].reshape(T, k)
    bound = _weight_grad_bound(H, bf16_bits_to_f32(g_bits).astype(np.float64), bf16_bits_to_f32(y_bits), slot)
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(got[slot < 0] == 0.0)
    return err, bound


@pytest.mark.parametrize("T,H,E,k,A,masked", [
    (1, 8, 4, 1, 1, 0.0), (77, 264, 12, 3, 4, 0.2), (300, 2048, 32, 8, 16, 0.05),
    (64, 16384, 16, 6, 1, 0.0),      # two vectors per lane
    (40, 1024, 8, 12, 2, 0.1),       # k > 8: two groups of pairs
    (24, 8200, 48, 32, 1, 0.1),      # largest top-k (four groups), 1025 vectors: the row loop wraps
])
def test_combine_weight_grad(T, H, E, k, A, masked):
    log("weight grad T=%d H=%d E=%d k=%d" % (T, H, E, k))
    rng = np.random.default_rng(T + H)
    idx = random_routing_table(rng, T, E, k, masked_frac=masked, distinct=masked == 0.0)
    lay = oracle.layout(0, T, E, k, A, 1, 0, idx)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A)
    h = ops.layout(cfg, to_dev(idx))
    R = cfg.recv_rows_bound()
    g = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    y = f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    _check_weight_grad(h, lay, g, y, k)


def test_combine_weight_grad_v3_full_size():
    """The 8192 x 7168 x top-8 shape: every pair within the bound."""
    case = workload_case("v3")
    wl, inp, lay = case["wl"], case["inp"], case["lay"]
    h = ops.layout(cfg_of(wl), to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
    rng = np.random.default_rng(41)
    g = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H)).astype(np.float32))
    err, bound = _check_weight_grad(h, lay, g, inp["y"], wl.k)
    log("v3 weight grad: max err/bound %.3g" % float((err / bound).max()))


def test_combine_backward_fp8_weighted_v3_shape():
    """Weighted FP8 combine_backward on 1024 tokens of the 7168 x top-8,
    256-expert shape (8 pairs per token, each with its own scales)."""
    wl = WORKLOADS["v3"].with_tokens(1024)
    inp = make_inputs(wl, with_y=False)
    lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, inp["topk_idx"], inp["topk_w"])
    h = ops.layout(cfg_of(wl), to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
    rng = np.random.default_rng(43)
    go = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H)).astype(np.float32))
    q, s = oracle.combine_backward_fp8(lay, go, wl.k, inp["topk_w"])
    gq, gs = ops.combine_backward(h, to_dev_bf16(go), ops.FP8_QUANTIZE, to_dev(inp["topk_w"]))
    rows = np.arange(lay["rows"])
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))


def test_combine_backward_fp8_weighted_all_patterns():
    """Weighted FP8 combine_backward on every finite bf16 pattern (sorted by
    magnitude, 128 to a block) under weights that reach the edges: signed
    zeros, +-1, products that become binary32 subnormals or zero, and a
    subnormal weight; every token sends to all 8 experts, each pair with its
    own weight, bit-exact against the oracle."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = bits[np.isfinite((bits << 16).view(np.float32))].astype(np.uint16)
    mag = np.abs((vals.astype(np.uint32) << 16).view(np.float32))
    vals = vals[np.argsort(mag, kind="stable")]
    H, k, E = 1024, 8, 8
    T = -(-vals.size // H)
    x = np.zeros(T * H, np.uint16)
    x[:vals.size] = vals
    x = x.reshape(T, H)
    special = np.array([0.0, -0.0, 1.0, -1.0, 0.3, -0.70710678, 2.0 ** -100, -3.0 * 2.0 ** -130], np.float32)
    w = np.stack([np.roll(special, t) for t in range(T)]).astype(np.float32)
    idx = np.stack([np.roll(np.arange(E), t) for t in range(T)]).astype(np.int64)
    log("weighted fp8 backward, all bf16 patterns: T=%d H=%d k=%d" % (T, H, k))
    lay = oracle.layout(0, T, E, k, 1, 1, 0, idx, w)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k)
    h = ops.layout(cfg, to_dev(idx), to_dev(w))
    q, sc = oracle.combine_backward_fp8(lay, x, k, w)
    gq, gs = ops.combine_backward(h, to_dev_bf16(x), ops.FP8_QUANTIZE, to_dev(w))
    rows = np.arange(lay["rows"])
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), sc[rows].view(np.uint32))


def test_fp8_prequant_passthrough():
    rng = np.random.default_rng(15)
    T, H, E, k, A = 300, 512, 16, 4, 16
    idx = random_routing_table(rng, T, E, k)
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = oracle.layout(0, T, E, k, A, 1, 0, idx)
    xq = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    xs = rng.standard_normal((T, H // 128)).astype(np.float32)
    q, s = oracle.dispatch_fp8_prequant(lay, xq, xs, k)
    cfg = ops.Config(max_tokens=T, hidden=H, num_experts=E, num_topk=k, expert_alignment=A)
    h = ops.layout(cfg, to_dev(idx))
    gq, gs = ops.dispatch(h, to_dev(xq), ops.FP8_PREQUANT, x_scales=to_dev(xs))
    rows = np.arange(lay["rows"])
    assert np.array_equal(host(gq)[rows], q[rows])
    assert np.array_equal(host(gs)[rows].view(np.uint32), s[rows].view(np.uint32))


def test_identity_round_trip_gpu():
    """dispatch -> identity experts -> combine with softmax weights == x."""
    wl = WORKLOADS["mid"]
    inp = make_inputs(wl, with_y=False)
    cfg = cfg_of(wl)
    h = ops.layout(cfg, to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
    recv = ops.dispatch(h, to_dev_bf16(inp["x"]))
    out = ops.combine(h, recv, to_dev(inp["topk_w"]))
    ref = np.where(inp["x"] == 0x8000, 0, inp["x"])
    assert np.array_equal(bf16_host(out), ref)


# ---------------------------------------------------------------- FP8 codec

def test_fp8_codec_all_bf16_patterns():
    """Every finite bf16 pattern is quantised on the GPU under a grid of block
    scales, bit-exact against the oracle. Values are sorted by magnitude
    and packed 127 per 128-block with one element setting the block's amax
    to (largest value in the block) * factor."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    vals = bits[np.isfinite(v)].astype(np.uint16)
    mag = np.abs((vals.astype(np.uint32) << 16).view(np.float32))
    vals = vals[np.argsort(mag, kind="stable")]
    nblk = -(-vals.size // 127)
    padded = np.zeros(nblk * 127, np.uint16)
    padded[:vals.size] = vals
    blocks = padded.reshape(nblk, 127)
    bm = np.abs((blocks.astype(np.uint32) << 16).view(np.float32)).max(axis=1)
    for factor in (1.0, 1.5, 3.0, 2.0 ** 9, 2.0 ** 20):
        top = float(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])   # largest finite bf16
        amax = f32_to_bf16_bits(np.minimum(np.maximum(bm.astype(np.float64), 2.0 ** -100) * factor, top)
                                .astype(np.float32))
        x = np.concatenate([amax[:, None], blocks], axis=1)            # [nblk, 128]
        T = nblk
        H = 128
        idx = np.zeros((T, 1), np.int64)
        lay = oracle.layout(0, T, 1, 1, 1, 1, 0, idx)
        q, s = oracle.dispatch_fp8(lay, x, 1)
        cfg = ops.Config(max_tokens=T, hidden=H, num_experts=1, num_topk=1)
        h = ops.layout(cfg, to_dev(idx))
        gq, gs = ops.dispatch(h, to_dev_bf16(x), ops.FP8_QUANTIZE)
        assert np.array_equal(host(gq)[:T], q[:T]), factor
        assert np.array_equal(host(gs)[:T].view(np.uint32), s[:T].view(np.uint32)), factor


def test_fp8_quantiser_every_pair():
    """Every pair of finite bf16 magnitudes |x| <= amax through the GPU FP8
    dispatch, bit-exact against the oracle: for each non-negative finite
    bf16 value a (the block's amax, element 0), blocks of 127 further
    elements hold every bf16 magnitude <= a, signs alternating so each value
    meets both signs. 4.2M blocks of 128 in five launches."""
    vals = np.arange(0x7F80, dtype=np.uint16)          # +0 .. largest finite, increasing
    n = vals.size
    nb = (np.arange(n) + 127) // 127                    # blocks needed for amax index i: ceil((i+1)/127)
    nb[0] = 0                                           # amax 0: all-zero blocks are tested elsewhere
    bounds = np.searchsorted(np.cumsum(nb), np.linspace(0, nb.sum(), 6)[1:-1])
    edges = [1] + [int(b) for b in bounds] + [n]
    for c in range(len(edges) - 1):
        i0, i1 = edges[c], edges[c + 1]
        cnt = nb[i0:i1]
        amax_idx = np.repeat(np.arange(i0, i1, dtype=np.int32), cnt)
        first = np.repeat(np.cumsum(cnt) - cnt, cnt)
        off = (np.arange(amax_idx.size) - first).astype(np.int32)
        idx = off[:, None] * 127 + np.arange(127, dtype=np.int32)[None, :]
        valid = idx <= amax_idx[:, None]
        xs = np.where(valid, vals[np.minimum(idx, n - 1)], 0).astype(np.uint16)
        xs |= (((idx + amax_idx[:, None]) & 1).astype(np.uint16) << 15) & np.where(valid, 0x8000, 0).astype(np.uint16)
        del idx, valid
        x = np.concatenate([vals[amax_idx][:, None], xs], axis=1)
        del xs
        T = x.shape[0]
        log("fp8 every pair: chunk %d, amax index %d..%d, %d blocks" % (c, i0, i1, T))
        topk = np.zeros((T, 1), np.int64)
        lay = oracle.layout(0, T, 1, 1, 1, 1, 0, topk)
        q, sc = oracle.dispatch_fp8(lay, x, 1)
        cfg = ops.Config(max_tokens=T, hidden=128, num_experts=1, num_topk=1)
        h = ops.layout(cfg, to_dev(topk))
        gq, gs = ops.dispatch(h, to_dev_bf16(x), ops.FP8_QUANTIZE)
        assert np.array_equal(host(gq), q), c
        assert np.array_equal(host(gs).view(np.uint32), sc.view(np.uint32)), c
        del q, sc, gq, gs, x
        torch.cuda.empty_cache()


# ---------------------------------------------------------------- determinism

def test_repeat_is_bit_identical():
    wl = WORKLOADS["skewed_v3"].with_tokens(2048)
    inp = make_inputs(wl, with_y=False)
    cfg = cfg_of(wl)
    outs = []
    for _ in range(2):
        h = ops.layout(cfg, to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
        q, s = ops.dispatch(h, to_dev_bf16(inp["x"]), ops.FP8_QUANTIZE)
        torch.cuda.synchronize()
        outs.append((host(h.slot).copy(), host(q).copy(), host(s).copy()))
    R = int(host(h.expert_off)[-1])
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1][:R], outs[1][1][:R])
    assert np.array_equal(outs[0][2][:R], outs[1][2][:R])


# ---------------------------------------------------------------- full workloads

@pytest.mark.parametrize("name", ["tiny", "mid", "decode", "v3", "skewed_v3", "skewed_v3_s06"])
def test_workload_full_size(name):
    """Every workload at its full size: layout, dispatch and combine through
    ep_layout + ep_dispatch, then the calls bench.py times for it (one
    ep_dispatch_forward, the weighted combine and, for the aligned layouts,
    the weighted BF16 combine_backward and dispatch_backward with the
    weight-gradient gather), each against the oracle."""
    log("workload %s: preparing inputs and oracle" % name)
    case = workload_case(name)
    wl, inp, lay = case["wl"], case["inp"], case["lay"]
    log("workload %s: GPU run" % name)
    cfg = cfg_of(wl)
    h = ops.layout(cfg, to_dev(inp["topk_idx"]), to_dev(inp["topk_w"]))
    compare_layout(h, lay)
    rows = written_rows(lay)
    x = to_dev_bf16(inp["x"])
    if wl.dispatch == "fp8":
        R = cfg.recv_rows_bound()
        recv = torch.full((R, wl.H), 0xEE, dtype=torch.uint8, device="cuda")
        rs = torch.full((R, wl.H // 128), -7.0, dtype=torch.float32, device="cuda")
        ops.dispatch(h, x, ops.FP8_QUANTIZE, recv=recv, recv_scales=rs)
        assert np.array_equal(host(recv)[rows], case["recv"][rows])
        assert np.array_equal(host(rs)[rows].view(np.uint32), case["recv_scales"][rows].view(np.uint32))
        if wl.mode == oracle.MODE_FIXED:
            untouched = np.setdiff1d(np.arange(R), rows)
            assert np.all(host(recv)[untouched] == 0xEE)
        del recv, rs
    else:
        recv = ops.dispatch(h, x)
        assert np.array_equal(bf16_host(recv)[rows], case["recv"][rows])
        del recv
    y = to_dev_bf16(inp["y"])
    out, vals = ops.combine(h, y, to_dev(inp["topk_w"]), row_vals=h.row_w)
    got = bf16_host(out)
    d = bf16_ulp_distance(got, case["out"])
    log("workload %s: combine max ulp %d, differing %d" % (name, d.max(), int((d > 0).sum())))
    assert d.max() <= 1
    assert np.array_equal(host(vals).view(np.uint32), case["out_vals"].view(np.uint32))
    del out, vals, h
    torch.cuda.empty_cache()

    log("workload %s: bench calls (dispatch_forward, combine, backward duals)" % name)
    R = cfg.recv_rows_bound()
    w = to_dev(inp["topk_w"])
    if wl.dispatch == "fp8":
        recv = torch.full((R, wl.H), 0xEE, dtype=torch.uint8, device="cuda")
        rs = torch.full((R, wl.H // 128), -7.0, dtype=torch.float32, device="cuda")
        h = ops.dispatch_forward(cfg, to_dev(inp["topk_idx"]), x, ops.FP8_QUANTIZE, topk_w=w, recv=recv,
                                 recv_scales=rs)[0]
        compare_layout(h, lay)
        assert np.array_equal(host(recv)[rows], case["recv"][rows])
        assert np.array_equal(host(rs)[rows].view(np.uint32), case["recv_scales"][rows].view(np.uint32))
        untouched = np.setdiff1d(np.arange(R), rows)
        assert np.all(host(recv)[untouched] == 0xEE)
        del recv, rs
    else:
        recv = torch.full((R, wl.H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        h = ops.dispatch_forward(cfg, to_dev(inp["topk_idx"]), x, ops.BF16, topk_w=w, recv=recv)[0]
        compare_layout(h, lay)
        got_recv = bf16_host(recv)
        assert np.array_equal(got_recv[rows], case["recv"][rows])
        assert np.all(got_recv[np.setdiff1d(np.arange(R), rows)] == 0xFFFF)
        del recv, got_recv
    out = ops.combine(h, y, w)
    assert bf16_ulp_distance(bf16_host(out), case["out"]).max() <= 1
    del out
    if wl.mode == oracle.MODE_COMPACT:
        rng = np.random.default_rng(5)
        go = f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H)).astype(np.float32))
        grw = rng.standard_normal(R).astype(np.float32)
        ref = oracle.combine_backward_bf16(lay, go, wl.k, inp["topk_w"])
        gy = ops.combine_backward(h, to_dev_bf16(go), ops.BF16, w)
        prow = np.arange(lay["rows"])
        assert np.array_equal(bf16_host(gy)[prow], ref[prow]), "combine_backward"
        del gy, ref
        # the expert-output rows serve as the receive-row gradients
        ref_x, ref_w = oracle.dispatch_backward(lay, inp["y"], wl.k, grw)
        gx, gw = ops.dispatch_backward(h, y, to_dev(grw))
        assert np.array_equal(bf16_host(gx), ref_x), "dispatch_backward"
        assert np.array_equal(host(gw).view(np.uint32), ref_w.view(np.uint32))
        del gx, gw
    del y, x, h
    torch.cuda.empty_cache()
