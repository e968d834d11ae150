"""Pins for the oracle's layout (counts, alignment, offsets, stable slots).

Each check holds independently of the oracle's code: hand-worked fixtures,
numpy library special cases (bincount, stable argsort), an O(P^2) brute-force
definition of the stable rank, and exhaustive enumeration of tiny routing
tables."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from ep_workloads import WORKLOADS, make_inputs, random_routing_table, draw_routing, _streams

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_layout(mode, T, E, k, A, D, C, idx):
    """Layout from the definition, with no shared code: rank of a pair among
    earlier pairs with the same expert, counted pair by pair."""
    idx = [int(v) for v in np.asarray(idx).ravel()]
    P = T * k
    valid = [0 <= v < E for v in idx]
    cnt = [sum(1 for p in range(P) if valid[p] and idx[p] == e) for e in range(E)]
    if mode == oracle.MODE_COMPACT:
        pad = [-(-c // A) * A for c in cnt]
        off = [sum(pad[:e]) for e in range(E + 1)]
    else:
        pad = [min(c, C) for c in cnt]
        off = [e * C for e in range(E + 1)]
    slot = []
    for p in range(P):
        if not valid[p]:
            slot.append(-1)
            continue
        rank = sum(1 for q in range(p) if valid[q] and idx[q] == idx[p])
        if mode == oracle.MODE_FIXED and rank >= C:
            slot.append(-1)
        else:
            slot.append(off[idx[p]] + rank)
    epd = E // D
    dest_tokens = [sum(1 for t in range(T)
                       if any(valid[t * k + j] and idx[t * k + j] // epd == d for j in range(k)))
                   for d in range(D)]
    flags = 0
    if any(not valid[p] and idx[p] != -1 for p in range(P)):
        flags |= oracle.FLAG_BAD_ID
    if mode == oracle.MODE_FIXED and any(c > C for c in cnt):
        flags |= oracle.FLAG_OVERFLOW
    return dict(cnt=cnt, pad=pad, expert_off=off, slot=slot,
                dest_off=[off[d * epd] for d in range(D + 1)], dest_tokens=dest_tokens, flags=flags)


def check_against_brute(mode, T, E, k, A, D, C, idx, w=None):
    lay = oracle.layout(mode, T, E, k, A, D, C, idx, w)
    bf = brute_force_layout(mode, T, E, k, A, D, C, idx)
    for key in ("cnt", "pad", "expert_off", "slot", "dest_off", "dest_tokens"):
        assert list(lay[key]) == list(bf[key]), key
    assert lay["flags"] == bf["flags"]
    # row_src / row_w are the inverse of slot
    for p, s in enumerate(bf["slot"]):
        if s >= 0:
            assert lay["row_src"][s] == p
            if w is not None:
                assert lay["row_w"][s] == np.asarray(w, np.float32).ravel()[p]
    if mode == oracle.MODE_COMPACT:
        for e in range(E):
            for r in range(bf["expert_off"][e] + bf["cnt"][e], bf["expert_off"][e + 1]):
                assert lay["row_src"][r] == -1
                if w is not None:
                    assert lay["row_w"][r] == 0.0
    return lay


def test_golden_hand_worked_layouts():
    with open(os.path.join(GOLDEN, "layout_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        idx = np.array(c["topk_idx"], np.int64)
        w = np.array(c["topk_w"], np.float32)
        lay = oracle.layout(c["mode"], c["T"], c["E"], c["k"], c["A"], c["D"], c["C"], idx, w)
        for key in ("cnt", "pad", "expert_off", "dest_off", "dest_tokens", "slot"):
            assert list(lay[key]) == c[key], (c["name"], key)
        assert lay["rows"] == c["rows"] and lay["flags"] == c["flags"], c["name"]
        for r, (src, wr) in enumerate(zip(c["row_src"], c["row_w"])):
            if src is None:
                continue
            assert lay["row_src"][r] == src, (c["name"], r)
            assert lay["row_w"][r] == np.float32(wr), (c["name"], r)


def test_exhaustive_tiny_tables():
    """Every routing table with T=3 tokens, E=4 experts, top-2 distinct
    (12^3 tables), plus all tables at T=4 for one alignment: the oracle
    equals the brute-force definition."""
    rows = [r for r in itertools.permutations(range(4), 2)]
    for A, D in ((1, 1), (2, 2), (3, 4)):
        for tab in itertools.product(rows, repeat=3):
            idx = np.array(tab, np.int64)
            check_against_brute(oracle.MODE_COMPACT, 3, 4, 2, A, D, 0, idx)
    for tab in itertools.product(rows, repeat=4):
        idx = np.array(tab, np.int64)
        check_against_brute(oracle.MODE_COMPACT, 4, 4, 2, 2, 2, 0, idx)


def test_exhaustive_tiny_fixed():
    rows = [r for r in itertools.product(range(3), repeat=2)]  # repeats allowed
    for C in (1, 2):
        for tab in itertools.product(rows, repeat=3):
            idx = np.array(tab, np.int64)
            check_against_brute(oracle.MODE_FIXED, 3, 3, 2, 1, 1, C, idx)


@pytest.mark.parametrize("seed", range(6))
def test_random_small_with_masks_and_bad_ids(seed):
    rng = np.random.default_rng(100 + seed)
    T, E, k = 37, 8, 3
    idx = random_routing_table(rng, T, E, k, masked_frac=0.1, bad_frac=0.05, distinct=(seed % 2 == 0))
    w = rng.random((T, k)).astype(np.float32)
    for mode, A, D, C in ((0, 1, 1, 0), (0, 4, 2, 0), (0, 5, 8, 0), (1, 1, 4, 3), (1, 1, 1, 40)):
        lay = check_against_brute(mode, T, E, k, A, D, C, idx, w)
        lay32 = oracle.layout(mode, T, E, k, A, D, C, idx.astype(np.int32), w)
        for key in ("cnt", "pad", "expert_off", "slot", "dest_tokens", "dest_off"):
            assert np.array_equal(lay[key], lay32[key])
        assert lay["flags"] == lay32["flags"]


@pytest.mark.parametrize("name", ["tiny", "mid", "v3", "skewed_v3", "skewed_v3_s06", "decode"])
def test_workload_invariants(name):
    """P1-P3 at the workloads' real shapes: counts are numpy's bincount,
    slots equal the stable argsort of the expert ids mapped through the
    offsets, alignment holds, and R never exceeds the rows bound."""
    wl = WORKLOADS[name]
    _, sr, sl, _, _ = _streams(0)
    idx = draw_routing(wl, sr)
    w = np.ones((wl.T, wl.k), np.float32)
    lay = oracle.layout(wl.mode, wl.T, wl.E, wl.k, wl.A, wl.D, wl.C, idx, w)
    flat = idx.ravel()
    assert lay["flags"] == 0
    cnt = np.bincount(flat, minlength=wl.E)
    assert np.array_equal(lay["cnt"], cnt)
    assert cnt.sum() == wl.T * wl.k
    order = np.argsort(flat, kind="stable")
    rank = np.empty_like(order)
    starts = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    rank[order] = np.arange(flat.size) - starts[flat[order]]
    if wl.mode == oracle.MODE_COMPACT:
        pad = lay["pad"]
        assert np.all(pad % wl.A == 0) and np.all(pad >= cnt) and np.all(pad - cnt < wl.A)
        assert np.array_equal(pad == 0, cnt == 0)
        assert np.all(np.diff(lay["expert_off"]) == pad)
        assert lay["rows"] <= wl.recv_rows_bound
    expect = lay["expert_off"][flat] + rank
    if wl.mode == oracle.MODE_FIXED:
        expect = np.where(rank < wl.C, expect, -1)
    assert np.array_equal(lay["slot"], expect)
    s = lay["slot"][lay["slot"] >= 0]
    assert np.unique(s).size == s.size
    assert np.array_equal(lay["row_src"][s], np.nonzero(lay["slot"] >= 0)[0])


def test_empty_and_degenerate():
    # zero tokens
    lay = oracle.layout(0, 0, 8, 2, 4, 2, 0, np.zeros((0, 2), np.int64))
    assert lay["rows"] == 0 and lay["cnt"].sum() == 0 and lay["flags"] == 0
    # every pair masked
    idx = np.full((5, 3), -1, np.int64)
    lay = oracle.layout(0, 5, 8, 3, 4, 1, 0, idx)
    assert lay["rows"] == 0 and np.all(lay["slot"] == -1) and lay["flags"] == 0
    # all pairs to one expert, k = E (every expert once per token)
    T, E = 9, 4
    idx = np.tile(np.arange(E, dtype=np.int64), (T, 1))
    lay = check_against_brute(0, T, E, E, 4, 2, 0, idx)
    assert list(lay["cnt"]) == [T] * E and list(lay["pad"]) == [12] * E
    # one expert
    idx = np.zeros((6, 1), np.int64)
    lay = check_against_brute(0, 6, 1, 1, 4, 1, 0, idx)
    assert list(lay["slot"]) == list(range(6)) and lay["rows"] == 8


def test_argument_checks():
    with pytest.raises(ValueError):
        oracle.layout(0, 2, 6, 2, 1, 4, 0, np.zeros((2, 2), np.int64))  # E % D
    with pytest.raises(ValueError):
        oracle.layout(0, 2, 6, 2, 0, 1, 0, np.zeros((2, 2), np.int64))  # A < 1
    with pytest.raises(ValueError):
        oracle.layout(1, 2, 6, 2, 1, 1, 0, np.zeros((2, 2), np.int64))  # C < 1


try:
    from hypothesis import given, settings, HealthCheck, strategies as st
except ImportError:  # pragma: no cover - hypothesis is installed in this image
    given = None

if given is not None:
    @st.composite
    def _layout_case(draw):
        """A routing table with masked (-1) and out-of-range ids, any D that
        divides E, either mode, small enough for the O(P^2) definition."""
        T = draw(st.integers(0, 12))
        k = draw(st.integers(1, 4))
        E = draw(st.sampled_from([1, 2, 3, 4, 6, 8]))
        D = draw(st.sampled_from([d for d in range(1, E + 1) if E % d == 0]))
        mode = draw(st.sampled_from([oracle.MODE_COMPACT, oracle.MODE_FIXED]))
        A = draw(st.integers(1, 6)) if mode == oracle.MODE_COMPACT else 1
        C = draw(st.integers(1, 5)) if mode == oracle.MODE_FIXED else 0
        ids = draw(st.lists(st.integers(-1, E + 1), min_size=T * k, max_size=T * k))
        return mode, T, E, k, A, D, C, np.array(ids, np.int64).reshape(T, k)

    @settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(_layout_case())
    def test_layout_matches_definition_on_random_tables(case):
        """Property form of the brute-force pin: every drawn table (duplicate
        experts within a token allowed, masked and bad ids mixed in) gives
        the definition's counts, offsets, slots and flags, and the same
        layout from int32 ids."""
        mode, T, E, k, A, D, C, idx = case
        lay = check_against_brute(mode, T, E, k, A, D, C, idx)
        bf = brute_force_layout(mode, T, E, k, A, D, C, idx)
        assert lay["flags"] == bf["flags"]
        lay32 = oracle.layout(mode, T, E, k, A, D, C, idx.astype(np.int32))
        for key in ("cnt", "pad", "expert_off", "slot", "dest_tokens", "dest_off"):
            assert np.array_equal(lay[key], lay32[key]), key
