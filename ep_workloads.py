"""Seeded synthetic workloads for MoE dispatch/combine.

This module is the only code shared by the CPU oracle side and the GPU side:
it draws the inputs (hidden states, routing, weights, expert outputs) and
holds the workload shapes. It contains none of the dispatch/combine
arithmetic: no layout, no copies, no quantisation, no reduction.

Shapes follow the DeepEP README (community translation), section
"Performance": 8K tokens per batch, hidden 7168, top-8 experts, FP8 dispatch,
BF16 combine (the V3 setting); the smaller shapes and the decode shape follow
the README's "Example use in inference decoding" section (a fixed per-expert
receive capacity for decode).

Recipe (every workload, seed 0 unless asked otherwise):
  * numpy ``SeedSequence(seed).spawn(5)`` gives five independent streams:
    0 hidden states, 1 routing, 2 weight logits, 3 outlier channels,
    4 expert outputs ``y`` for combine.
  * x ~ N(0, 1) drawn in float32, optional outlier channels multiplied by 100
    in float32, then rounded to bfloat16 (round to nearest even).
  * uniform routing: each token's k experts are the first k entries of an
    independent uniformly random permutation of the E experts (distinct).
  * Zipf routing: p(e) proportional to (e + 1) ** -s; k experts drawn without
    replacement by Gumbel-top-k on log p (expert 0 is the hottest).
  * weights: softmax over each token's k N(0, 1) logits, in float64, then
    stored as float32.
  * y ~ N(0, 1) in float32 rounded to bfloat16, one row per receive row.
bfloat16 arrays are returned as numpy uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MODE_COMPACT = 0
MODE_FIXED = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens
    H: int              # hidden size
    E: int              # experts
    k: int              # experts per token (top-k)
    A: int              # expert_alignment (row padding per expert)
    D: int              # destination buffers (experts grouped contiguously)
    mode: int           # MODE_COMPACT (aligned expert-major) or MODE_FIXED
    C: int              # FIXED: receive capacity per expert (rows)
    dispatch: str       # "bf16" or "fp8"
    routing: str        # "uniform" or "zipf"
    zipf_s: float = 0.0
    outlier_frac: float = 0.0

    @property
    def pairs(self) -> int:
        return self.T * self.k

    @property
    def recv_rows_bound(self) -> int:
        """Rows a receive buffer needs without knowing the counts."""
        if self.mode == MODE_FIXED:
            return self.E * self.C
        return self.T * self.k + self.E * (self.A - 1)

    def with_tokens(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)


WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=256, E=16, k=2, A=1, D=1,
                     mode=MODE_COMPACT, C=0, dispatch="bf16", routing="uniform"),
    "mid": Workload("mid", T=4096, H=4096, E=64, k=6, A=128, D=1,
                    mode=MODE_COMPACT, C=0, dispatch="bf16", routing="uniform"),
    "v3": Workload("v3", T=8192, H=7168, E=256, k=8, A=128, D=8,
                   mode=MODE_COMPACT, C=0, dispatch="fp8", routing="uniform"),
    "skewed_v3": Workload("skewed_v3", T=8192, H=7168, E=256, k=8, A=128, D=8,
                          mode=MODE_COMPACT, C=0, dispatch="fp8", routing="zipf",
                          zipf_s=1.2, outlier_frac=0.01),
    "decode": Workload("decode", T=128, H=7168, E=256, k=8, A=1, D=1,
                       mode=MODE_FIXED, C=128, dispatch="fp8", routing="uniform"),
    # the skewed shape at the stated load of the hottest expert (about 10x
    # the mean: 10.8x at seed 0), which Zipf s = 1.2 overshoots (29.7x)
    "skewed_v3_s06": Workload("skewed_v3_s06", T=8192, H=7168, E=256, k=8, A=128, D=8,
                              mode=MODE_COMPACT, C=0, dispatch="fp8", routing="zipf",
                              zipf_s=0.6, outlier_frac=0.01),
}


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(5)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) with torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_hidden(wl: Workload, rng: np.random.Generator,
                outlier_rng: np.random.Generator, T: Optional[int] = None) -> np.ndarray:
    T = wl.T if T is None else T
    x = rng.standard_normal((T, wl.H), dtype=np.float32)
    n_out = int(round(wl.outlier_frac * wl.H))
    if n_out:
        ch = outlier_rng.choice(wl.H, size=n_out, replace=False)
        x[:, ch] *= np.float32(100.0)
    return f32_to_bf16_bits(x)


def draw_routing(wl: Workload, rng: np.random.Generator, T: Optional[int] = None) -> np.ndarray:
    T = wl.T if T is None else T
    if wl.routing == "uniform":
        keys = rng.random((T, wl.E))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :wl.k]
    elif wl.routing == "zipf":
        logp = -wl.zipf_s * np.log(np.arange(1, wl.E + 1, dtype=np.float64))
        g = rng.gumbel(size=(T, wl.E))
        idx = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :wl.k]
    else:
        raise ValueError(wl.routing)
    return np.ascontiguousarray(idx, dtype=np.int64)


def draw_weights(wl: Workload, rng: np.random.Generator, T: Optional[int] = None) -> np.ndarray:
    T = wl.T if T is None else T
    z = rng.standard_normal((T, wl.k))
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def draw_expert_out(wl: Workload, rng: np.random.Generator, rows: int,
                    chunk_rows: int = 8192) -> np.ndarray:
    """bf16 N(0,1) rows, drawn in chunks to bound host memory."""
    out = np.empty((rows, wl.H), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, wl.H), dtype=np.float32))
    return out


def make_inputs(wl: Workload, seed: int = 0, *, with_y: bool = True) -> dict:
    """All host inputs of one workload: x, topk_idx, topk_w (and y)."""
    sx, sr, sl, so, sy = _streams(seed)
    inp = {
        "x": draw_hidden(wl, sx, so),
        "topk_idx": draw_routing(wl, sr),
        "topk_w": draw_weights(wl, sl),
    }
    if with_y:
        inp["y"] = draw_expert_out(wl, sy, wl.recv_rows_bound)
    return inp


def random_routing_table(rng: np.random.Generator, T: int, E: int, k: int,
                         masked_frac: float = 0.0, bad_frac: float = 0.0,
                         distinct: bool = True) -> np.ndarray:
    """Small routing tables for edge cases: optional -1 (masked) entries,
    out-of-range ids, and repeated experts within a row."""
    if distinct:
        idx = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :k].astype(np.int64)
    else:
        idx = rng.integers(0, E, size=(T, k), dtype=np.int64)
    if masked_frac > 0:
        idx[rng.random((T, k)) < masked_frac] = -1
    if bad_frac > 0:
        m = rng.random((T, k)) < bad_frac
        idx[m] = rng.choice(np.array([E, E + 7, -2, -100], dtype=np.int64), size=int(m.sum()))
    return np.ascontiguousarray(idx)
