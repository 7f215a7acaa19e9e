"""Seeded synthetic inputs for the LRKV workloads.

Random draws only.  This module holds none of the method's arithmetic: no projection, no
attention, no cache layout.  It serves both the oracle side (tests) and the library side
(tests, bench.py).  Every generator takes its seed explicitly; the draw order is part of
each docstring so a workload can be rebuilt exactly.

Distributions follow the workload statements: activations X ~ N(0, 1); projection weights
W_S_K, W_S_V, U_K, U_V, W_q ~ N(0, 1/fan_in) with fan_in = d; expansion bases B_K, B_V ~
N(0, 1/r) (fan_in r, since the private row of width r is what B expands); decode queries
q ~ N(0, 1).  Floats are drawn in float64 by numpy's PCG64 generator and stored as float32;
`to_bf16_bits` turns them into bfloat16 codes (round to nearest even, via torch's own cast).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = 0
BF16 = 1


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 codes (uint16), nearest-even, by torch's dtype cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 codes -> float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape) * std).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    """Shape of one workload.  `lens` is the per-request token count after the append."""

    name: str
    dtype: int
    H: int
    d_h: int
    r: int
    d: int
    B: int
    lens: tuple
    page_size: int = 16

    @property
    def max_len(self) -> int:
        return max(self.lens) if self.lens else 0

    @property
    def tokens(self) -> int:
        return int(sum(self.lens))


# The five workloads.  Sizes as stated for each; C2's lengths are drawn (see c2_lengths).
C0 = Workload("c0_tiny_fp32", F32, H=4, d_h=16, r=4, d=64, B=1, lens=(65,))
C1 = Workload("c1_bf16_b8_t4096", BF16, H=16, d_h=128, r=56, d=2048, B=8, lens=(4096,) * 8)
C3 = Workload("c3_bf16_b4_t131072", BF16, H=32, d_h=128, r=32, d=4096, B=4, lens=(131072,) * 4)
C4 = Workload("c4_bf16_prefill_b4_t8192", BF16, H=16, d_h=128, r=56, d=2048, B=4,
              lens=(8192,) * 4)


def c2_lengths(seed: int = 2, B: int = 32, lo: int = 512, hi: int = 32768) -> tuple:
    """Per-request lengths for the ragged paged workload: integers uniform on [lo, hi]."""
    g = np.random.default_rng(seed)
    return tuple(int(x) for x in g.integers(lo, hi + 1, size=B))


C2 = Workload("c2_bf16_paged_ragged_b32", BF16, H=16, d_h=128, r=56, d=2048, B=32,
              lens=c2_lengths())


def projection_weights(seed: int, d: int, H: int, d_h: int, r: int, with_wq: bool = False):
    """Weights of one layer, drawn in this order from default_rng(seed):
    W_SK [d, d_h], W_SV [d, d_h], U_K [d, H, r], U_V [d, H, r] ~ N(0, 1/d);
    B_K [H, d_h, r], B_V [H, d_h, r] ~ N(0, 1/r); then, if asked, W_q [d, H*d_h] ~ N(0, 1/d).
    """
    g = np.random.default_rng(seed)
    sd = 1.0 / math.sqrt(d)
    w = {
        "W_SK": _normal(g, (d, d_h), sd),
        "W_SV": _normal(g, (d, d_h), sd),
        "U_K": _normal(g, (d, H, r), sd),
        "U_V": _normal(g, (d, H, r), sd),
        "B_K": _normal(g, (H, d_h, r), 1.0 / math.sqrt(r)),
        "B_V": _normal(g, (H, d_h, r), 1.0 / math.sqrt(r)),
    }
    if with_wq:
        w["W_q"] = _normal(g, (d, H * d_h), sd)
    return w


def activations(seed: int, n_rows: int, d: int) -> np.ndarray:
    """X [n_rows, d] ~ N(0, 1), from default_rng(seed) (a stream separate from the weights)."""
    g = np.random.default_rng(seed)
    return g.standard_normal((n_rows, d), dtype=np.float32)


def queries(seed: int, B: int, q_len: int, H: int, d_h: int, scale: float = 1.0) -> np.ndarray:
    """q [B, q_len, H, d_h] ~ N(0, scale^2), from default_rng(seed)."""
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, q_len, H, d_h), dtype=np.float32) * np.float32(scale))


def factored_rows(seed: int, n: int, H: int, d_h: int, r: int):
    """Cached rows drawn directly, i.i.d. N(0, 1), from default_rng(seed) in this order:
    S_K [n, d_h], S_V [n, d_h], R_K [n, H, r], R_V [n, H, r].

    A row x of N(0, 1) activations projected through N(0, 1/d) weights has entries of
    variance |x|^2 / d ~ 1 and cross-covariances of order d^(-1/2); i.i.d. N(0, 1) is the
    large-d law of those projections.  Used where projecting every row in float64 would
    cost teraflops (hundreds of thousands of cached rows).
    """
    g = np.random.default_rng(seed)
    SK = g.standard_normal((n, d_h), dtype=np.float32)
    SV = g.standard_normal((n, d_h), dtype=np.float32)
    RK = g.standard_normal((n, H, r), dtype=np.float32)
    RV = g.standard_normal((n, H, r), dtype=np.float32)
    return SK, SV, RK, RV


def page_assignment(seed: int, lens, page_size: int, permute: bool):
    """Page ids for each request's positions.

    Request b needs ceil(lens[b] / page_size) pages; pages are numbered request by request
    and, when `permute` is set, shuffled by default_rng(seed).permutation over the whole
    pool.  Returns (page_table [B, max_pages] int32, num_pages).  Entries past a request's
    last page hold 0, a valid page id, so that no table entry ever points outside the pool.
    """
    n_pages = [-(-int(t) // page_size) for t in lens]
    total = int(sum(n_pages))
    ids = np.arange(total, dtype=np.int64)
    if permute and total:
        ids = np.random.default_rng(seed).permutation(total)
    width = max(1, max(n_pages) if n_pages else 1)
    table = np.zeros((len(lens), width), dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = ids[off:off + n]
        off += n
    return table, max(total, 1)


def rope_table(n_pos: int, d_h: int, base: float = 10000.0) -> np.ndarray:
    """Rotary table [n_pos, d_h/2, 2] float32: (cos, sin) of the angle j * base^(-2m/d_h)
    for position j and feature pair m (the usual rotary frequencies; the factored-cache
    method takes whatever table the model was trained with).  Angles in float64, then
    rounded to float32; the table itself is the input both sides read."""
    j = np.arange(n_pos, dtype=np.float64)[:, None]
    theta = base ** (-2.0 * np.arange(d_h // 2, dtype=np.float64) / d_h)
    ang = j * theta[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
