"""Seeded synthetic inputs for the LLM.int8() linear layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no detection, no quantization, no product).  Both the CPU
oracle and the HIP path take their inputs from here, byte for byte.

The shapes stand in for the first feed-forward layer of decoder models whose
intermediate width is four times the model width (the speed study in the
"INT8演算による速度改善" section of the zenn.dev summary of the LLM.int8()
paper), plus, at 13B width, the second feed-forward layer (K = 4h, N = h)
and an attention projection (K = N = h) of the same block; the planted
outlier columns follow that page's "outlierは極めて"系統的"に出現する"
section (about 0.1 % of hidden dims carry the outliers at 6.7B scale).  No
dataset, model or trained weight is used.

Recipe (one ``numpy.random.default_rng(seed)`` stream, PCG64, drawn in this
order): X base ~ N(0, sigma) -> outlier column indices (``rng.choice``
without replacement; Tiny fixes columns 3 and 41) -> per column, the rows it
is planted on (all rows, or a fraction drawn without replacement) ->
magnitudes U(lo, hi) -> a fair-coin sign per planted element -> W ~ N(0,
w_sigma) -> bias ~ N(0, b_sigma) when the workload has one.  The decode
sweep draws its one weight from ``default_rng([seed, 1])`` instead, so every
T sees the same CB/SCB.  Planted values
replace the base value.  Everything is drawn in float64 and rounded to fp16
(round to nearest even) on the host; large W is drawn in row chunks, which
yields the same stream as one draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

THRESHOLD = 6.0


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    K: int
    N: int
    x_sigma: float
    n_planted: int
    planted_lo: float
    planted_hi: float
    planted_row_frac: float  # 1.0 = every row
    w_sigma: float
    b_sigma: Optional[float]  # None = no bias
    fixed_columns: Sequence[int] = field(default_factory=tuple)
    threshold: float = THRESHOLD


WORKLOADS = {
    # the pages' 64x64 nn.Linear example, 16 tokens
    "tiny": Workload("tiny", 16, 64, 64, 1.0, 2, 8.0, 20.0, 1.0, 0.02, 0.01, (3, 41)),
    "6.7b": Workload("6.7b", 2048, 4096, 16384, 1.0, 4, 6.0, 60.0, 0.2, 0.02, None),
    "13b": Workload("13b", 2048, 5120, 20480, 1.0, 6, 6.0, 60.0, 1.0, 0.02, 0.01),
    "175b": Workload("175b", 4096, 12288, 49152, 1.5, 12, 6.0, 80.0, 1.0, 0.015, None),
    # one GPU's share of that layer under an 8-way split of the output
    # channels: the same X, and (W drawn in row chunks from the same stream)
    # exactly the first 6144 rows of its W
    "175b-n8": Workload("175b-n8", 4096, 12288, 6144, 1.5, 12, 6.0, 80.0, 1.0, 0.015, None),
    # the rest of a 13B block: the second FF layer (down projection, K = 4h,
    # N = h) and an attention projection (K = N = h); same activation recipe
    "13b-down": Workload("13b-down", 2048, 20480, 5120, 1.0, 20, 6.0, 60.0, 1.0, 0.01, 0.01),
    "13b-attn": Workload("13b-attn", 2048, 5120, 5120, 1.0, 6, 6.0, 60.0, 1.0, 0.02, 0.01),
    # decode sweep: the 175B layer's weight, T tokens of activations
    "decode1": Workload("decode1", 1, 12288, 49152, 1.0, 12, 6.0, 80.0, 1.0, 0.015, None),
    "decode8": Workload("decode8", 8, 12288, 49152, 1.0, 12, 6.0, 80.0, 1.0, 0.015, None),
    "decode32": Workload("decode32", 32, 12288, 49152, 1.0, 12, 6.0, 80.0, 1.0, 0.015, None),
}

_W_CHUNK_ROWS = 2048


def _fp16(a: np.ndarray) -> np.ndarray:
    return a.astype(np.float16)


def make_activations(rng: np.random.Generator, T: int, K: int, x_sigma: float,
                     n_planted: int, lo: float, hi: float, row_frac: float,
                     fixed_columns: Sequence[int] = ()):
    """X fp16 [T,K] with planted large-magnitude columns; returns (X, cols)."""
    X = rng.standard_normal((T, K)) * x_sigma
    if fixed_columns:
        cols = np.asarray(fixed_columns, dtype=np.int64)
    elif n_planted > 0:
        cols = np.sort(rng.choice(K, size=n_planted, replace=False)).astype(np.int64)
    else:
        cols = np.zeros(0, dtype=np.int64)
    if row_frac >= 1.0:
        rows = [np.arange(T)] * len(cols)
    else:
        nr = int(round(row_frac * T))
        rows = [np.sort(rng.choice(T, size=nr, replace=False)) for _ in cols]
    for c, r in zip(cols, rows):
        mag = rng.uniform(lo, hi, size=len(r))
        sign = np.where(rng.integers(0, 2, size=len(r)) == 1, 1.0, -1.0)
        X[r, c] = sign * mag
    return _fp16(X), cols


def make_weight(rng: np.random.Generator, N: int, K: int, w_sigma: float) -> np.ndarray:
    """W fp16 [N,K] (nn.Linear layout), drawn in row chunks."""
    W = np.empty((N, K), dtype=np.float16)
    for r0 in range(0, N, _W_CHUNK_ROWS):
        r1 = min(N, r0 + _W_CHUNK_ROWS)
        W[r0:r1] = _fp16(rng.standard_normal((r1 - r0, K)) * w_sigma)
    return W


def make_inputs(name: str, seed: int = 0, with_weight: bool = True):
    """Return dict(X, W, bias, threshold, planted, workload) for a named workload."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    X, cols = make_activations(rng, wl.T, wl.K, wl.x_sigma, wl.n_planted,
                               wl.planted_lo, wl.planted_hi, wl.planted_row_frac,
                               wl.fixed_columns)
    W = None
    if with_weight:
        # the decode sweep quantizes one weight once and reuses it for every T,
        # so its W comes from a stream of its own that does not depend on T
        wrng = np.random.default_rng([seed, 1]) if name.startswith("decode") else rng
        W = make_weight(wrng, wl.N, wl.K, wl.w_sigma)
    bias = None
    if wl.b_sigma is not None:
        bias = _fp16(rng.standard_normal(wl.N) * wl.b_sigma)
    return dict(X=X, W=W, bias=bias, threshold=wl.threshold, planted=cols, workload=wl)


def make_random_case(seed: int, T: int, K: int, N: int, *, x_sigma: float = 1.0,
                     n_planted: int = 0, lo: float = 6.0, hi: float = 40.0,
                     row_frac: float = 1.0, w_sigma: float = 0.02,
                     bias: bool = True, b_sigma: float = 0.01):
    """A free-shape case drawn with the same recipe (used for ragged shapes)."""
    rng = np.random.default_rng(seed)
    X, cols = make_activations(rng, T, K, x_sigma, min(n_planted, K), lo, hi, row_frac)
    W = make_weight(rng, N, K, w_sigma)
    b = _fp16(rng.standard_normal(N) * b_sigma) if bias else None
    return dict(X=X, W=W, bias=b, threshold=THRESHOLD, planted=cols)
