"""Seeded synthetic inputs for the soft top-k path.

This module only draws numbers: it holds none of the operator's arithmetic, so
both the GPU path's tests and the CPU oracle's tests can take their inputs from
it.  Every array is drawn with numpy's PCG64 ``default_rng(seed)`` in fp64 and
rounded once to fp32, so the oracle (which widens fp32 exactly) and the GPU see
the same bytes.

Named workloads (score vector, budget k, temperature alpha):

  c1  n=4,096        N(0,1)                           k=64         alpha=0.1
  c2  n=1,000,000    N(0,1)                           k=10,000     alpha=0.05
  c3  n=10,000,000   0.5 * Student-t(3)               k=100,000    alpha=0.02
  c4  n=100,000,000  U(0,1)                           k=1,000,000  alpha=1e-3
  c5  n=10,000,000   6,000,000 x 0.5 exactly, 3,900,000 x N(0,1),
                     100,000 x N(5, 0.1), shuffled;   k=#{s>0.5}+3,000,000, alpha=1e-4

The upstream gradient for the backward pass is an independent stream,
``default_rng(seed + 1).standard_normal(n)`` rounded to fp32.

Batched-row workloads (rows x n_row scores, one soft top-k per row, shared k
and alpha), shaped after the uses the pages name (expert routing, attention
pruning):

  r1  65,536 rows x 256      N(0,1)   k=8    alpha=0.1
  r2  8,192 rows x 2,048     N(0,1)   k=64   alpha=0.05
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DISTRIBUTIONS = ("normal", "student_t3_half", "uniform", "clustered", "sorted_normal", "equal")


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    dist: str
    k: float
    alpha: float
    seed: int = 0
    description: str = ""


WORKLOADS = {
    "c1": Workload("c1", 4096, "normal", 64.0, 0.1, 0,
                   "n=4096 N(0,1), k=64, alpha=0.1"),
    "c2": Workload("c2", 1_000_000, "normal", 10_000.0, 0.05, 0,
                   "n=1e6 N(0,1), k=1e4, alpha=0.05"),
    "c3": Workload("c3", 10_000_000, "student_t3_half", 100_000.0, 0.02, 0,
                   "n=1e7 0.5*t(3), k=1e5, alpha=0.02"),
    "c4": Workload("c4", 100_000_000, "uniform", 1_000_000.0, 1e-3, 0,
                   "n=1e8 U(0,1), k=1e6, alpha=1e-3"),
    # k of c5 depends on the drawn scores; it is filled in by make_workload.
    "c5": Workload("c5", 10_000_000, "clustered", float("nan"), 1e-4, 0,
                   "n=1e7 clustered (60% exactly 0.5), k=#{s>0.5}+3e6, alpha=1e-4"),
}


def draw_scores(dist: str, n: int, seed: int = 0) -> np.ndarray:
    """Draw n fp32 scores of the named distribution with default_rng(seed)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal(n)
    elif dist == "student_t3_half":
        x = 0.5 * rng.standard_t(3, size=n)
    elif dist == "uniform":
        x = rng.random(n)
    elif dist == "clustered":
        n_tie = (6 * n) // 10
        n_far = n // 100
        n_mid = n - n_tie - n_far
        x = np.concatenate([
            np.full(n_tie, 0.5),
            rng.standard_normal(n_mid),
            rng.normal(5.0, 0.1, size=n_far),
        ])
        x = x[rng.permutation(n)]
    elif dist == "sorted_normal":
        x = np.sort(rng.standard_normal(n))
    elif dist == "equal":
        x = np.full(n, 0.25)
    else:
        raise ValueError("unknown distribution %r" % dist)
    return np.ascontiguousarray(x.astype(np.float32))


def clustered_budget(s: np.ndarray) -> float:
    """Budget of the clustered workload: all scores above the tie plus half the tie."""
    n_tie = (6 * s.size) // 10
    return float(np.count_nonzero(s > np.float32(0.5)) + n_tie // 2)


def draw_grad(n: int, seed: int = 0) -> np.ndarray:
    """Upstream gradient for the backward pass: an independent N(0,1) stream."""
    rng = np.random.default_rng(seed + 1)
    return np.ascontiguousarray(rng.standard_normal(n).astype(np.float32))


def make_workload(name: str, n: int | None = None, seed: int | None = None):
    """Return (scores fp32, k, alpha, workload) for a named workload.

    ``n`` overrides the size (the budget is scaled to keep k/n fixed); this is
    how the tests build small instances with the same distribution.
    """
    w = WORKLOADS[name]
    nn = w.n if n is None else int(n)
    sd = w.seed if seed is None else int(seed)
    s = draw_scores(w.dist, nn, sd)
    if w.dist == "clustered":
        k = clustered_budget(s)
    else:
        k = w.k if nn == w.n else max(1.0, round(w.k * nn / w.n))
    return s, float(k), float(w.alpha), w


@dataclass(frozen=True)
class RowWorkload:
    name: str
    rows: int
    n_row: int
    dist: str
    k: float
    alpha: float
    seed: int = 0
    description: str = ""


ROW_WORKLOADS = {
    "r1": RowWorkload("r1", 65536, 256, "normal", 8.0, 0.1, 0,
                      "65536 rows x 256 N(0,1), k=8, alpha=0.1"),
    "r2": RowWorkload("r2", 8192, 2048, "normal", 64.0, 0.05, 0,
                      "8192 rows x 2048 N(0,1), k=64, alpha=0.05"),
}


def make_row_workload(name: str, rows: int | None = None):
    """Return (scores fp32 [rows, n_row], k, alpha, workload) for a named row workload;
    ``rows`` overrides the row count (same rows, fewer of them)."""
    w = ROW_WORKLOADS[name]
    r = w.rows if rows is None else int(rows)
    s = draw_scores(w.dist, r * w.n_row, w.seed).reshape(r, w.n_row)
    return np.ascontiguousarray(s), float(w.k), float(w.alpha), w
