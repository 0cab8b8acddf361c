"""Choosing (N, W, G) for a GPU from its measured step times and the pages'
acceptance model.

[LD] §4 "Scaling Law: Trading Per-Step FLOPs for Fewer Steps" models a
lookahead step as b = W (= G) parallel speculations of length gamma = N - 1,
each token accepted with probability alpha:

  Eq. 5   E(#tokens) = (gamma + 1) - sum_{i=1..gamma} (1 - alpha^i)^b
  Eq. 7   S = (f - 1 + E(#tokens)) / f

with the fudge factor f (one step in f carries a good speculation).  The
pages fit alpha = 0.425, f = 3.106 for a 7B chat model on MT-Bench.

Speedup over autoregressive decoding on a given GPU is S / (t_step / t_AR):
the compression the model reaches divided by the compression the step's cost
demands.  `best_config` maximises it over a measured table of step times;
`fit` recovers (alpha, f) from measured compressions.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

PAGES_ALPHA = 0.425
PAGES_F = 3.106


def expected_tokens(alpha: float, gamma: int, b: int) -> float:
    """Eq. 5: expected tokens accepted from b speculations of length gamma."""
    if not 0.0 <= alpha <= 1.0 or gamma < 0 or b < 0:
        raise ValueError("need 0 <= alpha <= 1, gamma >= 0, b >= 0")
    miss = 0.0
    p = 1.0
    for _ in range(gamma):
        p *= alpha                 # alpha^i: one speculation survives to position i
        miss += (1.0 - p) ** b     # every one of the b fails by position i
    return (gamma + 1) - miss


def compression(alpha: float, N: int, W: int, f: float) -> float:
    """Eq. 7 with gamma = N - 1 and b = W (= G)."""
    if f < 1.0:
        raise ValueError("f >= 1")
    return (f - 1.0 + expected_tokens(alpha, N - 1, W)) / f


def predicted_speedup(alpha: float, f: float, N: int, W: int, step_ms: float,
                      ar_step_ms: float) -> float:
    """Lookahead tokens/s over AR tokens/s on a GPU whose lookahead step at
    (N, W, G = W) takes step_ms and whose AR step takes ar_step_ms."""
    return compression(alpha, N, W, f) * ar_step_ms / step_ms


def best_config(table: Iterable[dict], ar_step_ms: float, alpha: float = PAGES_ALPHA,
                f: float = PAGES_F) -> dict:
    """The row of `table` (dicts with N, W, step_ms) with the highest
    predicted speedup; returns that row with `S` and `speedup` added."""
    best = None
    for row in table:
        s = compression(alpha, row["N"], row["W"], f)
        sp = s * ar_step_ms / row["step_ms"]
        if best is None or sp > best["speedup"]:
            best = dict(row, S=s, speedup=sp)
    if best is None:
        raise ValueError("empty table")
    return best


def fit(points: Sequence[tuple[int, int, float]], f_max: float = 20.0,
        steps: int = 100) -> tuple[float, float]:
    """Least-squares (alpha, f) for measured (N, W, S) triples: a grid of
    steps x steps cells over alpha in (0, 1) and f in [1, f_max], then the
    same grid over the best cell's neighbourhood."""
    if not points:
        raise ValueError("no points")

    def err(a: float, ff: float) -> float:
        return sum((compression(a, n, w, ff) - s) ** 2 for n, w, s in points)

    def search(a0: float, a1: float, f0: float, f1: float) -> tuple[float, float, float]:
        best = (math.inf, a0, f0)
        for i in range(steps + 1):
            a = a0 + (a1 - a0) * i / steps
            for j in range(steps + 1):
                ff = f0 + (f1 - f0) * j / steps
                e = err(a, ff)
                if e < best[0]:
                    best = (e, a, ff)
        return best

    lo_a, hi_a = 1e-6, 1.0 - 1e-6
    _, a, ff = search(lo_a, hi_a, 1.0, f_max)
    da, df = (hi_a - lo_a) / steps, (f_max - 1.0) / steps
    _, a, ff = search(max(lo_a, a - da), min(hi_a, a + da), max(1.0, ff - df),
                      min(f_max, ff + df))
    return a, ff
