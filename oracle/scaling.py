"""Closed forms of the pages' scaling law -- test infrastructure only.

[LD] §3.4 "Scaling Law: Trading Per-Step FLOPs for Fewer Steps":
  Eq. 5  E(#tokens) = (gamma + 1) - sum_{i=1..gamma} (1 - alpha^i)^b
         for b parallel speculations of length gamma = N - 1 with per-token
         acceptance alpha;
  Eq. 4  b = 1: (1 - alpha^(gamma+1)) / (1 - alpha);
  Eq. 7  S = (f - 1 + E) / f with the fitted fudge factor f.
"""
from __future__ import annotations


def expected_tokens(alpha: float, gamma: int, b: int) -> float:
    return (gamma + 1) - sum((1.0 - alpha ** i) ** b for i in range(1, gamma + 1))


def expected_tokens_single(alpha: float, gamma: int) -> float:
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def compression(alpha: float, gamma: int, b: int, f: float) -> float:
    return (f - 1.0 + expected_tokens(alpha, gamma, b)) / f
