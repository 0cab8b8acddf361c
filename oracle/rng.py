"""Counter-based random numbers for sampling verification -- test
infrastructure only.

Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3" (SC 2011), §3 (the Philox S-box:
two 32x32 -> 64-bit multiplications per round with the multipliers
0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl constants 0x9E3779B9
and 0xBB67AE85 between rounds, ten rounds).  Written from that description;
pinned by the authors' known-answer vectors.

The draws of a sampling step ([LD] §3.4 "Sampling verification
(Algorithm 4)"): uniform k of step s under seed x is word 0 of
Philox(counter = (s mod 2^32, s >> 32, k, 0), key = (x mod 2^32, x >> 32)),
mapped to ((word >> 8) + 1) / 2^24, a value in (0, 1] (a token of
probability 0 is never accepted, one of probability 1 always is).
"""
from __future__ import annotations

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Four 32-bit counter words and two key words -> four output words."""
    c0, c1, c2, c3 = (int(x) & _MASK for x in counter)
    k0, k1 = (int(x) & _MASK for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0                       # 64-bit products
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & _MASK, p1 & _MASK, \
                         ((p0 >> 32) ^ c3 ^ k1) & _MASK, p0 & _MASK
    return c0, c1, c2, c3


def uniform(seed: int, step: int, k: int) -> float:
    """Draw k of step `step` under `seed`, in (0, 1]."""
    w = philox4x32_10((step & _MASK, (step >> 32) & _MASK, k & _MASK, 0),
                      (seed & _MASK, (seed >> 32) & _MASK))[0]
    return ((w >> 8) + 1) / 16777216.0
