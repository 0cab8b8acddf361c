"""The configuration planner: Eq. 5/7 of the pages' scaling law ([LD] §4
"Scaling Law"), checked against the oracle's closed forms, against brute
force, and the (alpha, f) fit against data made from known values."""
import itertools
import random

import pytest

from exact_decoding_amd import planner
from oracle import scaling


def test_matches_oracle_closed_forms():
    for alpha, N, W, f in itertools.product((0.0, 0.1, 0.425, 0.9, 1.0), (2, 3, 5, 7),
                                            (1, 2, 7, 15, 30), (1.0, 3.106, 8.0)):
        E = scaling.expected_tokens(alpha, N - 1, W)
        assert planner.expected_tokens(alpha, N - 1, W) == pytest.approx(E, rel=1e-12, abs=1e-12)
        assert planner.compression(alpha, N, W, f) == pytest.approx(
            scaling.compression(alpha, N - 1, W, f), rel=1e-12)


def test_monte_carlo():
    # b independent speculations, token i of each accepted with probability
    # alpha given the earlier ones; the step emits the longest surviving prefix + 1
    rng = random.Random(5)
    alpha, gamma, b, trials = 0.5, 4, 3, 40000
    tot = 0
    for _ in range(trials):
        best = 0
        for _ in range(b):
            k = 0
            while k < gamma and rng.random() < alpha:
                k += 1
            best = max(best, k)
        tot += best + 1
    assert tot / trials == pytest.approx(planner.expected_tokens(alpha, gamma, b), abs=0.03)


def test_best_config_and_speedup():
    table = [{"N": 5, "W": 1, "step_ms": 3.5}, {"N": 5, "W": 7, "step_ms": 4.5},
             {"N": 5, "W": 15, "step_ms": 5.7}, {"N": 5, "W": 20, "step_ms": 8.9}]
    b = planner.best_config(table, ar_step_ms=3.45)
    sp = {r["W"]: planner.predicted_speedup(planner.PAGES_ALPHA, planner.PAGES_F, 5, r["W"],
                                            r["step_ms"], 3.45) for r in table}
    assert b["W"] == max(sp, key=sp.get)
    assert b["speedup"] == pytest.approx(sp[b["W"]])
    with pytest.raises(ValueError):
        planner.best_config([], 1.0)


def test_fit_recovers_known_values():
    alpha, f = 0.425, 3.106
    pts = [(N, W, planner.compression(alpha, N, W, f)) for N in (3, 5, 7) for W in (1, 2, 4, 7, 15, 30)]
    a, ff = planner.fit(pts, steps=60)
    assert a == pytest.approx(alpha, abs=0.01)
    assert ff == pytest.approx(f, rel=0.03)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        planner.expected_tokens(1.5, 4, 2)
    with pytest.raises(ValueError):
        planner.compression(0.4, 5, 2, 0.5)


def test_fit_reproduces_oracle_compressions():
    """Eq. 5/7 fitted to the step compressions of the oracle's lookahead runs
    on the two small random-init models that repeat n-grams
    (tests/golden/scaling_points.json, written by make_scaling_points.py
    from oracle/ alone: N in {3, 4, 5}, W = G in {1 .. 15}, 16 prompts of 128
    tokens).  One (alpha, f) per model reproduces its 24 measured S values
    (1.7 to 3.7) with a root-mean-square error below 0.2 and none off by
    more than 0.4; S grows with W at every N, as the model's diminishing
    returns in b say it should."""
    import json
    import math
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "scaling_points.json")
    data = json.load(open(path))
    for name, pts in data["models"].items():
        trip = [(p["N"], p["W"], p["S"]) for p in pts]
        assert all(p["S"] == p["tokens"] / p["steps"] for p in pts)
        alpha, f = planner.fit(trip)
        assert 0.0 < alpha < 1.0 and f >= 1.0
        res = [planner.compression(alpha, n, w, f) - s for n, w, s in trip]
        rms = math.sqrt(sum(r * r for r in res) / len(res))
        assert rms < 0.2, (name, alpha, f, rms)
        assert max(abs(r) for r in res) < 0.4, (name, alpha, f, res)
        for N in (3, 4, 5):
            s_n = [s for n, w, s in trip if n == N]
            assert s_n[-1] > s_n[0]
