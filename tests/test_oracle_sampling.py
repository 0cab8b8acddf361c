"""Pins of the oracle's sampling verification ([LD] §3.4 "Sampling
verification (Algorithm 4)") and of its random draws.

The pages claim (and prove in their Appendix B) that Algorithm 4 leaves the
output distribution that of sampling from the model.  These tests check the
oracle against that claim and against the generator's published
known-answer vectors, not against its own formulas:
  * Philox4x32-10 against the Random123 known-answer vectors;
  * the draws are uniform on (0, 1] (chi-square);
  * one verification step on synthetic logits emits its first token with
    probability softmax(row 0 / T) and, after accepting candidate token c,
    its second with probability softmax(row of c / T) (rejection sampling);
  * T -> 0 reduces Algorithm 4 to greedy verification (Algorithm 3);
  * lookahead decoding with sampling on an 8-token model reproduces the
    exact distribution of the first two tokens of autoregressive sampling,
    enumerated from the model's conditionals, also under top-K / top-P;
  * the top-K / top-P cuts on hand-worked rows (ties, shares exactly at and
    past a boundary).
"""
import collections
import itertools
import os

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import rng
from oracle import lookahead as LA
from oracle.model import OracleModel

from sampling_util import MICRO_PROMPT, _gof, _softmax, exact_ar_probs

HERE = os.path.dirname(__file__)


def test_philox_known_answers():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        assert rng.philox4x32_10(v[0:4], v[4:6]) == tuple(v[6:10])


def test_draws_uniform_on_open_closed_interval():
    u = np.array([rng.uniform(1234, s, k) for s in range(40) for k in range(250)])
    assert u.min() > 0.0 and u.max() <= 1.0
    assert np.all(np.mod(u * 2 ** 24, 1.0) == 0)          # multiples of 2^-24
    counts, _ = np.histogram(u, bins=20, range=(0.0, 1.0))
    assert stats.chisquare(counts).pvalue > 1e-3
    # different keys and counters give different streams
    assert rng.uniform(1, 0, 0) != rng.uniform(2, 0, 0) != rng.uniform(1, 1, 0)


def test_one_step_is_rejection_sampling():
    gen = np.random.default_rng(3)
    V, N, T = 6, 3, 1.3
    cands = [(2, 4), (2, 1), (5, 0), (2, 4), (3, 3)]
    base = 1                      # no lookahead rows: verification rows follow row 0
    M = 1 + len(cands) * (N - 1)
    logits = gen.normal(0, 1.2, size=(M, V))
    n = 20000
    first = collections.Counter()
    second = collections.defaultdict(collections.Counter)
    for seed in range(n):
        emit, acc, g0, _ = LA.sample_verify(logits, cands, N, base, T, seed, 0)
        first[emit[0]] += 1
        if acc >= 1:
            second[emit[0]][emit[1]] += 1
            assert cands[g0][0] == emit[0]
    p1 = _softmax(logits[0], T)
    assert _gof(first, dict(enumerate(p1)), n) > 1e-3
    # after accepting c the next token follows the row of the first candidate
    # starting with c
    for c, cnt in second.items():
        g = next(g for g, cd in enumerate(cands) if cd[0] == c)
        p2 = _softmax(logits[base + g * (N - 1)], T)
        tot = sum(cnt.values())
        if tot >= 400:
            assert _gof(cnt, dict(enumerate(p2)), tot) > 1e-3, c
    assert sum(sum(c.values()) for c in second.values()) > 2000   # candidates were accepted


def test_zero_temperature_limit_is_greedy():
    gen = np.random.default_rng(4)
    V, N = 7, 4
    for trial in range(30):
        G = int(gen.integers(0, 5))
        cands = [tuple(int(x) for x in gen.integers(0, V, N - 1)) for _ in range(G)]
        base = 1
        M = 1 + G * (N - 1)
        logits = gen.normal(0, 1.0, size=(M, V))
        # plant agreement so longer prefixes get accepted sometimes
        a = logits.argmax(axis=1)
        if G:
            g = int(gen.integers(0, G))
            c = [int(a[0])]
            for i in range(1, N - 1):
                c.append(int(a[base + g * (N - 1) + i - 1]))
            cands[g] = tuple(c)
            a = logits.argmax(axis=1)
        emit_s, acc_s, _, _ = LA.sample_verify(logits, cands, N, base, 1e-4, trial, 0)
        emit_g, acc_g, _, _ = LA._greedy_verify(a, cands, N, base)
        assert (emit_s, acc_s) == (emit_g, acc_g)


@pytest.fixture(scope="module")
def micro():
    s = synth.SHAPES["micro"]
    w = [synth.gen_tensor(s, 0, i) for i in range(len(synth.weight_names(s)))]
    return OracleModel(s, w)


def test_ar_sampling_matches_enumeration(micro):
    T = 1.5
    probs = exact_ar_probs(micro, MICRO_PROMPT, 2, T)
    assert sum(probs.values()) == pytest.approx(1.0)
    n = 1500
    cnt = collections.Counter(tuple(LA.greedy_ar(micro, MICRO_PROMPT, 2, temperature=T,
                                                 seed=s).tokens) for s in range(n))
    assert _gof(cnt, probs, n) > 1e-3


def test_lookahead_sampling_preserves_the_distribution(micro):
    T, N, W, G = 1.5, 3, 3, 3
    probs = exact_ar_probs(micro, MICRO_PROMPT, 2, T)
    n = 1500
    cnt = collections.Counter()
    accepted = 0
    for s in range(n):
        win = synth.gen_window(N, W, micro.s.vocab, seed=100 + s)
        r = LA.lookahead(micro, MICRO_PROMPT, N, W, G, 2, win, prompt_ref=True,
                         temperature=T, seed=s)
        cnt[tuple(r.tokens)] += 1
        accepted += r.accepted[0] > 0
    assert accepted > n // 10          # the rejection path was exercised
    assert _gof(cnt, probs, n) > 1e-3


def test_top_k_top_p_cuts_by_hand():
    """R20 on rows worked out by hand (T = 1)."""
    def kept(l, k=0, p=1.0):
        e, _ = LA.restricted_weights(np.array(l, dtype=np.float64), 1.0, k, p)
        return sorted(np.nonzero(e)[0].tolist())
    l = [1.0, 3.0, 3.0, 2.0, 3.0]
    assert kept(l) == [0, 1, 2, 3, 4]
    assert kept(l, 1) == [1]                 # three-way tie for the top: lowest id
    assert kept(l, 2) == [1, 2]
    assert kept(l, 3) == [1, 2, 4]
    assert kept(l, 4) == [1, 2, 3, 4]
    assert kept(l, 9) == [0, 1, 2, 3, 4]     # K past the vocabulary keeps all
    # probabilities 0.05, 0.5, 0.15, 0.3 (ranked 1, 3, 2, 0)
    lp = np.log([0.05, 0.5, 0.15, 0.3])
    assert kept(lp, 0, 0.4) == [1]           # 0.5 already holds 0.4
    assert kept(lp, 0, 0.75) == [1, 3]       # 0.5 + 0.3
    assert kept(lp, 0, 0.9) == [1, 2, 3]     # + 0.15
    assert kept(lp, 0, 0.99) == [0, 1, 2, 3]
    # top-K first, then top-P of what is left: 0.5 / (0.5 + 0.3) = 0.625
    assert kept(lp, 2, 0.6) == [1]
    assert kept(lp, 2, 0.7) == [1, 3]
    # the kept weights are the unrestricted ones
    e, _ = LA.restricted_weights(lp, 1.0, 2, 1.0)
    assert e[1] == pytest.approx(1.0) and e[3] == pytest.approx(0.6)


def test_restricted_ar_sampling_matches_enumeration(micro):
    T, K, Pp = 1.5, 4, 0.8
    probs = exact_ar_probs(micro, MICRO_PROMPT, 2, T, K, Pp)
    assert sum(probs.values()) == pytest.approx(1.0)
    assert sum(1 for v in probs.values() if v == 0.0) > 0      # the cut removed something
    n = 1500
    cnt = collections.Counter(tuple(LA.greedy_ar(micro, MICRO_PROMPT, 2, temperature=T, seed=s,
                                                 top_k=K, top_p=Pp).tokens) for s in range(n))
    assert all(probs[key] > 0 for key in cnt)                  # nothing outside the cut
    assert _gof(cnt, probs, n) > 1e-3


def test_restricted_lookahead_sampling_preserves_the_distribution(micro):
    T, N, W, G, K, Pp = 1.5, 3, 3, 3, 4, 0.8
    probs = exact_ar_probs(micro, MICRO_PROMPT, 2, T, K, Pp)
    n = 1500
    cnt = collections.Counter()
    accepted = 0
    for s in range(n):
        win = synth.gen_window(N, W, micro.s.vocab, seed=100 + s)
        r = LA.lookahead(micro, MICRO_PROMPT, N, W, G, 2, win, prompt_ref=True,
                         temperature=T, seed=s, top_k=K, top_p=Pp)
        cnt[tuple(r.tokens)] += 1
        accepted += r.accepted[0] > 0
    assert accepted > n // 10
    assert all(probs[key] > 0 for key in cnt)
    assert _gof(cnt, probs, n) > 1e-3
