"""Helpers shared by the sampling tests: softmax, a pooled chi-square
goodness of fit, and the exact distribution of autoregressive sampling of a
small-vocabulary model (every continuation enumerated, [LD] §3.4
"Mathematical Reformulation": each token conditioned on all before it)."""
import itertools

import numpy as np
from scipy import stats

from oracle import lookahead as LA


def _softmax(l, T):
    p = np.exp((l - l.max()) / T)
    return p / p.sum()


def _gof(counts: dict, probs: dict, n: int, min_expected: float = 5.0) -> float:
    """Chi-square p-value of observed counts against probabilities, rare
    cells pooled."""
    obs, exp, rare_o, rare_e = [], [], 0, 0.0
    for key, p in probs.items():
        if p * n < min_expected:
            rare_o += counts.get(key, 0)
            rare_e += p * n
        else:
            obs.append(counts.get(key, 0))
            exp.append(p * n)
    if rare_e > 0:
        obs.append(rare_o)
        exp.append(rare_e)
    obs, exp = np.array(obs, float), np.array(exp, float)
    exp *= obs.sum() / exp.sum()
    return stats.chisquare(obs, exp).pvalue


def _restricted(l, T, top_k=0, top_p=1.0):
    """softmax(l / T) over the top-K tokens by logit (ties to the lower id),
    then over the shortest run of those, best first, holding a top_p share
    of their probability; written as a plain loop over the ranked tokens."""
    ranked = sorted(range(len(l)), key=lambda v: (-l[v], v))
    if top_k > 0:
        ranked = ranked[:top_k]
    w = {v: np.exp((l[v] - l.max()) / T) for v in ranked}
    total = sum(w.values())
    keep, run = [], 0.0
    for v in ranked:
        keep.append(v)
        run += w[v]
        if top_p < 1.0 and run >= top_p * total:
            break
    p = np.zeros(len(l))
    z = sum(w[v] for v in keep)
    for v in keep:
        p[v] = w[v] / z
    return p


def exact_ar_probs(model, prompt, k: int, T: float, top_k: int = 0, top_p: float = 1.0) -> dict:
    """P(y_1..y_k) = product of the conditionals softmax(logits / T) (restricted
    to top-K / top-P when asked), every continuation of the 8-token vocabulary
    enumerated."""
    V = model.s.vocab
    out = {}
    for seq in itertools.product(range(V), repeat=k - 1):
        lg = LA.score(model, list(prompt) + list(seq))
        p = 1.0
        for j, t in enumerate(seq):
            p *= _restricted(lg[len(prompt) - 1 + j], T, top_k, top_p)[t]
        last = _restricted(lg[len(prompt) - 1 + k - 1], T, top_k, top_p)
        for t in range(V):
            out[tuple(seq) + (t,)] = p * last[t]
    return out


# [1, 2] and the start of the micro model's own greedy continuation of it, so
# the prompt's n-grams are likely continuations and candidates are accepted
# in most first steps
MICRO_PROMPT = [1, 2, 7, 5, 4, 5, 7, 5, 7, 0, 5, 5, 7, 5]
