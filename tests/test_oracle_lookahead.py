"""Pins of the oracle's lookahead algorithm: brute-force mask enumeration,
the pages' Fig. 1 / Fig. 2(b) examples, row equivalence against plain causal
forwards, exactness against greedy AR, verification special cases, pool and
window invariants, and the scaling-law closed forms."""
import itertools
import json
import os

import numpy as np
import pytest

import synth
from oracle import lookahead as la
from oracle.model import OracleModel, causal_vis, argmax_lowest
from oracle.scaling import expected_tokens, expected_tokens_single, compression

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _model(dtype="f32", seed=0, **kw):
    base = dict(name="t", n_layers=2, d_model=64, n_heads=4, n_kv_heads=4, head_dim=16,
                d_ff=256, vocab=256, dtype=dtype)
    base.update(kw)
    s = synth.ModelShape(**base)
    return OracleModel(s, synth.gen_weights(s, seed))


def _chain(q, N, W, G):
    """Rows making up row q's context, built from the n-gram / trajectory
    reading directly (not from the set rules): the current token, then for
    a lookahead row the oldest level's columns left of its own and its own
    column up to its level; for a verification row its own n-gram prefix."""
    kd = la.row_kind(q, N, W, G)
    rows = [0]
    if kd[0] == "la":
        _, l, k = kd
        rows += [1 + 0 * W + kk for kk in range(k)]
        rows += [1 + ll * W + k for ll in range(l + 1)]
    elif kd[0] == "ver":
        _, g, i = kd
        base = 1 + W * (N - 1)
        rows += [base + g * (N - 1) + ii - 1 for ii in range(1, i + 1)]
    return rows


# -- mask ----------------------------------------------------------------------

def test_mask_enumeration_small():
    for N in range(2, 7):
        for W in range(0, 7):
            for G in range(0, 7):
                M = la.n_rows(N, W, G)
                mask = la.block_mask(N, W, G)
                for q in range(M):
                    expect = np.zeros(M, bool)
                    expect[_chain(q, N, W, G)] = True
                    assert np.array_equal(mask[q], expect), (N, W, G, q)


def test_mask_chain_property():
    """Each row sees exactly one block row at every position from P to its
    own position, i.e. 'only tokens with a smaller position index' and a
    causal chain ([LD] §3.4 'The custom attention mask')."""
    for N, W, G in itertools.product(range(2, 7), range(0, 7), range(0, 7)):
        M = la.n_rows(N, W, G)
        mask = la.block_mask(N, W, G)
        off = np.array([la.row_offset(r, N, W, G) for r in range(M)])
        for q in range(M):
            seen = sorted(off[mask[q]])
            assert seen == list(range(off[q] + 1)), (N, W, G, q)


def test_mask_no_cross_branch():
    N, W, G = 5, 4, 3
    mask = la.block_mask(N, W, G)
    M = mask.shape[0]
    kinds = [la.row_kind(r, N, W, G)[0] for r in range(M)]
    for q in range(M):
        for r in range(M):
            if {kinds[q], kinds[r]} == {"la", "ver"}:
                assert not mask[q, r]
            if kinds[q] == "ver" and kinds[r] == "ver":
                if la.row_kind(q, N, W, G)[1] != la.row_kind(r, N, W, G)[1]:
                    assert not mask[q, r]


def test_fig2b_example():
    fx = json.load(open(os.path.join(GOLD, "fig2b_mask.json")))
    N, W, G = fx["N"], fx["W"], fx["G"]
    q = fx["query"]
    M = la.n_rows(N, W, G)
    qrow = [r for r in range(M) if la.row_kind(r, N, W, G) == ("la", q["level"], q["column"])][0]
    assert la.row_offset(qrow, N, W, G) == q["position"]
    vis = {la.row_kind(r, N, W, G) for r in range(M) if la.block_visible(qrow, r, N, W, G)}
    assert vis == {tuple(v) for v in fx["visible"]}


def test_fig1_ngram_example():
    fx = json.load(open(os.path.join(GOLD, "fig1_ngram.json")))
    N, W, G = fx["N"], fx["W"], fx["G"]
    win = np.array([[100 + k for k in range(W)], [200 + k for k in range(W)]])  # levels 0, 1
    new = np.array([300 + k for k in range(W)])
    grams = la.harvest(win, new)
    # the n-gram of column 0 is (level-0 @ pos 1, level-1 @ pos 2, new @ pos 3)
    M = la.n_rows(N, W, G)
    pos_of = {la.row_kind(r, N, W, G): la.row_offset(r, N, W, G) for r in range(M)}
    want = []
    for e in fx["ngram"]:
        if e["level"] == "new":
            # the new token of column 0 is the output of its newest-level row
            assert pos_of[("la", N - 2, 0)] + 1 == e["position"]
            want.append(300)
        else:
            assert pos_of[("la", e["level"], 0)] == e["position"]
            want.append(100 * (e["level"] + 1))
    assert grams[0] == want
    assert len(grams) == W


# -- row equivalence ---------------------------------------------------------------

@pytest.mark.parametrize("N,W,G", [(3, 4, 4), (4, 3, 2), (2, 5, 3), (5, 2, 1)])
def test_row_equivalence(N, W, G):
    """Every block row's logits equal the last-position logits of a plain
    causal forward over prefix ++ that row's chain at positions 0..pos."""
    om = _model()
    rng = np.random.default_rng(N * 100 + W * 10 + G)
    prefix = rng.integers(0, 256, 9)
    P = len(prefix)
    M = la.n_rows(N, W, G)
    toks = rng.integers(0, 256, M)
    pos = np.array([P + la.row_offset(r, N, W, G) for r in range(M)])
    _, kv = om.forward(prefix, np.arange(P), causal_vis(0, P))
    vis = np.concatenate([np.ones((M, P), bool), la.block_mask(N, W, G)], axis=1)
    got, _ = om.forward(toks, pos, vis, past=kv)
    for q in range(M):
        seq = np.concatenate([prefix, toks[_chain(q, N, W, G)]])
        ref, _ = om.forward(seq, np.arange(len(seq)), causal_vis(0, len(seq)))
        np.testing.assert_allclose(got[q], ref[-1], atol=1e-9, rtol=0)


# -- exactness -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lookahead_equals_greedy(dtype):
    """Lookahead decoding reproduces greedy AR decoding exactly ([LD] §3.4
    'Greedy verification algorithm'; the abstract's 'exact')."""
    om = _model(dtype=dtype, seed=11)
    for seed in range(3):
        prompt = synth.prompt_motif(256, seed=seed)
        ar = la.greedy_ar(om, prompt, 24)
        for (N, W, G), ref in itertools.product([(2, 3, 3), (3, 4, 4), (4, 2, 5), (5, 3, 1)],
                                                [False, True]):
            r = la.lookahead(om, prompt, N, W, G, 24, synth.gen_window(N, W, 256, seed), prompt_ref=ref)
            assert r.tokens == ar.tokens, (seed, N, W, G, ref)
            assert all(1 <= e <= N for e in r.emitted)
            assert 1.0 <= r.S <= N


def test_G0_gives_one_token_per_step():
    om = _model()
    prompt = synth.prompt_motif(256)
    r = la.lookahead(om, prompt, 4, 3, 0, 20, synth.gen_window(4, 3, 256), prompt_ref=True)
    assert r.steps == 20 and r.S == 1.0 and set(r.accepted) == {0}


def test_correct_candidate_accepts_all():
    """Seed the pool with the AR continuation: every step accepts N-1 tokens
    and emits N (the bonus argmax P_N)."""
    om = _model(seed=5)
    prompt = synth.prompt_motif(256, seed=2)
    # W = 0: no harvests, so the seeded n-grams stay; the bucket is large
    # enough to hold every continuation of every key in the AR stream.
    N, W, G = 4, 0, 16
    ar = la.greedy_ar(om, prompt, 40)
    full = [int(prompt[-1])] + ar.tokens
    pool = la.NGramPool(G)
    for j in range(0, len(full) - N + 1):
        pool.insert(full[j], full[j + 1:j + N])
    assert pool.evictions == 0
    r = la.lookahead(om, prompt, N, W, G, 32, np.zeros(0, np.int64), pool=pool)
    assert r.tokens == ar.tokens[:32]
    assert r.accepted == [N - 1] * r.steps and r.emitted == [N] * r.steps


def test_wrong_candidates_accept_none():
    om = _model(seed=5)
    prompt = synth.prompt_motif(256, seed=2)
    N, W, G = 3, 2, 3
    ar = la.greedy_ar(om, prompt, 10)
    full = [int(prompt[-1])] + ar.tokens
    pool = la.NGramPool(G)
    for j in range(len(full) - 1):      # suffixes that are wrong in their first token
        pool.insert(full[j], [(full[j + 1] + 1) % 256, full[j + 1]])
    r = la.lookahead(om, prompt, N, 0, G, 10, np.zeros(0, np.int64), pool=pool)
    assert r.tokens == ar.tokens and r.accepted == [0] * 10


def test_budget_and_eos():
    om = _model(seed=5)
    prompt = synth.prompt_motif(256, seed=2)
    ar = la.greedy_ar(om, prompt, 30)
    r = la.lookahead(om, prompt, 4, 3, 3, 7, synth.gen_window(4, 3, 256), prompt_ref=True)
    assert r.tokens == ar.tokens[:7]
    eos = ar.tokens[5]
    stop = ar.tokens.index(eos)
    r = la.lookahead(om, prompt, 4, 3, 3, 30, synth.gen_window(4, 3, 256), prompt_ref=True, eos_id=eos)
    assert r.tokens == ar.tokens[:stop + 1]


# -- pool and window ------------------------------------------------------------

def test_pool_invariants_after_decode():
    om = _model(seed=2)
    prompt = synth.prompt_motif(256, seed=4)
    N, W, G = 4, 5, 3
    r = la.lookahead(om, prompt, N, W, G, 40, synth.gen_window(N, W, 256, 4), prompt_ref=True)
    pool = r.pool
    n_prompt_grams = len(prompt) - N + 1
    assert pool.inserts + pool.dup_skips == n_prompt_grams + W * r.steps
    for key, b in pool.buckets.items():
        assert len(b) <= G
        assert len(set(b)) == len(b)
        assert all(len(sfx) == N - 1 for sfx in b)
    assert pool.n_ngrams() == pool.inserts - pool.evictions


def test_pool_fifo_and_select():
    p = la.NGramPool(3)
    for s in [(1,), (2,), (1,), (3,), (4,)]:
        p.insert(7, s)
    assert p.buckets[7] == [(2,), (3,), (4,)]
    assert (p.inserts, p.dup_skips, p.evictions) == (4, 1, 1)
    assert p.select(7, 2) == [(3,), (4,)]
    assert p.select(8, 2) == []


def test_pool_lru_by_hand():
    """R21 worked by hand, cap 2: a, b, a again, c.  FIFO keeps [a, b] at the
    repeat and evicts a for c; recency moves a behind b and evicts b."""
    seq = [(1, 1), (2, 2), (1, 1), (3, 3)]
    fifo, lru = la.NGramPool(2), la.NGramPool(2, lru=True)
    for sfx in seq:
        fifo.insert(5, sfx)
        lru.insert(5, sfx)
    assert fifo.buckets[5] == [(2, 2), (3, 3)]
    assert lru.buckets[5] == [(1, 1), (3, 3)]
    for p in (fifo, lru):
        assert (p.inserts, p.dup_skips, p.evictions) == (3, 1, 1)
    # selection is the newest G in the bucket's order under both policies
    assert lru.select(5, 1) == [(3, 3)]
    lru.insert(5, (1, 1))                 # a again: now the most recent
    assert lru.buckets[5] == [(3, 3), (1, 1)] and lru.select(5, 1) == [(1, 1)]


def test_pool_lru_cap_one_and_no_repeat_equal_fifo():
    """Recency only reorders on a repeat, and a one-entry bucket has no order:
    with cap 1, or with no repeated suffix, both policies hold the same pool."""
    rng = np.random.default_rng(3)
    for cap, vocab in ((1, 3), (3, 1000)):
        fifo, lru = la.NGramPool(cap), la.NGramPool(cap, lru=True)
        for _ in range(400):
            key, sfx = int(rng.integers(4)), tuple(int(v) for v in rng.integers(vocab, size=2))
            fifo.insert(key, sfx)
            lru.insert(key, sfx)
        assert fifo.buckets == lru.buckets
        assert (fifo.inserts, fifo.dup_skips, fifo.evictions) == \
            (lru.inserts, lru.dup_skips, lru.evictions)


def test_pool_lru_is_recency_order():
    """Against a brute-force definition: after any insert sequence, an LRU
    bucket is the distinct suffixes ordered by their last appearance, the
    oldest dropped to the capacity, provided no suffix was ever evicted."""
    rng = np.random.default_rng(4)
    for trial in range(50):
        cap = int(rng.integers(2, 6))
        seq = [tuple(int(v) for v in rng.integers(cap, size=1)) for _ in range(30)]
        p = la.NGramPool(cap, lru=True)
        for sfx in seq:
            p.insert(0, sfx)
        last = {sfx: i for i, sfx in enumerate(seq)}
        assert p.buckets[0] == sorted(last, key=last.get)
        assert p.evictions == 0


def test_pool_context_selection_by_hand():
    """R22 worked by hand: bucket a(7) b(3) c(7) d(1), oldest first, G = 2."""
    p = la.NGramPool(8)
    for sfx, ctx in [((1,), 7), ((2,), 3), ((3,), 7), ((4,), 1)]:
        p.insert(9, sfx, ctx)
    assert p.select(9, 2) == [(3,), (4,)]                 # R6: the newest two
    assert p.select(9, 2, prev=7) == [(1,), (3,)]         # both context-7 entries
    assert p.select(9, 2, prev=3) == [(2,), (4,)]         # b, then the newest other (d)
    assert p.select(9, 3, prev=5) == [(2,), (3,), (4,)]   # no match: the newest three
    p.insert(9, (1,), 5)                                  # a repeat takes the new context
    assert p.context[(9, (1,))] == 5 and p.select(9, 1, prev=5) == [(1,)]
    p2 = la.NGramPool(2)
    for sfx in [(1,), (2,), (3,)]:
        p2.insert(0, sfx, 4)
    assert set(p2.context) == {(0, (2,)), (0, (3,))}      # an evicted entry's context goes too


def test_pool_context_selection_properties():
    """Without a matching context, or when the bucket fits in G, selection by
    context takes the same set as R6."""
    rng = np.random.default_rng(6)
    for _ in range(200):
        cap, G = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        p = la.NGramPool(cap)
        for _ in range(int(rng.integers(1, 20))):
            p.insert(0, (int(rng.integers(6)),), int(rng.integers(3)))
        b = p.buckets[0]
        assert p.select(0, G, prev=99) == p.select(0, G)
        if len(b) <= G:
            assert p.select(0, G, prev=int(rng.integers(3))) == b


def test_prompt_ngram_contexts():
    """Prompt n-grams (R11) carry the prompt token before them (none for the
    first); a repeated n-gram keeps its last occurrence's context."""
    s = synth.SHAPES["micro"]
    om = OracleModel(s, synth.gen_weights(s, 0))
    prompt = np.array([1, 2, 3, 4, 1, 2, 3, 5, 1, 2, 3, 4, 6], dtype=np.int64)
    N = 3
    r = la.lookahead(om, prompt, N, 0, 4, 1, np.zeros((N - 1, 0), dtype=np.int64),
                     prompt_ref=True, pool_cap=16, pool_context=True)
    want = {}
    for j in range(len(prompt) - N + 1):
        want[(int(prompt[j]), tuple(int(t) for t in prompt[j + 1:j + N]))] = \
            int(prompt[j - 1]) if j else -1
    got = {k: v for k, v in r.pool.context.items() if k in want}
    assert got == want


@pytest.mark.parametrize("N,W,G,cap,lru", [(4, 5, 5, 20, False), (4, 5, 5, 10, True),
                                           (3, 4, 2, 8, False), (5, 3, 3, 3, False)])
def test_lookahead_context_selection_is_exact(N, W, G, cap, lru):
    """Selection by context only changes which guesses are verified: the
    output equals greedy AR; with cap <= G it changes nothing at all."""
    s = synth.SHAPES["micro"]
    om = OracleModel(s, synth.gen_weights(s, 0))
    for seed in range(3):
        prompt = synth.prompt_motif(s.vocab, seed=seed)
        win = synth.gen_window(N, W, s.vocab, seed=2)
        ref = la.greedy_ar(om, prompt, 64).tokens
        r = la.lookahead(om, prompt, N, W, G, 64, win, prompt_ref=True, pool_cap=cap,
                         pool_lru=lru, pool_context=True)
        assert r.tokens == ref
        if cap <= G:
            f = la.lookahead(om, prompt, N, W, G, 64, win, prompt_ref=True, pool_cap=cap,
                             pool_lru=lru)
            assert f.accepted == r.accepted


@pytest.mark.parametrize("N,W,G,cap", [(3, 4, 4, None), (4, 5, 3, 2), (5, 3, 3, 1)])
def test_lookahead_lru_pool_is_exact(N, W, G, cap):
    """The pool's policy only changes which guesses are verified, never the
    output: lookahead with the recency pool equals greedy AR."""
    s = synth.SHAPES["micro"]
    om = OracleModel(s, synth.gen_weights(s, 0))
    prompt = np.array([1, 2, 3, 4, 1, 2, 3, 4, 5, 6, 7, 1, 2, 3], dtype=np.int64) % s.vocab
    win = synth.gen_window(N, W, s.vocab, seed=2)
    ref = la.greedy_ar(om, prompt, 40).tokens
    r = la.lookahead(om, prompt, N, W, G, 40, win, prompt_ref=True, pool_cap=cap, pool_lru=True)
    assert r.tokens == ref
    assert r.pool.lru and all(len(b) <= r.pool.cap for b in r.pool.buckets.values())
    if (N, W, G) == (3, 4, 4):
        # this run repeats suffixes in full buckets: the two policies diverge
        f = la.lookahead(om, prompt, N, W, G, 40, win, prompt_ref=True, pool_cap=cap)
        assert (f.pool.inserts, f.pool.evictions) != (r.pool.inserts, r.pool.evictions)


def test_slide():
    win = np.arange(12).reshape(3, 4)
    new = np.array([90, 91, 92, 93])
    out = la.slide(win, new)
    assert np.array_equal(out[:2], win[1:]) and np.array_equal(out[2], new)


# -- scaling law -------------------------------------------------------------------

def test_scaling_law_closed_forms():
    for a in [0.0, 0.1, 0.425, 0.9]:
        for g in [1, 2, 4, 7]:
            assert abs(expected_tokens(a, g, 1) - expected_tokens_single(a, g)) < 1e-12
    assert expected_tokens(0.0, 4, 15) == 1.0
    assert expected_tokens(1.0, 4, 15) == 5.0
    assert expected_tokens(0.425, 4, 15) > expected_tokens(0.425, 4, 2)
    assert abs(compression(0.425, 4, 15, 3.106) - (2.106 + expected_tokens(0.425, 4, 15)) / 3.106) < 1e-15
