"""End-to-end GPU parity of the lookahead step through the C-ABI.

1. tiny fp32 model: GPU lookahead tokens == oracle greedy AR tokens; the
   per-step accepted counts, S and pool counters equal the oracle's
   lookahead run; the block-row logits of a step match the oracle's within
   1e-4.
2. bf16 models (MHA and GQA, head_dim 128): GPU lookahead tokens are
   bit-identical to the GPU's own AR decode; GPU logits along the stream
   match the oracle's teacher-forced logits within 2e-2; every token whose
   oracle top-2 margin exceeds 2 * tol equals the oracle's argmax.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from exact_decoding_amd import binding as B
from exact_decoding_amd.runtime import Model
from oracle import lookahead as la
from oracle.model import OracleModel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    s = synth.SHAPES["tiny"]
    w = synth.gen_weights(s, 0)
    return s, w, Model(s, w), OracleModel(s, w)


@pytest.mark.parametrize("prompt_ref", [False, True])
@pytest.mark.parametrize("graph", [True, False])
def test_tiny_fp32_matches_oracle(tiny, prompt_ref, graph):
    s, w, gm, om = tiny
    N, W, G, n_new = 3, 4, 4, 32
    prompt = synth.prompt_motif(s.vocab, seed=1)
    win = synth.gen_window(N, W, s.vocab, seed=2)
    print(f"tiny fp32 prompt_ref={prompt_ref} graph={graph}", flush=True)
    ar = la.greedy_ar(om, prompt, n_new)
    ref = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=prompt_ref, keep_logits=True)
    assert ref.tokens == ar.tokens
    ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=prompt_ref, graph=graph,
                     debug_logits=True)
    first = ses.step()
    lg = ses.logits()
    np.testing.assert_allclose(lg, ref.step_logits[0], atol=1e-4, rtol=0)
    toks = first + [t for t in ses.decode()[len(first):]]
    assert ses.tokens == ar.tokens
    assert ses.per_step == ref.emitted
    st = ses.stats()
    assert st["steps"] == ref.steps and st["tokens"] == n_new
    assert [st["accept_hist"][j] for j in range(N)] == [ref.accepted.count(j) for j in range(N)]
    assert st["inserts"] == ref.pool.inserts and st["dup_skips"] == ref.pool.dup_skips
    assert st["evictions"] == ref.pool.evictions
    assert st["pool_ngrams"] == ref.pool.n_ngrams() and st["pool_keys_nonempty"] == ref.pool.n_keys()
    ses.close()
    del toks


def test_tiny_fp32_ar_session(tiny):
    s, w, gm, om = tiny
    prompt = synth.prompt_motif(s.vocab, seed=3)
    ar = la.greedy_ar(om, prompt, 20)
    ses = gm.session(prompt, 3, 4, 4, 20, ar=True)
    assert ses.rows == 1
    assert ses.decode() == ar.tokens
    assert ses.per_step == [1] * 20
    ses.close()


def test_tiny_budget_and_eos(tiny):
    s, w, gm, om = tiny
    prompt = synth.prompt_motif(s.vocab, seed=1)
    ar = la.greedy_ar(om, prompt, 30)
    win = synth.gen_window(4, 3, s.vocab, seed=2)
    ses = gm.session(prompt, 4, 3, 3, 7, window=win, prompt_ref=True)
    assert ses.decode() == ar.tokens[:7]
    ses.close()
    eos = ar.tokens[9]
    ses = gm.session(prompt, 4, 3, 3, 30, window=win, prompt_ref=True, eos_id=eos)
    assert ses.decode() == ar.tokens[:ar.tokens.index(eos) + 1]
    ses.close()


def _bf16_case(name, N, W, G, n_new, prompt):
    s = synth.SHAPES[name]
    w = synth.gen_weights(s, 0)
    gm = Model(s, w)
    win = synth.gen_window(N, W, s.vocab, seed=2)
    la_ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True)
    la_toks = la_ses.decode()
    st = la_ses.stats()
    la_ses.close()
    ar_ses = gm.session(prompt, N, W, G, n_new, ar=True, debug_logits=True)
    ar_logits = []
    while not ar_ses.done:
        tok = ar_ses.step()
        ar_logits.append(ar_ses.logits(1)[0])
        # the LM head's per-block argmax keys give the logits' argmax
        # (ties to the lowest id)
        row = ar_logits[-1]
        assert tok[0] == int(np.flatnonzero(row == row.max())[0])
    ar_toks = ar_ses.tokens
    ar_ses.close()
    return s, w, gm, la_toks, ar_toks, np.array(ar_logits), st


@pytest.mark.parametrize("name,N,W,G", [("small_bf16", 5, 7, 7), ("small_gqa_bf16", 4, 5, 3)])
def test_bf16_lookahead_bit_exact_and_oracle(name, N, W, G):
    print(f"bf16 decode {name} N={N} W={W} G={G}", flush=True)
    s = synth.SHAPES[name]
    prompt = synth.prompt_zipf_spans(s.vocab, length=64, seed=1)
    n_new = 48
    s, w, gm, la_toks, ar_toks, ar_logits, st = _bf16_case(name, N, W, G, n_new, prompt)
    assert la_toks == ar_toks, "lookahead stream differs from the same engine's AR stream"
    assert st["tokens"] == n_new and 1 <= n_new / st["steps"] <= N
    om = OracleModel(s, w)
    seq = np.concatenate([prompt, np.array(ar_toks[:-1], dtype=np.int64)])
    ref = la.score(om, seq)[len(prompt) - 1:]
    tol = 2e-2
    assert np.abs(ar_logits - ref).max() < tol
    srt = np.sort(ref, axis=1)
    margin = srt[:, -1] - srt[:, -2]
    top = np.argmax(ref, axis=1)
    sure = margin > 2 * tol
    assert np.array_equal(np.array(ar_toks)[sure], top[sure])
    gm.close()


def test_bf16_exact_whatever_the_context_capacity():
    """A row's attention arithmetic depends on its position only: a lookahead
    session and an AR session with very different max_ctx (so different
    sizes of every context-sized buffer) emit identical tokens, with
    positions crossing the 1024 boundary of the prefix chunk partition."""
    s = synth.SHAPES["small_bf16"]
    gm = Model(s, synth.gen_weights(s, 0))
    prompt = synth.prompt_zipf_spans(s.vocab, length=1000, seed=5)
    n_new = 48
    la_ses = gm.session(prompt, 5, 7, 7, n_new, window=synth.gen_window(5, 7, s.vocab, seed=2),
                        prompt_ref=True, max_ctx=len(prompt) + n_new + 20)
    la_toks = la_ses.decode()
    la_ses.close()
    ar_ses = gm.session(prompt, 5, 7, 7, n_new, ar=True, max_ctx=6000)
    ar_toks = ar_ses.decode()
    ar_ses.close()
    gm.close()
    assert len(la_toks) == n_new
    assert la_toks == ar_toks


@pytest.mark.parametrize("N,W,G,plen,prompt_ref", [
    (2, 1, 1, 16, True),     # shortest n-grams
    (2, 4, 0, 16, False),    # no verification branch
    (3, 0, 4, 16, True),     # no lookahead branch: candidates from the prompt only
    (16, 2, 2, 16, True),    # longest n-grams (LA_MAX_N)
    (4, 3, 3, 1, False),     # one-token prompt: no prefill forward
    (4, 3, 3, 2, True),      # prompt shorter than an n-gram: nothing to seed
    (5, 0, 0, 8, False),     # M = 1: the step degenerates to AR
])
def test_tiny_edge_configs_match_oracle(tiny, N, W, G, plen, prompt_ref):
    """Degenerate shapes of the method against the oracle: every token, the
    tokens of each step and every pool counter."""
    s, w, gm, om = tiny
    n_new = 24
    prompt = synth.prompt_motif(s.vocab, seed=1)[:plen]
    win = synth.gen_window(N, W, s.vocab, seed=2)
    print(f"tiny fp32 N={N} W={W} G={G} prompt={plen} ref={prompt_ref}", flush=True)
    ref = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=prompt_ref)
    assert ref.tokens == la.greedy_ar(om, prompt, n_new).tokens
    ses = gm.session(prompt, N, W, G, n_new, window=win if W else None, prompt_ref=prompt_ref)
    ses.decode()
    st = ses.stats()
    assert ses.tokens == ref.tokens
    assert ses.per_step == ref.emitted
    assert st["steps"] == ref.steps
    assert [st["accept_hist"][j] for j in range(N)] == [ref.accepted.count(j) for j in range(N)]
    assert st["inserts"] == ref.pool.inserts and st["dup_skips"] == ref.pool.dup_skips
    assert st["evictions"] == ref.pool.evictions
    assert st["pool_ngrams"] == ref.pool.n_ngrams() and st["pool_keys_nonempty"] == ref.pool.n_keys()
    ses.close()


@pytest.mark.parametrize("N,W,G", [(3, 70, 4), (4, 130, 6)])
def test_tiny_wide_window_pool_matches_oracle(tiny, N, W, G):
    """Windows wider than one wavefront (W > 64): every window column is
    harvested, whatever its place, so tokens, steps, the accepted-length
    histogram and every pool counter equal the oracle's; each step makes
    exactly W insert attempts (inserts + duplicates = prompt n-grams +
    W * steps)."""
    s, w, gm, om = tiny
    n_new = 24
    prompt = synth.prompt_motif(s.vocab, seed=1)
    win = synth.gen_window(N, W, s.vocab, seed=2)
    # columns past the first 64 whose key appears in none of the first 64:
    # their n-grams reach the pool only if those columns are harvested
    level0 = [int(t) for t in win[:W]]  # level-major: level 0 is the first W tokens
    wide_only = set(level0[64:]) - set(level0[:64])
    assert wide_only
    print(f"tiny fp32 wide window N={N} W={W} G={G}", flush=True)
    ref = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=True)
    assert ref.tokens == la.greedy_ar(om, prompt, n_new).tokens
    ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True)
    ses.decode()
    st = ses.stats()
    ses.close()
    assert ses.tokens == ref.tokens
    assert ses.per_step == ref.emitted
    assert st["steps"] == ref.steps
    assert [st["accept_hist"][j] for j in range(N)] == [ref.accepted.count(j) for j in range(N)]
    assert st["inserts"] == ref.pool.inserts and st["dup_skips"] == ref.pool.dup_skips
    assert st["evictions"] == ref.pool.evictions
    assert st["pool_ngrams"] == ref.pool.n_ngrams() and st["pool_keys_nonempty"] == ref.pool.n_keys()
    n_prompt_ngrams = max(0, len(prompt) - N + 1)
    assert st["inserts"] + st["dup_skips"] == n_prompt_ngrams + W * st["steps"]


def _adaptive_rows(ncand, N, W, G):
    """Rows an LA_ADAPTIVE_G session processes: the first step the full
    width; every later step the most candidate rows (at most G) that fit the
    16-row tiles the step's candidate count needs."""
    n1 = N - 1
    full = 1 + (W + G) * n1
    rows = full
    for g in ncand[1:]:
        tiles = -(-(1 + (W + g) * n1) // 16)
        w = min(G, (16 * tiles - 1) // n1 - W)
        rows += 1 + (W + max(w, g)) * n1
    return rows


@pytest.mark.parametrize("graph", [True, False])
@pytest.mark.parametrize("N,W,G,prompt_ref", [(3, 4, 4, True), (4, 3, 6, True), (5, 2, 7, False),
                                              (3, 70, 4, True), (4, 2, 20, True)])
def test_tiny_adaptive_g_matches_oracle(tiny, N, W, G, prompt_ref, graph):
    """LA_ADAPTIVE_G: candidate rows past the pool's candidates are left out,
    which changes nothing a step computes for the rows that remain, so every
    token, the tokens of each step, the accepted-length histogram and every
    pool counter equal the oracle's fixed-G run; the rows processed follow
    the oracle's candidate count of each step."""
    s, w, gm, om = tiny
    n_new = 32
    prompt = synth.prompt_motif(s.vocab, seed=1)
    win = synth.gen_window(N, W, s.vocab, seed=2)
    print(f"tiny fp32 adaptive G N={N} W={W} G={G} ref={prompt_ref} graph={graph}", flush=True)
    ref = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=prompt_ref)
    ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=prompt_ref, graph=graph,
                     adaptive_g=True)
    ses.decode()
    st = ses.stats()
    ses.close()
    assert ses.tokens == ref.tokens
    assert ses.per_step == ref.emitted
    assert st["steps"] == ref.steps
    assert [st["accept_hist"][j] for j in range(N)] == [ref.accepted.count(j) for j in range(N)]
    assert st["inserts"] == ref.pool.inserts and st["dup_skips"] == ref.pool.dup_skips
    assert st["evictions"] == ref.pool.evictions
    assert st["pool_ngrams"] == ref.pool.n_ngrams() and st["pool_keys_nonempty"] == ref.pool.n_keys()
    assert st["cand_total"] == sum(ref.ncand)
    assert st["rows_total"] == _adaptive_rows(ref.ncand, N, W, G)
    assert st["rows_total"] <= st["steps"] * (1 + (W + G) * (N - 1))


def test_context_full_is_reported(tiny):
    """A step that would write past max_ctx is refused with LA_ECTX before any
    device work; the tokens emitted until then are the AR stream's prefix."""
    s, w, gm, om = tiny
    N, W, G = 3, 4, 4
    prompt = synth.prompt_motif(s.vocab, seed=1)
    max_ctx = len(prompt) + 12
    ses = gm.session(prompt, N, W, G, 64, window=synth.gen_window(N, W, s.vocab, seed=2),
                     max_ctx=max_ctx)
    with pytest.raises(B.LaError) as ei:
        while not ses.done:
            ses.step()
    assert ei.value.code == B.LA_ECTX
    ar = la.greedy_ar(om, prompt, len(ses.tokens))
    assert len(ses.tokens) >= 1 and ses.tokens == ar.tokens
    ses.close()


def test_bf16_near_maximum_rows_bit_exact():
    """M = 1 + (66 + 66) * 15 = 1981 rows (the limit is 2048): sixteen 128-row
    GEMM tiles, chains up to N + W - 1 = 81 keys long, and still the AR stream
    bit for bit."""
    s = synth.SHAPES["small_bf16"]
    gm = Model(s, synth.gen_weights(s, 0))
    N, W, G, n_new = 16, 66, 66, 24
    prompt = synth.prompt_zipf_spans(s.vocab, length=64, seed=1)
    la_ses = gm.session(prompt, N, W, G, n_new, window=synth.gen_window(N, W, s.vocab, seed=2),
                        prompt_ref=True)
    assert la_ses.rows == 1981
    la_toks = la_ses.decode()
    st = la_ses.stats()
    la_ses.close()
    # pool invariants at 66 columns: W insert attempts per step after the
    # prompt's n-grams; the pool holds what was inserted less what was evicted
    n_prompt_ngrams = max(0, len(prompt) - N + 1)
    assert st["inserts"] + st["dup_skips"] == n_prompt_ngrams + W * st["steps"]
    assert st["pool_ngrams"] == st["inserts"] - st["evictions"]
    assert 1 <= st["pool_keys_nonempty"] <= st["pool_ngrams"]
    ar_ses = gm.session(prompt, N, W, G, n_new, ar=True)
    ar_toks = ar_ses.decode()
    ar_ses.close()
    gm.close()
    assert la_toks == ar_toks


def test_vocab_not_multiple_of_four_matches_oracle():
    """A vocabulary of 253 ids takes the argmax's scalar path."""
    import dataclasses
    s = dataclasses.replace(synth.SHAPES["tiny"], name="tiny_v253", vocab=253)
    w = synth.gen_weights(s, 0)
    gm, om = Model(s, w), OracleModel(s, w)
    prompt = synth.prompt_motif(s.vocab, seed=4)
    N, W, G = 3, 4, 4
    win = synth.gen_window(N, W, s.vocab, seed=5)
    print("tiny vocab 253", flush=True)
    ar = la.greedy_ar(om, prompt, 16)
    ses = gm.session(prompt, N, W, G, 16, window=win, prompt_ref=True)
    assert ses.decode() == ar.tokens
    ses.close()
    gm.close()


@pytest.fixture(scope="module")
def micro():
    s = synth.SHAPES["micro"]
    w = synth.gen_weights(s, 0)
    return s, w, Model(s, w), OracleModel(s, w)


MICRO_PROMPT = [1, 2, 3, 4, 1, 2, 3, 4, 5, 6, 7, 1, 2, 3]


@pytest.mark.parametrize("N,W,G,cap,graph", [(3, 4, 4, 0, True), (3, 4, 4, 0, False),
                                             (4, 5, 3, 2, True), (5, 3, 3, 1, True)])
def test_micro_lru_pool_matches_oracle(micro, N, W, G, cap, graph):
    """Recency eviction (LA_POOL_LRU): on the 8-token fp32 model, whose
    greedy decisions all have top-2 margins above 1e-2 in every block row,
    the GPU emits the greedy AR tokens in the oracle's steps, with the
    oracle's accepted-length histogram and pool counters under the same
    policy.  At (3, 4, 4) the two policies' counters differ on the GPU as
    they do in the oracle, so the recency path is exercised."""
    s, w, gm, om = micro
    n_new = 40
    prompt = np.array(MICRO_PROMPT, dtype=np.int64) % s.vocab
    win = synth.gen_window(N, W, s.vocab, seed=2)
    print(f"micro lru N={N} W={W} G={G} cap={cap} graph={graph}", flush=True)
    ar = la.greedy_ar(om, prompt, n_new)
    stats = {}
    for lru in (True, False):
        ref = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=True,
                           pool_cap=cap or None, pool_lru=lru)
        assert ref.tokens == ar.tokens
        ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True, graph=graph,
                         pool_cap=cap, pool_lru=lru)
        toks = ses.decode()
        st = ses.stats()
        ses.close()
        assert toks == ar.tokens
        assert st["steps"] == ref.steps
        assert [st["accept_hist"][j] for j in range(N)] == [ref.accepted.count(j) for j in range(N)]
        got = (st["inserts"], st["dup_skips"], st["evictions"], st["pool_ngrams"],
               st["pool_keys_nonempty"])
        assert got == (ref.pool.inserts, ref.pool.dup_skips, ref.pool.evictions,
                       ref.pool.n_ngrams(), ref.pool.n_keys()), (lru, got)
        stats[lru] = got
    if (N, W, G) == (3, 4, 4):
        assert stats[True] != stats[False]


@pytest.mark.parametrize("N,W,G,cap,lru", [(4, 5, 5, 20, False), (4, 5, 5, 10, True),
                                           (3, 4, 2, 8, False)])
def test_micro_context_selection_matches_oracle(micro, N, W, G, cap, lru):
    """Selection by context (LA_POOL_CONTEXT) with a pool cap above G, where
    it changes which candidates are verified: for two motif prompts the GPU
    emits the greedy AR tokens in the oracle's steps, with its accepted-length
    histogram and pool counters.  The oracle's block rows of these runs have
    top-2 margins above 1e-3 (checked here), far above the fp32 error.  At
    (4, 5, 5, cap 20) selection by context takes fewer steps than the newest-G
    rule for prompt 0, so the selection path is exercised."""
    s, w, gm, om = micro
    n_new = 64
    win = synth.gen_window(N, W, s.vocab, seed=2)
    for seed in (0, 2):
        prompt = synth.prompt_motif(s.vocab, seed=seed)
        print(f"micro context N={N} W={W} G={G} cap={cap} lru={lru} prompt={seed}", flush=True)
        ar = la.greedy_ar(om, prompt, n_new)
        ref = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=True, pool_cap=cap,
                           pool_lru=lru, pool_context=True, keep_logits=True)
        margin = min(float((np.sort(l, axis=1)[:, -1] - np.sort(l, axis=1)[:, -2]).min())
                     for l in ref.step_logits)
        assert margin > 1e-3
        assert ref.tokens == ar.tokens
        ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True, pool_cap=cap,
                         pool_lru=lru, pool_context=True)
        toks = ses.decode()
        st = ses.stats()
        ses.close()
        assert toks == ar.tokens
        assert st["steps"] == ref.steps
        assert [st["accept_hist"][j] for j in range(N)] == [ref.accepted.count(j) for j in range(N)]
        assert (st["inserts"], st["dup_skips"], st["evictions"], st["pool_ngrams"]) == \
            (ref.pool.inserts, ref.pool.dup_skips, ref.pool.evictions, ref.pool.n_ngrams())
        if (N, W, G, cap, lru, seed) == (4, 5, 5, 20, False, 0):
            plain = la.lookahead(om, prompt, N, W, G, n_new, win, prompt_ref=True, pool_cap=cap)
            assert plain.steps != ref.steps


@pytest.mark.parametrize("graph", [True, False])
def test_bf16_pool_variants_bit_exact(graph):
    """The pool variants change only which guesses are verified: with a cap
    above G, recency eviction and selection by context, the bf16 model's
    lookahead stream still equals the same engine's AR stream bit for bit."""
    s = synth.SHAPES["small_bf16"]
    gm = Model(s, synth.gen_weights(s, 0))
    prompt = synth.prompt_zipf_spans(s.vocab, length=64, seed=1)
    N, W, G, n_new = 5, 7, 7, 48
    win = synth.gen_window(N, W, s.vocab, seed=2)
    ar = gm.session(prompt, N, W, G, n_new, ar=True, graph=graph)
    ar_toks = ar.decode()
    ar.close()
    for lru, ctx in ((True, False), (False, True), (True, True)):
        print(f"bf16 pool variant lru={lru} context={ctx} graph={graph}", flush=True)
        ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True, graph=graph,
                         pool_cap=3 * G, pool_lru=lru, pool_context=ctx)
        assert ses.decode() == ar_toks
        ses.close()
    gm.close()


@pytest.mark.parametrize("name,N,W,G", [("small_bf16", 5, 7, 7), ("small_gqa_bf16", 4, 5, 9)])
def test_bf16_adaptive_g_bit_exact(name, N, W, G):
    """bf16 models: the LA_ADAPTIVE_G stream is the same engine's AR stream
    bit for bit, and the same as the fixed-G lookahead stream, with no more
    rows processed."""
    s = synth.SHAPES[name]
    gm = Model(s, synth.gen_weights(s, 0))
    prompt = synth.prompt_zipf_spans(s.vocab, length=64, seed=1)
    win = synth.gen_window(N, W, s.vocab, seed=2)
    n_new = 48
    out = {}
    for adaptive in (False, True):
        ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True, adaptive_g=adaptive)
        out[adaptive] = (ses.decode(), ses.stats())
        ses.close()
    ar = gm.session(prompt, N, W, G, n_new, ar=True)
    ar_toks = ar.decode()
    ar.close()
    gm.close()
    assert out[True][0] == ar_toks == out[False][0]
    fixed, adapt = out[False][1], out[True][1]
    for k in ("steps", "tokens", "inserts", "dup_skips", "evictions", "cand_total"):
        assert fixed[k] == adapt[k], k
    assert adapt["rows_total"] <= fixed["rows_total"] == fixed["steps"] * (1 + (W + G) * (N - 1))


def test_bf16_argmax_ties_and_logits_on_demand():
    """A zero LM head makes every logit 0: the argmax over the LM head's
    per-block keys must take the lowest id, 0, at every row, so lookahead
    and AR both emit only 0s.  A bf16 session keeps no logits unless asked
    (LA_DEBUG_LOGITS); one that is asked returns them."""
    s = synth.SHAPES["small_bf16"]
    w = synth.gen_weights(s, 0)
    w[-1] = np.zeros_like(w[-1])
    gm = Model(s, w)
    prompt = synth.prompt_zipf_spans(s.vocab, length=32, seed=3)
    N, W, G = 4, 5, 5
    la_ses = gm.session(prompt, N, W, G, 20, window=synth.gen_window(N, W, s.vocab, seed=2),
                        prompt_ref=True)
    assert la_ses.decode() == [0] * 20
    with pytest.raises(B.LaError) as ei:
        la_ses.logits()
    assert ei.value.code == B.LA_ESTATE
    la_ses.close()
    ar = gm.session(prompt, N, W, G, 8, ar=True, debug_logits=True)
    assert ar.step() == [0]
    assert not ar.logits(1).any()
    assert ar.decode() == [0] * 8
    ar.close()
    gm.close()


def test_bf16_step_profile_counts_and_tokens():
    """la_step_profile runs the step eagerly with every launch timed on the
    device: its tokens equal la_step's, each launch class is counted once
    per launch (four projections, one attention and four epilogues per
    layer; embed and first norm; LM head; argmax; gather, verify, commit),
    every class has a positive time, and the classes together take less
    than the call's wall time."""
    import time
    s = synth.SHAPES["small_bf16"]
    gm = Model(s, synth.gen_weights(s, 0))
    prompt = synth.prompt_zipf_spans(s.vocab, length=48, seed=4)
    N, W, G = 5, 7, 7
    win = synth.gen_window(N, W, s.vocab, seed=2)
    ref = gm.session(prompt, N, W, G, 24, window=win, prompt_ref=True)
    ref_toks = ref.decode()
    ref.close()
    ses = gm.session(prompt, N, W, G, 24, window=win, prompt_ref=True)
    L = s.n_layers
    want = {"gemm": 4 * L, "lm_head": 1, "attention": L, "norm": 2, "epilogue": 4 * L,
            "argmax": 1, "bookkeeping": 3}
    while not ses.done:
        t0 = time.perf_counter()
        _, prof = ses.step_profile()
        wall_ms = (time.perf_counter() - t0) * 1e3
        for k, n in want.items():
            assert prof[k]["launches"] == n, (k, prof[k])
            assert prof[k]["ms"] > 0, (k, prof[k])
        assert sum(v["ms"] for v in prof.values()) < wall_ms
    assert ses.tokens == ref_toks
    ses.close()
    gm.close()
