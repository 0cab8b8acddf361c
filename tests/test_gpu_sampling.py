"""Sampling verification on the GPU ([LD] §3.4 "Sampling verification
(Algorithm 4)") through the C-ABI, against the oracle.

1. The device draws equal the oracle's Philox4x32-10 draws bit for bit.
2. 8-token fp32 model: the GPU's lookahead (graph and eager) and AR sampling
   emit the oracle's tokens, step by step, as long as every decision of the
   oracle's step is further than TOL (relative to the normaliser) from its
   threshold; the GPU's and the oracle's logits differ by ~1e-6.
3. The same model, 1500 seeds: the first two tokens of GPU lookahead
   sampling follow the exact distribution of autoregressive sampling
   (chi-square), with candidates accepted in most first steps.
4. tiny fp32 (vocab 256) sampling matches the oracle while decided; a bf16
   model at T = 1e-6 emits its greedy tokens.
5. Top-K / top-P cuts: the micro model's lookahead and AR sampling under
   cuts match the oracle while decided (the cuts' margins included), and
   follow the exact cut distribution over 1500 seeds; on a 4000-token bf16
   model top-K = 1, or a vanishing top-P share, reproduces the greedy stream
   exactly at T = 1.
"""
import collections

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from exact_decoding_amd import binding as B
from exact_decoding_amd.runtime import Model
from oracle import lookahead as la
from oracle import rng
from oracle.model import OracleModel
from sampling_util import MICRO_PROMPT, _gof, exact_ar_probs

pytestmark = pytest.mark.gpu

TOL = 1e-4


def test_device_draws_match_oracle():
    n = 4096
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    for seed, step in [(0, 0), (1234, 7), ((1 << 40) + 5, (1 << 33) + 3)]:
        print(f"draws seed={seed} step={step}", flush=True)
        B.la_philox_uniform(seed, step, n, out, None)
        torch.cuda.synchronize()
        ref = np.array([rng.uniform(seed, step, k) for k in range(n)], dtype=np.float32)
        assert np.array_equal(out.cpu().numpy(), ref)


@pytest.fixture(scope="module")
def micro():
    s = synth.SHAPES["micro"]
    w = synth.gen_weights(s, 0)
    return s, w, Model(s, w), OracleModel(s, w)


def _decided_prefix(ref, per_step, tokens):
    """Number of steps compared: the GPU's steps must equal the oracle's up
    to the first step with a decision closer than TOL to its threshold."""
    pos = 0
    for i, m in enumerate(ref.margins):
        if m < TOL or i >= len(per_step):
            return i
        k = ref.emitted[i]
        assert per_step[i] == k, f"step {i}"
        assert tokens[pos:pos + k] == ref.tokens[pos:pos + k], f"step {i}"
        pos += k
    return len(ref.margins)


@pytest.mark.parametrize("graph", [True, False])
@pytest.mark.parametrize("T", [0.7, 1.5])
def test_micro_lookahead_sampling_matches_oracle(micro, T, graph):
    s, w, gm, om = micro
    N, W, G, n_new = 3, 3, 3, 24
    compared = accepted = 0
    for seed in range(4):
        print(f"micro T={T} graph={graph} seed={seed}", flush=True)
        win = synth.gen_window(N, W, s.vocab, seed=100 + seed)
        ref = la.lookahead(om, MICRO_PROMPT, N, W, G, n_new, win, prompt_ref=True,
                           temperature=T, seed=seed)
        ses = gm.session(MICRO_PROMPT, N, W, G, n_new, window=win, prompt_ref=True,
                         temperature=T, seed=seed, graph=graph)
        toks = ses.decode()
        k = _decided_prefix(ref, ses.per_step, toks)
        if k == len(ref.margins):
            assert toks == ref.tokens
            st = ses.stats()
            assert [st["accept_hist"][j] for j in range(N)] == \
                [ref.accepted.count(j) for j in range(N)]
        compared += k
        accepted += sum(1 for a in ref.accepted[:k] if a > 0)
        ses.close()
    assert compared >= 24 and accepted >= 4


def test_micro_ar_sampling_matches_oracle(micro):
    s, w, gm, om = micro
    compared = 0
    for seed in range(4):
        print(f"micro AR seed={seed}", flush=True)
        ref = la.greedy_ar(om, MICRO_PROMPT, 16, temperature=1.2, seed=seed)
        ses = gm.session(MICRO_PROMPT, 3, 0, 0, 16, ar=True, temperature=1.2, seed=seed)
        toks = ses.decode()
        ses.close()
        for i, m in enumerate(ref.margins):
            if m < TOL:
                break
            assert toks[i] == ref.tokens[i], f"seed {seed} token {i}"
            compared += 1
    assert compared >= 32


def test_micro_lookahead_sampling_distribution(micro):
    s, w, gm, om = micro
    T, N, W, G = 1.5, 3, 3, 3
    probs = exact_ar_probs(om, MICRO_PROMPT, 2, T)
    n = 1500
    cnt = collections.Counter()
    accepted = 0
    print("micro distribution over 1500 seeds", flush=True)
    for seed in range(n):
        win = synth.gen_window(N, W, s.vocab, seed=100 + seed)
        ses = gm.session(MICRO_PROMPT, N, W, G, 2, window=win, prompt_ref=True,
                         temperature=T, seed=seed, graph=False)
        first = ses.step()
        accepted += len(first) > 1
        cnt[tuple(ses.decode())] += 1
        ses.close()
    assert accepted > n // 3
    assert _gof(cnt, probs, n) > 1e-3


def test_tiny_sampling_matches_oracle():
    s = synth.SHAPES["tiny"]
    w = synth.gen_weights(s, 0)
    gm, om = Model(s, w), OracleModel(s, w)
    prompt = synth.prompt_motif(s.vocab, seed=1)
    N, W, G = 3, 4, 4
    compared = 0
    for seed in range(2):
        print(f"tiny sampling seed={seed}", flush=True)
        win = synth.gen_window(N, W, s.vocab, seed=2)
        ref = la.lookahead(om, prompt, N, W, G, 16, win, prompt_ref=True, temperature=1.0,
                           seed=seed)
        ses = gm.session(prompt, N, W, G, 16, window=win, prompt_ref=True, temperature=1.0,
                         seed=seed)
        toks = ses.decode()
        compared += _decided_prefix(ref, ses.per_step, toks)
        ses.close()
    gm.close()
    assert compared >= 8


def test_bf16_near_zero_temperature_is_greedy():
    s = synth.SHAPES["small_bf16"]
    w = synth.gen_weights(s, 0)
    gm = Model(s, w)
    prompt = synth.prompt_zipf_spans(s.vocab, length=64, seed=1)
    N, W, G, n_new = 4, 6, 6, 32
    win = synth.gen_window(N, W, s.vocab, seed=2)
    print("small_bf16 T=1e-6", flush=True)
    ar = gm.session(prompt, N, W, G, n_new, ar=True)
    greedy = ar.decode()
    ar.close()
    ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True, temperature=1e-6,
                     seed=9)
    assert ses.decode() == greedy
    ses.close()
    gm.close()


def test_sampling_argument_checks(micro):
    s, w, gm, om = micro
    with pytest.raises(B.LaError):
        gm.session(MICRO_PROMPT, 3, 3, 3, 4, temperature=-1.0)
    with pytest.raises(B.LaError):
        gm.session(MICRO_PROMPT, 3, 3, 3, 4, temperature=float("inf"))


@pytest.mark.parametrize("N,W,G", [(2, 3, 3), (3, 0, 3), (3, 3, 0), (5, 2, 6)])
def test_micro_sampling_edge_configs_match_oracle(micro, N, W, G):
    """Degenerate and uneven configurations: one-token n-grams, no window,
    no candidates, more candidates than window columns."""
    s, w, gm, om = micro
    compared = 0
    for seed in range(3):
        print(f"micro sampling N={N} W={W} G={G} seed={seed}", flush=True)
        win = synth.gen_window(N, W, s.vocab, seed=200 + seed) if W else None
        ref = la.lookahead(om, MICRO_PROMPT, N, W, G, 12, win if W else np.zeros((N - 1, 0)),
                           prompt_ref=True, temperature=1.3, seed=seed)
        ses = gm.session(MICRO_PROMPT, N, W, G, 12, window=win, prompt_ref=True,
                         temperature=1.3, seed=seed)
        toks = ses.decode()
        compared += _decided_prefix(ref, ses.per_step, toks)
        ses.close()
    assert compared >= 6


def test_micro_sampling_budget_and_eos(micro):
    s, w, gm, om = micro
    N, W, G = 3, 3, 3
    win = synth.gen_window(N, W, s.vocab, seed=7)
    ref = la.lookahead(om, MICRO_PROMPT, N, W, G, 7, win, prompt_ref=True, temperature=1.0, seed=5)
    ses = gm.session(MICRO_PROMPT, N, W, G, 7, window=win, prompt_ref=True, temperature=1.0,
                     seed=5)
    toks = ses.decode()
    ses.close()
    assert len(toks) == 7
    if min(ref.margins) >= TOL:
        assert toks == ref.tokens
        # stop after the first emission of the stream's third token
        eos = ref.tokens[2]
        ref2 = la.lookahead(om, MICRO_PROMPT, N, W, G, 7, win, prompt_ref=True,
                            temperature=1.0, seed=5, eos_id=eos)
        ses = gm.session(MICRO_PROMPT, N, W, G, 7, window=win, prompt_ref=True,
                         temperature=1.0, seed=5, eos_id=eos)
        assert ses.decode() == ref2.tokens and ref2.tokens[-1] == eos
        ses.close()


@pytest.mark.parametrize("K,Pp", [(3, 0.0), (0, 0.8), (4, 0.9)])
def test_micro_restricted_sampling_matches_oracle(micro, K, Pp):
    s, w, gm, om = micro
    N, W, G, T = 3, 3, 3, 1.3
    compared = 0
    for seed in range(4):
        print(f"micro top_k={K} top_p={Pp} seed={seed}", flush=True)
        win = synth.gen_window(N, W, s.vocab, seed=300 + seed)
        ref = la.lookahead(om, MICRO_PROMPT, N, W, G, 20, win, prompt_ref=True, temperature=T,
                           seed=seed, top_k=K, top_p=Pp)
        ses = gm.session(MICRO_PROMPT, N, W, G, 20, window=win, prompt_ref=True,
                         temperature=T, seed=seed, top_k=K, top_p=Pp)
        compared += _decided_prefix(ref, ses.per_step, ses.decode())
        ses.close()
        ref = la.greedy_ar(om, MICRO_PROMPT, 12, temperature=T, seed=seed, top_k=K, top_p=Pp)
        ar = gm.session(MICRO_PROMPT, 3, 0, 0, 12, ar=True, temperature=T, seed=seed, top_k=K,
                        top_p=Pp)
        toks = ar.decode()
        ar.close()
        for i, m in enumerate(ref.margins):
            if m < TOL:
                break
            assert toks[i] == ref.tokens[i], f"AR seed {seed} token {i}"
            compared += 1
    assert compared >= 24


def test_micro_restricted_sampling_distribution(micro):
    s, w, gm, om = micro
    T, N, W, G, K, Pp = 1.5, 3, 3, 3, 4, 0.8
    probs = exact_ar_probs(om, MICRO_PROMPT, 2, T, K, Pp)
    n = 1500
    cnt = collections.Counter()
    print("micro top-K / top-P distribution over 1500 seeds", flush=True)
    for seed in range(n):
        win = synth.gen_window(N, W, s.vocab, seed=100 + seed)
        ses = gm.session(MICRO_PROMPT, N, W, G, 2, window=win, prompt_ref=True,
                         temperature=T, seed=seed, graph=False, top_k=K, top_p=Pp)
        cnt[tuple(ses.decode())] += 1
        ses.close()
    assert all(probs[key] > 0 for key in cnt)      # nothing outside the cut
    assert _gof(cnt, probs, n) > 1e-3


def test_bf16_top1_and_vanishing_top_p_are_greedy():
    s = synth.SHAPES["small_bf16"]
    w = synth.gen_weights(s, 0)
    gm = Model(s, w)
    prompt = synth.prompt_zipf_spans(s.vocab, length=64, seed=1)
    N, W, G, n_new = 4, 6, 6, 32
    win = synth.gen_window(N, W, s.vocab, seed=2)
    ar = gm.session(prompt, N, W, G, n_new, ar=True)
    greedy = ar.decode()
    ar.close()
    for K, Pp in [(1, 0.0), (0, 1e-7), (1, 0.5)]:
        print(f"small_bf16 T=1 top_k={K} top_p={Pp}", flush=True)
        ses = gm.session(prompt, N, W, G, n_new, window=win, prompt_ref=True, temperature=1.0,
                         seed=3, top_k=K, top_p=Pp)
        assert ses.decode() == greedy
        ses.close()
        ar = gm.session(prompt, N, W, G, n_new, ar=True, temperature=1.0, seed=4, top_k=K,
                        top_p=Pp)
        assert ar.decode() == greedy
        ar.close()
    gm.close()


@pytest.mark.parametrize("lru,ctx", [(True, False), (False, True), (True, True)])
def test_micro_sampling_pool_variants_match_oracle(micro, lru, ctx):
    """Sampling verification with the pool variants and a cap above G: the
    candidates the sampling kernel accepts set the token before cur for the
    next selection by context; while decided, the GPU matches the oracle's
    tokens and, for a fully decided run, its pool counters."""
    s, w, gm, om = micro
    N, W, G, n_new, T = 3, 3, 3, 24, 0.7
    compared = 0
    for seed in range(4):
        print(f"micro sampling pool lru={lru} context={ctx} seed={seed}", flush=True)
        win = synth.gen_window(N, W, s.vocab, seed=100 + seed)
        ref = la.lookahead(om, MICRO_PROMPT, N, W, G, n_new, win, prompt_ref=True,
                           temperature=T, seed=seed, pool_cap=2 * G, pool_lru=lru,
                           pool_context=ctx)
        ses = gm.session(MICRO_PROMPT, N, W, G, n_new, window=win, prompt_ref=True,
                         temperature=T, seed=seed, pool_cap=2 * G, pool_lru=lru,
                         pool_context=ctx)
        toks = ses.decode()
        k = _decided_prefix(ref, ses.per_step, toks)
        if k == len(ref.margins):
            assert toks == ref.tokens
            st = ses.stats()
            assert (st["inserts"], st["dup_skips"], st["evictions"]) == \
                (ref.pool.inserts, ref.pool.dup_skips, ref.pool.evictions)
        compared += k
        ses.close()
    assert compared >= 24


@pytest.mark.parametrize("graph", [True, False])
def test_micro_sampling_adaptive_g_matches_oracle(micro, graph):
    """Sampling verification in a LA_ADAPTIVE_G session: the candidate rows
    left out are padding, so the draws (one per candidate tried) and every
    decided token follow the oracle's fixed-G run; a fully decided run also
    has the oracle's accepted-length histogram and pool counters."""
    s, w, gm, om = micro
    N, W, G, n_new, T = 3, 3, 6, 24, 0.7
    compared = full = 0
    for seed in range(6):
        print(f"micro sampling adaptive G graph={graph} seed={seed}", flush=True)
        win = synth.gen_window(N, W, s.vocab, seed=100 + seed)
        ref = la.lookahead(om, MICRO_PROMPT, N, W, G, n_new, win, prompt_ref=True,
                           temperature=T, seed=seed)
        ses = gm.session(MICRO_PROMPT, N, W, G, n_new, window=win, prompt_ref=True,
                         temperature=T, seed=seed, graph=graph, adaptive_g=True)
        toks = ses.decode()
        k = _decided_prefix(ref, ses.per_step, toks)
        if k == len(ref.margins):
            full += 1
            assert toks == ref.tokens
            st = ses.stats()
            assert [st["accept_hist"][j] for j in range(N)] == \
                [ref.accepted.count(j) for j in range(N)]
            assert (st["inserts"], st["dup_skips"], st["evictions"]) == \
                (ref.pool.inserts, ref.pool.dup_skips, ref.pool.evictions)
            assert st["rows_total"] <= st["steps"] * (1 + (W + G) * (N - 1))
        compared += k
        ses.close()
    assert compared >= 24 and full >= 1
