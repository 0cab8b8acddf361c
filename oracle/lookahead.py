"""Oracle lookahead decoding and greedy AR decoding -- test infrastructure only.

Follows [LD] §3.2 "Big-Picture Architecture" and §3.4 ("The Lookahead
Branch", "N-gram harvesting and pool update", "Sliding window update",
"N-gram selection from the pool", "Greedy verification algorithm
(Algorithm 3)", "The custom attention mask (Figure 2)", "N-gram pool
update"), plus the prompt-as-reference variant ([LD] §5 Table 3 ⑨, [LDs]).

Notation: N = n-gram length, W = window width, G = max candidates.
The window has N-1 levels (level 0 = oldest Jacobi step) of W tokens.

Readings where the pages are silent or garbled:

R1  Row layout of one step (M = 1 + W(N-1) + G(N-1) rows):
      row 0                          = cur (last emitted token), position P
      lookahead row 1 + l*W + k      = win[l][k], position P + 1 + l + k
      verification row 1 + W(N-1) + g(N-1) + (i-1)
                                     = cand[g][i-1], position P + i
    P = number of committed tokens (prompt minus its last token, plus all
    emitted tokens before cur).
R2  Visibility inside the block (the Fig. 2(b) mask).  Committed tokens are
    visible to all rows; row 0 to all rows; a lookahead row (l, k) sees the
    lookahead row (l', k') iff (l' = 0 and k' < k) or (k' = k and l' <= l);
    a verification row (g, i) sees (g', i') iff g' = g and i' <= i; no
    lookahead <-> verification visibility; every row sees itself.
R3  Window init: supplied (seeded uniform over the vocabulary); all N-1
    levels are full from the first step, and n-grams are harvested from the
    first step on.
R4  The window slides one level per step whatever is accepted; its
    positions are re-based on the new P.
R5  Pool: per first token, a FIFO of at most pool_cap (default G) distinct
    suffixes; an identical suffix is skipped; at capacity the oldest is
    evicted.
R6  Selection: the bucket of cur, oldest first; if it holds more than G,
    the newest G.
R7  The candidates of step t come from the pool after step t-1's insert;
    step t's n-grams are inserted after its forward pass.
R8  Unused candidate slots hold token 0; their rows are computed and
    ignored.
R9  Argmax ties go to the lowest token id.
R10 Budget: the emitted tokens of the last step are truncated to max_new;
    eos_id < 0 means no EOS, else decoding stops after emitting it.
R11 Prompt as reference: every prompt n-gram prompt[j .. j+N-1],
    j = 0 .. n-N, is inserted in increasing j before the first step.
R12 Only lookahead harvests and the prompt feed the pool.
R21 Pool eviction by recency (the pages leave the pool's size cap and its
    eviction policy unablated and name LRU and FIFO as the policies to
    compare, [LD] "What is not ablated" and "Memory-efficient n-gram pool
    management"): an n-gram is "used" when it is generated again (a
    duplicate insert from the lookahead branch or the prompt); it then
    becomes the bucket's most recent entry, and a full bucket evicts its
    least recent entry. Acceptance by verification is not counted as a use.
    FIFO (R5, the default) leaves a duplicate where it is. Selection (R6)
    takes the newest G in the bucket's order under either policy.
R22 Selection by a longer match (the pages contrast matching only the first
    token with matching longer prefixes, and note that the prompt-lookup
    baseline tries more than one starting token, [LD] Table 3 and "What is not
    ablated"): every entry also keeps its context, the token just before the
    n-gram's first token where it was generated (a window column's context
    is the level-0 token of the column to its left, or the step's current
    token for the first column; a prompt n-gram's is the prompt token before
    it, none for the first). A repeat takes the new context. With selection
    by context, the G taken are the newest entries whose context equals the
    token before cur, then the newest of the rest; they are presented in the
    bucket's order, oldest first, as in R6.
R18 Sampling verification (Algorithm 4, [LD] §3.4 "Sampling verification"):
    at position i the row predicting P+i (row 0, then the row of the
    accepted prefix) gives weights e_v = exp((l_v - max l) / T); the
    surviving candidates' i-th tokens are tried in candidate order, a token
    already rejected at this position being skipped without a draw; token c
    is accepted when r * (Z - sum of rejected weights) <= e_c for the next
    draw r in (0, 1]; when all are rejected, the first token (index order,
    rejected ones left out) whose running weight sum reaches u * (sum of the
    remaining weights) is drawn and ends the step; after N-1 accepted tokens
    one token is drawn that way from the last row.  Draw k of step s comes
    from rng.uniform(seed, s, k), k counting the draws of the step in the
    order they are used.  The lookahead branch stays greedy (argmax).
R20 Top-K / top-P with temperature (the pages' examples of a target
    sampling distribution, [LD] §3.4 "Sampling verification"): tokens are
    ranked by logit, higher first, ties to the lower id; top-K keeps the
    first K (K = 0: all); top-P then keeps the shortest leading run of the
    kept tokens whose weight sum reaches p times their total (p = 1, or
    0, keeps all).
    The other tokens get weight 0, and Algorithm 4 runs on what is left.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import rng
from .model import OracleModel, argmax_lowest, causal_vis


# ---------------------------------------------------------------------------
# row layout and mask (R1, R2)
# ---------------------------------------------------------------------------

def n_rows(N: int, W: int, G: int) -> int:
    return 1 + (W + G) * (N - 1)


def row_kind(r: int, N: int, W: int, G: int):
    """('cur',) | ('la', l, k) | ('ver', g, i) for block row r (R1)."""
    if r == 0:
        return ("cur",)
    r -= 1
    if r < W * (N - 1):
        return ("la", r // W, r % W)
    r -= W * (N - 1)
    return ("ver", r // (N - 1), r % (N - 1) + 1)


def row_offset(r: int, N: int, W: int, G: int) -> int:
    """Position of row r relative to P (R1)."""
    kd = row_kind(r, N, W, G)
    if kd[0] == "cur":
        return 0
    if kd[0] == "la":
        return 1 + kd[1] + kd[2]
    return kd[2]


def block_visible(q: int, r: int, N: int, W: int, G: int) -> bool:
    """Whether block row q attends to block row r: the set rules of R2,
    written case by case from [LD] §3.4 "The custom attention mask"."""
    a = row_kind(q, N, W, G)
    b = row_kind(r, N, W, G)
    if b[0] == "cur":
        return True                  # the current token is visible to all
    if a[0] == "cur":
        return False                 # row 0 sees only itself (and the prefix)
    if a[0] != b[0]:
        return False                 # no cross-branch visibility
    if a[0] == "la":
        (_, l, k), (_, l2, k2) = a, b
        return (l2 == 0 and k2 < k) or (k2 == k and l2 <= l)
    (_, g, i), (_, g2, i2) = a, b
    return g2 == g and i2 <= i


def block_mask(N: int, W: int, G: int) -> np.ndarray:
    M = n_rows(N, W, G)
    return np.array([[block_visible(q, r, N, W, G) for r in range(M)] for q in range(M)],
                    dtype=bool)


# ---------------------------------------------------------------------------
# n-gram pool (R5, R6)
# ---------------------------------------------------------------------------

class NGramPool:
    """Key = first token of the n-gram, value = list of suffixes ([LD] §3.4
    "N-gram pool update"), capacity `cap` per key, oldest first: FIFO (R5)
    or, with lru, ordered by the last time each suffix was generated (R21)."""

    def __init__(self, cap: int, lru: bool = False):
        self.cap = cap
        self.lru = lru
        self.buckets: dict[int, list[tuple[int, ...]]] = {}
        self.context: dict[tuple[int, tuple[int, ...]], int] = {}   # R22
        self.inserts = 0
        self.dup_skips = 0
        self.evictions = 0

    def insert(self, key: int, suffix, context: int = -1) -> None:
        key = int(key)
        suffix = tuple(int(t) for t in suffix)
        b = self.buckets.setdefault(key, [])
        if suffix in b:
            self.dup_skips += 1
            if self.lru:                                     # R21
                b.remove(suffix)
                b.append(suffix)
            self.context[(key, suffix)] = int(context)       # R22
            return
        self.inserts += 1
        if len(b) == self.cap:
            del self.context[(key, b.pop(0))]
            self.evictions += 1
        b.append(suffix)
        self.context[(key, suffix)] = int(context)

    def select(self, key: int, G: int, prev: int | None = None) -> list[tuple[int, ...]]:
        """Up to G suffixes whose n-gram starts with `key`: the newest (R6),
        or, given the token `prev` before key, the newest whose context is
        prev and then the newest of the rest (R22); oldest first."""
        b = self.buckets.get(int(key), [])
        if G <= 0:
            return []
        if prev is None:
            return list(b[-G:])
        newest_first = list(range(len(b) - 1, -1, -1))
        match = [i for i in newest_first if self.context[(int(key), b[i])] == prev]
        rest = [i for i in newest_first if self.context[(int(key), b[i])] != prev]
        return [b[i] for i in sorted((match + rest)[:G])]

    def n_ngrams(self) -> int:
        return sum(len(b) for b in self.buckets.values())

    def n_keys(self) -> int:
        return sum(1 for b in self.buckets.values() if b)


# ---------------------------------------------------------------------------
# window (R3, R4)
# ---------------------------------------------------------------------------

def harvest(win: np.ndarray, new: np.ndarray) -> list[list[int]]:
    """One n-gram per column k = 0 .. W-1 ([LD] §3.4 "N-gram harvesting and
    pool update", Fig. 1): the column's tokens from the oldest level to the
    newest, then the column's new token.  Under R1 these sit at consecutive
    positions and come from consecutive Jacobi steps."""
    L, W = win.shape
    return [[int(win[l, k]) for l in range(L)] + [int(new[k])] for k in range(W)]


def slide(win: np.ndarray, new: np.ndarray) -> np.ndarray:
    """Drop the oldest level; every level moves one step older; the new
    tokens become the newest level ([LD] §3.4 "Sliding window update")."""
    if win.shape[0] == 0 or win.shape[1] == 0:
        return win
    return np.concatenate([win[1:], np.asarray(new, dtype=win.dtype)[None, :]], axis=0)


# ---------------------------------------------------------------------------
# sampling verification (R18)
# ---------------------------------------------------------------------------

def row_weights(logits_row: np.ndarray, T: float) -> np.ndarray:
    """e_v = exp((l_v - max l) / T): softmax(l / T) up to its normaliser."""
    l = np.asarray(logits_row, dtype=np.float64)
    return np.exp((l - l.max()) / T)


def restricted_weights(logits_row: np.ndarray, T: float, top_k: int = 0,
                       top_p: float = 1.0) -> tuple[np.ndarray, float]:
    """row_weights with the top-K / top-P restriction of R20.  Returns (e,
    margin): margin is the smallest distance of a cut from deciding the
    other way, the logit gap at the top-K cut and, for top-P, the distance
    of p times the total from the nearest running sum, relative to the
    total (inf when nothing is cut)."""
    l = np.asarray(logits_row, dtype=np.float64)
    e = row_weights(l, T)
    V = len(l)
    order = np.lexsort((np.arange(V), -l))       # logit descending, then id ascending
    margin = np.inf
    n = V if top_k <= 0 else min(int(top_k), V)
    if n < V:
        margin = float(l[order[n - 1]] - l[order[n]])
    if 0.0 < top_p < 1.0:
        cs = np.cumsum(e[order[:n]])
        target = top_p * cs[-1]
        cut = int(np.searchsorted(cs, target, side="left"))
        cut = min(cut, n - 1)
        lo = cs[cut - 1] if cut > 0 else 0.0
        margin = min(margin, float(min(target - lo, cs[cut] - target) / cs[-1]))
        n = cut + 1
    out = np.zeros_like(e)
    out[order[:n]] = e[order[:n]]
    return out, margin


def draw_from(e: np.ndarray, removed: set, u: float) -> tuple[int, float]:
    """The first token v, in index order and leaving out `removed`, whose
    running weight sum reaches u * (sum of the remaining weights); returns
    (v, margin), margin = distance of that threshold from the nearest running
    sum, relative to the remaining sum."""
    w = e.copy()
    if removed:
        w[list(removed)] = 0.0
    cum = np.cumsum(w)
    total = cum[-1]
    target = u * total
    v = int(np.searchsorted(cum, target, side="left"))
    if v >= len(w):                      # rounding: the last positive weight
        v = int(np.nonzero(w > 0)[0][-1])
    lo = cum[v - 1] if v > 0 else 0.0
    margin = min(target - lo, cum[v] - target) / total
    return v, float(margin)


def sample_verify(logits: np.ndarray, cands, N: int, base: int, T: float, seed: int,
                  step: int, top_k: int = 0, top_p: float = 1.0):
    """Algorithm 4 over one step's block-row logits (R18).  Returns (emit,
    acc, g0, margin): the emitted tokens (acc accepted candidate tokens, then
    the drawn one), the candidate whose rows are committed, and the smallest
    decision margin of the step (relative to the normaliser in play)."""
    k = 0
    survivors = list(range(len(cands)))
    row = 0
    emit: list[int] = []
    margin = np.inf
    for i in range(1, N + 1):
        e, mr = restricted_weights(logits[row], T, top_k, top_p)
        margin = min(margin, mr)
        z = float(e.sum())
        removed: set = set()
        zr = z
        pick = None
        if i <= N - 1:
            for g in survivors:
                c = int(cands[g][i - 1])
                if c in removed:
                    continue
                r = rng.uniform(seed, step, k)
                k += 1
                margin = min(margin, abs(r * zr - e[c]) / z)
                if r * zr <= e[c]:
                    pick = c
                    break
                removed.add(c)
                zr -= e[c]
        if pick is None:
            u = rng.uniform(seed, step, k)
            k += 1
            t, m = draw_from(e, removed, u)
            margin = min(margin, m)
            emit.append(t)
            break
        emit.append(pick)
        survivors = [g for g in survivors if int(cands[g][i - 1]) == pick]
        row = base + survivors[0] * (N - 1) + (i - 1)
    acc = len(emit) - 1
    g0 = survivors[0] if acc > 0 else 0
    return emit, acc, g0, margin


# ---------------------------------------------------------------------------
# decoding
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeResult:
    tokens: list[int]
    steps: int
    accepted: list[int]                 # accepted candidate tokens per step
    emitted: list[int]                  # emitted tokens per step
    step_logits: list[np.ndarray]       # per step: block-row logits (if kept)
    step_rows: list[np.ndarray]         # per step: block-row tokens
    pool: NGramPool | None = None
    margins: list[float] = dataclasses.field(default_factory=list)  # sampling: per step
    ncand: list[int] = dataclasses.field(default_factory=list)      # candidates per step

    @property
    def S(self) -> float:
        """Step compression ratio: generated tokens / steps ([LD] §3.4
        "Scaling Law", step compression ratio)."""
        return len(self.tokens) / max(self.steps, 1)


def prefill(model: OracleModel, prompt):
    """Committed cache of prompt[:-1]; cur = prompt[-1]."""
    prompt = np.asarray(prompt, dtype=np.int64)
    n = len(prompt)
    if n < 1:
        raise ValueError("empty prompt")
    if n == 1:
        s = model.s
        empty = np.zeros((0, s.n_kv_heads, s.head_dim))
        return [(empty, empty) for _ in range(s.n_layers)], int(prompt[0])
    _, kv = model.forward(prompt[:-1], np.arange(n - 1), causal_vis(0, n - 1))
    return kv, int(prompt[-1])


def _append(cache, new_kv, rows=None):
    out = []
    for (K, V), (k, v) in zip(cache, new_kv):
        if rows is not None:
            k, v = k[rows], v[rows]
        out.append((np.concatenate([K, k]), np.concatenate([V, v])))
    return out


def greedy_ar(model: OracleModel, prompt, max_new: int, eos_id: int = -1,
              keep_logits: bool = False, temperature: float = 0.0,
              seed: int = 0, top_k: int = 0, top_p: float = 1.0) -> DecodeResult:
    """Plain autoregressive decoding ([LD] §3.4 "Mathematical
    Reformulation", the autoregressive system): y_{j+1} = argmax of the
    logits at the last position given prompt and y_1..y_j, or, with a
    temperature, a draw from softmax(logits / T) restricted by top-K / top-P
    (draw 0 of step j, R18, R20)."""
    cache, cur = prefill(model, prompt)
    P = cache[0][0].shape[0]
    out: list[int] = []
    logits_kept = []
    margins = []
    while len(out) < max_new:
        logits, kv = model.forward([cur], [P], causal_vis(P, 1), past=cache)
        if keep_logits:
            logits_kept.append(logits[0].copy())
        cache = _append(cache, kv)
        P += 1
        if temperature > 0:
            e, mr = restricted_weights(logits[0], temperature, top_k, top_p)
            cur, m = draw_from(e, set(), rng.uniform(seed, len(out), 0))
            margins.append(min(m, mr))
        else:
            cur = int(argmax_lowest(logits)[0])
        out.append(cur)
        if eos_id >= 0 and cur == eos_id:
            break
    return DecodeResult(out, len(out), [0] * len(out), [1] * len(out), logits_kept, [],
                        margins=margins)


def score(model: OracleModel, tokens) -> np.ndarray:
    """Teacher-forced logits at every position of `tokens` (causal)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    T = len(tokens)
    logits, _ = model.forward(tokens, np.arange(T), causal_vis(0, T))
    return logits


def lookahead(model: OracleModel, prompt, N: int, W: int, G: int, max_new: int,
              init_window, prompt_ref: bool = False, pool_cap: int | None = None,
              eos_id: int = -1, keep_logits: bool = False,
              pool: NGramPool | None = None, temperature: float = 0.0,
              seed: int = 0, top_k: int = 0, top_p: float = 1.0,
              pool_lru: bool = False, pool_context: bool = False) -> DecodeResult:
    """Lookahead decoding, one step per loop iteration ([LD] §3.2, §3.4).

    Each step: select candidates for cur from the pool; run one forward
    pass over [cur, window, candidates] under the lookahead mask; verify
    the candidates greedily (Algorithm 3); commit the accepted tokens; take
    the top level's outputs as the new window level, harvest one n-gram per
    column into the pool and slide the window.
    """
    if N < 2:
        raise ValueError("N >= 2")
    prompt = np.asarray(prompt, dtype=np.int64)
    cache, cur = prefill(model, prompt)
    P = cache[0][0].shape[0]
    if pool is None:
        pool = NGramPool(pool_cap if pool_cap is not None else max(G, 1), lru=pool_lru)
    if prompt_ref:                                           # R11
        for j in range(len(prompt) - N + 1):
            pool.insert(prompt[j], prompt[j + 1:j + N], prompt[j - 1] if j else -1)
    prev = int(prompt[-2]) if len(prompt) >= 2 else -1       # token before cur
    win = np.asarray(init_window, dtype=np.int64).reshape(N - 1, W).copy()
    M = n_rows(N, W, G)
    bmask = block_mask(N, W, G)
    out: list[int] = []
    res = DecodeResult([], 0, [], [], [], [], pool)
    while len(out) < max_new:
        # (3) selection: n-grams whose first token is the last output token
        cands = pool.select(cur, G, prev if pool_context else None)
        # block rows (R1), unused candidate slots hold token 0 (R8)
        toks = np.zeros(M, dtype=np.int64)
        toks[0] = cur
        for l in range(N - 1):
            for k in range(W):
                toks[1 + l * W + k] = win[l, k]
        base = 1 + W * (N - 1)
        for g, c in enumerate(cands):
            toks[base + g * (N - 1): base + (g + 1) * (N - 1)] = c
        pos = np.array([P + row_offset(r, N, W, G) for r in range(M)], dtype=np.int64)
        vis = np.concatenate([np.ones((M, P), dtype=bool), bmask], axis=1)
        logits, kv = model.forward(toks, pos, vis, past=cache)
        a = argmax_lowest(logits)
        if keep_logits:
            res.step_logits.append(logits)
            res.step_rows.append(toks.copy())

        if temperature > 0:
            emit, acc, g0, m = sample_verify(logits, cands, N, base, temperature, seed,
                                             res.steps, top_k, top_p)
            res.margins.append(m)
            bonus = emit[-1]
            prev_survivors = [g0]
        else:
            emit, acc, bonus, prev_survivors = _greedy_verify(a, cands, N, base)
        # commit: cur and the accepted tokens become committed rows
        committed_rows = [0]
        if acc:
            g0 = prev_survivors[0]
            committed_rows += [base + g0 * (N - 1) + j for j in range(acc)]
        cache = _append(cache, kv, rows=committed_rows)
        P += len(committed_rows)

        # lookahead branch: new tokens = outputs of the newest level
        new = np.array([a[1 + (N - 2) * W + k] for k in range(W)], dtype=np.int64)
        for k, gram in enumerate(harvest(win, new)):
            pool.insert(gram[0], gram[1:], win[0, k - 1] if k else cur)   # R22 context
        win = slide(win, new)

        # emit, truncated to the budget / at EOS (R10)
        room = max_new - len(out)
        step_emit = emit[:room]
        if eos_id >= 0 and eos_id in step_emit:
            step_emit = step_emit[:step_emit.index(eos_id) + 1]
        out.extend(step_emit)
        res.steps += 1
        res.accepted.append(acc)
        res.emitted.append(len(step_emit))
        res.ncand.append(len(cands))
        prev = int(emit[-2]) if len(emit) >= 2 else int(cur)
        cur = bonus
        if eos_id >= 0 and out and out[-1] == eos_id:
            break
    res.tokens = out
    return res


def _greedy_verify(a, cands, N: int, base: int):
    """Algorithm 3 on the block rows' argmax `a`, token by token along the
    suffixes (survivors = the candidates that matched so far): returns
    (emit, acc, bonus, survivors of the accepted prefix)."""
    def dist_row(g, i):            # row whose output is P_i for candidate g
        return 0 if i == 1 else base + g * (N - 1) + (i - 2)
    survivors = list(range(len(cands)))
    prev_survivors = [0]
    emit: list[int] = []
    i = 1
    # when no candidate matches, accept argmax P_i (from the last surviving
    # prefix; for i = 1 that is row 0) and stop
    while survivors and i <= N - 1:
        top = int(a[dist_row(survivors[0], i)])
        matched = [g for g in survivors if cands[g][i - 1] == top]
        if not matched:
            break
        emit.append(top)
        survivors = prev_survivors = matched
        i += 1
    acc = len(emit)
    if acc == 0:
        bonus = int(a[0])
    else:
        # argmax P_{acc+1} from a surviving candidate
        bonus = int(a[base + prev_survivors[0] * (N - 1) + (acc - 1)])
    emit.append(bonus)
    return emit, acc, bonus, prev_survivors
