// Device-side n-gram pool, candidate gather, greedy verification, window
// slide and KV commit of one lookahead step.
//
// Pool ([LD] §3.4 "N-gram pool update": key = first token, value = list of
// suffixes): direct-mapped by first token, V buckets of `cap` suffixes of
// N-1 tokens, each bucket a FIFO ring (head = oldest).  An identical suffix is
// skipped; a full bucket evicts its oldest entry.
//
// Gather ([LD] §3.4 "N-gram selection from the pool"): the bucket of the
// current token, oldest first; the newest G if it holds more.
//
// Verify ([LD] §3.4 "Greedy verification algorithm (Algorithm 3)") as a
// longest-prefix scan: candidate g's accepted length is the longest j with
// cand[g][i-1] == argmax(row predicting position P+i) for all i <= j; the
// first candidate with the longest match wins; the emitted tokens are its
// accepted prefix plus the argmax that follows it (argmax of row 0 when
// nothing is accepted), so every step emits 1..N tokens.
//
// Sampling verification ([LD] §3.4 "Sampling verification (Algorithm 4)"),
// used when the session has a temperature T > 0: at position i the
// distribution P_i = softmax(logits(row) / T) of the row that predicts
// position P+i (row 0 for i = 1, then the row of the accepted prefix) is
// tested against the surviving candidates' tokens in candidate order.  A
// token c is accepted when a draw r in (0, 1] satisfies r <= P_i'(c), where
// P_i' is P_i with the tokens rejected so far at this position set to zero
// and renormalised; a rejected token is set to zero (a second candidate with
// the same token is skipped without a draw).  When every candidate is
// rejected, a token drawn from P_i' ends the step; after N-1 accepted tokens
// a token drawn from P_N does.  The lookahead branch stays greedy (the window
// and the pool use the argmax), which the pages show leaves the output
// distribution that of sampling from the model.
#include "la_internal.h"

namespace {

__device__ __forceinline__ int32_t* bucket(const PoolDesc& p, int key, int e) {
  return p.tok + ((size_t)key * p.cap + e) * p.n1;
}
__device__ __forceinline__ int32_t& ctx_of(const PoolDesc& p, int key, int e) {
  return p.ctx[(size_t)key * p.cap + e];
}

struct InsertCounts {
  int ins, dup, ev, ngr, keys;
};

// Insert (key, sfx[0..n1)) with context token ctx (the token before the
// n-gram, -1 for none) into the pool; one thread.  A bucket is a ring of cap
// entries, oldest at head.  A suffix already present is counted as a repeat
// and takes the new context; with lru it also moves to the newest end (the
// entries after it move one place towards the head), so that eviction drops
// the suffix generated least recently ([LD] "Memory-efficient n-gram pool
// management" names LRU and FIFO as the policies to compare; FIFO leaves it
// in place).
__device__ void pool_insert(const PoolDesc& p, int key, const int32_t* sfx, int ctx,
                            InsertCounts& c) {
  const int cnt = p.cnt[key];
  const int head = p.head[key];
  for (int e = 0; e < cnt; ++e) {
    int idx = head + e;
    if (idx >= p.cap) idx -= p.cap;
    const int32_t* b = bucket(p, key, idx);
    bool same = true;
    for (int i = 0; i < p.n1; ++i) same = same && (b[i] == sfx[i]);
    if (same) {
      ++c.dup;
      if (p.lru) {
        for (int f = e; f + 1 < cnt; ++f) {
          int from = head + f + 1;
          if (from >= p.cap) from -= p.cap;
          int to = head + f;
          if (to >= p.cap) to -= p.cap;
          int32_t* dst = bucket(p, key, to);
          const int32_t* src = bucket(p, key, from);
          for (int i = 0; i < p.n1; ++i) dst[i] = src[i];
          ctx_of(p, key, to) = ctx_of(p, key, from);
        }
        int last = head + cnt - 1;
        if (last >= p.cap) last -= p.cap;
        int32_t* dst = bucket(p, key, last);
        for (int i = 0; i < p.n1; ++i) dst[i] = sfx[i];
        idx = last;
      }
      ctx_of(p, key, idx) = ctx;
      return;
    }
  }
  ++c.ins;
  int idx;
  if (cnt < p.cap) {
    idx = head + cnt;
    if (idx >= p.cap) idx -= p.cap;
    p.cnt[key] = cnt + 1;
    ++c.ngr;
    if (cnt == 0) ++c.keys;
  } else {
    idx = head;
    p.head[key] = head + 1 == p.cap ? 0 : head + 1;
    ++c.ev;
  }
  int32_t* b = bucket(p, key, idx);
  for (int i = 0; i < p.n1; ++i) b[i] = sfx[i];
  ctx_of(p, key, idx) = ctx;
}

// Candidate g of the step is bucket entry s_sel[g] (ring index): the newest
// G entries in bucket order, or, selecting by context, the newest entries
// whose context is the token before cur and then the newest of the rest,
// still in bucket order (one thread marks them walking from the newest end).
constexpr int GATHER_MAX_G = 1024;
__global__ __launch_bounds__(256) void k_gather(PoolDesc pool, StepIO io, RowLayout L) {
  __shared__ int s_take;
  __shared__ int s_sel[GATHER_MAX_G];
  DevState* st = io.st;
  const int cur = st->cur, P = st->P;
  const int n1 = L.N - 1;
  if (threadIdx.x == 0) {
    const int cnt = L.G > 0 ? pool.cnt[cur] : 0;
    const int take = cnt < L.G ? cnt : L.G;
    const int head = pool.head[cur];
    s_take = take;
    if (!pool.by_ctx || take == cnt) {
      for (int g = 0; g < take; ++g) {
        int e = head + (cnt - take) + g;
        if (e >= pool.cap) e -= pool.cap;
        s_sel[g] = e;
      }
    } else {
      // the bucket position (0 = oldest) of the entries taken, in bucket
      // order: first count the matches among the newest, then merge
      const int prev = st->prev;
      int nm = 0;
      for (int j = cnt - 1; j >= 0 && nm < take; --j) {
        int e = head + j;
        if (e >= pool.cap) e -= pool.cap;
        nm += ctx_of(pool, cur, e) == prev;
      }
      // take the nm newest matches and the take - nm newest others
      int need_m = nm, need_o = take - nm, g = take;
      for (int j = cnt - 1; j >= 0 && g > 0; --j) {
        int e = head + j;
        if (e >= pool.cap) e -= pool.cap;
        const bool m = ctx_of(pool, cur, e) == prev;
        if (m && need_m > 0) { s_sel[--g] = e; --need_m; }
        else if (!m && need_o > 0) { s_sel[--g] = e; --need_o; }
      }
    }
    st->ncand = take;
    st->stats[ST_GATHER_NE] += take > 0;
    st->stats[ST_CAND_TOTAL] += take;
  }
  __syncthreads();
  const int take = s_take;
  for (int u = threadIdx.x; u < L.G * n1; u += blockDim.x) {
    const int g = u / n1, i = u - g * n1;
    int v = 0;  // unused candidate slots hold token 0
    if (g < take) v = bucket(pool, cur, s_sel[g])[i];
    io.cand[u] = v;
    io.ids[1 + L.W * n1 + u] = v;
    io.pos[1 + L.W * n1 + u] = P + i + 1;
  }
  for (int u = threadIdx.x; u < L.W * n1; u += blockDim.x) {
    const int l = u / L.W, k = u - l * L.W;
    io.ids[1 + u] = io.win[u];
    io.pos[1 + u] = P + 1 + l + k;
  }
  if (threadIdx.x == 0) {
    io.ids[0] = cur;
    io.pos[0] = P;
  }
}

constexpr int VMAX_M = 2048;  // rows staged in LDS by the verify kernel
constexpr int VFY_T = 256;    // threads of the verify kernel (four waves)

// Greedy verification ([LD] §3.4 "Greedy verification algorithm (Algorithm
// 3)"), then the lookahead branch's harvest, pool insert and slide.
//  * compare: slot u = g(N-1) + i-1 of the G x (N-1) grid says whether
//    candidate token cand[g][i-1] equals the argmax of the row that predicts
//    position P+i (row 0 for i = 1, else candidate g's row i-2); the slots
//    are spread over all lanes of the four waves;
//  * longest-prefix scan: candidate g's accepted length is the count of its
//    leading matching slots; the best candidate is found with a max over
//    the key (length << 11 | 2047 - g), i.e. the longest, then the first;
//  * one thread then commits, emits and updates the counters (<= N tokens).
// The harvest forms one n-gram per window column k, for every k < W: key
// win[0][k], suffix win[1..N-2][k] followed by the column's new token
// ([LD] §3.4 "N-gram harvesting and pool update").  Columns with the same
// key go to the same bucket and must be inserted in column order (a repeat
// within the step is a duplicate), so the lowest column of each key inserts
// all of that key's columns in order; different keys touch different
// buckets.  Columns are dealt to the 256 threads with a stride, so any W the
// step allows is harvested.
__global__ __launch_bounds__(VFY_T) void k_verify(PoolDesc pool, StepIO io, RowLayout L) {
  __shared__ int32_t a[VMAX_M];
  __shared__ int32_t cand[VMAX_M];
  __shared__ int32_t win[VMAX_M];
  __shared__ uint8_t match[VMAX_M];
  __shared__ int s_key[VFY_T / 64];
  __shared__ int red[VFY_T / 64][5];
  DevState* st = io.st;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n1 = L.N - 1, W = L.W, G = L.G, M = L.M;
  const int cur_old = io.ids[0];  // the step's current token (row 0)
  const int vbase = 1 + W * n1;
  for (int i = tid; i < M; i += VFY_T) a[i] = io.amax[i];
  for (int i = tid; i < G * n1; i += VFY_T) cand[i] = io.cand[i];
  for (int i = tid; i < W * n1; i += VFY_T) win[i] = io.win[i];
  __syncthreads();

  if (io.temp <= 0.f) {
    const int ncand = st->ncand;
    for (int u = tid; u < G * n1; u += VFY_T) {
      const int g = u / n1, i = u - g * n1 + 1;
      const int pred = i == 1 ? 0 : vbase + g * n1 + (i - 2);
      match[u] = g < ncand && cand[u] == a[pred];
    }
    __syncthreads();
    int key = 2047;  // nothing accepted, candidate 0
    for (int g = tid; g < ncand; g += VFY_T) {
      int acc = 0;
      while (acc < n1 && match[g * n1 + acc]) ++acc;
      key = max(key, (acc << 11) | (2047 - g));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, 64));
    if (lane == 0) s_key[wv] = key;
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < VFY_T / 64; ++w) key = max(key, s_key[w]);
      const int best = key >> 11, bg = 2047 - (key & 2047);
      const int bonus = best == 0 ? a[0] : a[vbase + bg * n1 + best - 1];
      // commit: row 0 and the accepted candidate rows become cache rows P..P+best
      st->commit_p = st->P;
      st->commit_n = best + 1;
      st->commit_rows[0] = 0;
      for (int j = 1; j <= best; ++j) st->commit_rows[j] = vbase + bg * n1 + j - 1;
      st->P += best + 1;
      // emit, truncated to the budget; stop after EOS
      const int room = io.max_new - st->total;
      int n = 0, done = 0;
      for (int j = 0; j <= best && n < room; ++j) {
        const int tok = j < best ? cand[bg * n1 + j] : bonus;
        st->out[n++] = tok;
        if (io.eos >= 0 && tok == io.eos) { done = 1; break; }
      }
      st->n_out = n;
      st->total += n;
      if (st->total >= io.max_new) done = 1;
      if (done) st->done = 1;
      st->cur = bonus;
      st->stats[ST_HIST0 + best] += 1;
      st->stats[ST_STEPS] += 1;
      st->stats[ST_TOKENS] += n;
    }
  }
  if (tid == 0) {
    // the token before the new cur: the second to last emitted, or the old
    // cur when one token was emitted (greedy above, or sampling verification
    // before this kernel); a truncated step ends the session
    const int n = st->n_out;
    st->prev = n >= 2 ? st->out[n - 2] : cur_old;
  }

  InsertCounts c = {0, 0, 0, 0, 0};
  for (int k = tid; k < W; k += VFY_T) {
    const int key = win[k];
    bool leader = true;
    for (int k2 = 0; k2 < k; ++k2)
      if (win[k2] == key) { leader = false; break; }
    if (!leader) continue;
    int32_t sfx[LA_MAX_N];
    for (int k2 = k; k2 < W; ++k2) {
      if (win[k2] != key) continue;
      for (int l = 1; l < n1; ++l) sfx[l - 1] = win[l * W + k2];
      sfx[n1 - 1] = a[1 + (n1 - 1) * W + k2];
      // context: the level-0 token to the column's left, or the step's cur
      pool_insert(pool, key, sfx, k2 > 0 ? win[k2 - 1] : cur_old, c);
    }
  }
  int cv[5] = {c.ins, c.dup, c.ev, c.ngr, c.keys};
#pragma unroll
  for (int j = 0; j < 5; ++j) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cv[j] += __shfl_xor(cv[j], o, 64);
    if (lane == 0) red[wv][j] = cv[j];
  }
  __syncthreads();
  if (tid == 0) {
    long long t[5] = {0, 0, 0, 0, 0};
    for (int w = 0; w < VFY_T / 64; ++w)
      for (int j = 0; j < 5; ++j) t[j] += red[w][j];
    st->stats[ST_INSERTS] += t[0];
    st->stats[ST_DUPS] += t[1];
    st->stats[ST_EVICT] += t[2];
    st->stats[ST_NGRAMS] += t[3];
    st->stats[ST_KEYS] += t[4];
    // candidates the next step's gather will take for the new cur (every
    // insert of this step is done: they precede the barrier above)
    const int nc = io.gmax > 0 ? pool.cnt[st->cur] : 0;
    st->next_g = nc < io.gmax ? nc : io.gmax;
  }
  // slide: drop the oldest level, the new tokens become the newest level
  for (int u = tid; u < W * n1; u += VFY_T) {
    const int l = u / W, k = u - l * W;
    io.win[u] = l + 1 < n1 ? win[(l + 1) * W + k] : a[1 + (n1 - 1) * W + k];
  }
}

// ---------------------------------------------------------------------------
// Counter-based draws: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011): per round two 32x32-bit
// products with the multipliers 0xD2511F53 and 0xCD9E8D57, the key advanced
// by 0x9E3779B9 / 0xBB67AE85 between rounds, ten rounds.  Draw k of step s
// under seed x is word 0 of Philox((s lo, s hi, k, 0), (x lo, x hi)), mapped
// to ((w >> 8) + 1) * 2^-24 in (0, 1].
__device__ __forceinline__ uint32_t philox_w0(unsigned long long seed, unsigned long long step,
                                              uint32_t k) {
  uint32_t c0 = (uint32_t)step, c1 = (uint32_t)(step >> 32), c2 = k, c3 = 0;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}
__device__ __forceinline__ float draw01(unsigned long long seed, unsigned long long step,
                                        uint32_t k) {
  return (float)((philox_w0(seed, step, k) >> 8) + 1u) * (1.0f / 16777216.0f);
}

__global__ void k_philox_uniform(unsigned long long seed, unsigned long long step, int n,
                                 float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = draw01(seed, step, (uint32_t)i);
}

constexpr int SV_T = 1024;  // threads of the sampling verification

// Sampling weights of the rows the verification may visit: row 0 and every
// verification row of a gathered candidate, one workgroup each, all at once
// (they depend on their row's logits only).  Block b takes row 0 (b = 0) or
// verification row b - 1; it leaves e[v] = exp((logit_v - max) / T), cut to
// the top-K / top-P set, in sw[b][v] and their sum Z in sz[b].  Thread t
// owns the contiguous vocabulary slice [t*CH, (t+1)*CH).  Sums: each thread
// adds its slice in index order; the 1024 slice sums are added by a fixed
// halving tree (Z) or scanned (wave scans by shuffles, then the 16 wave
// totals in order).
__global__ __launch_bounds__(SV_T) void k_sample_weights(StepIO io, RowLayout L) {
  __shared__ __align__(16) float e[SAMPLE_VMAX];
  __shared__ float red[SV_T];
  // wave totals, double-buffered: a reduction writes the buffer the one
  // before it did not, so one barrier per reduction suffices (every thread
  // has read a buffer before it passes the next reduction's barrier)
  __shared__ float wtot[2][SV_T / 64];
  __shared__ int wcnt[2][SV_T / 64];
  int par = 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n1 = L.N - 1, V = io.V;
  const int b = blockIdx.x;
  // a verification row of a candidate the gather did not fill is never visited
  if (b > 0 && (b - 1) / n1 >= io.st->ncand) return;
  const int row = b == 0 ? 0 : 1 + L.W * n1 + (b - 1);
  const int CH = (V + SV_T - 1) / SV_T;
  const int v0 = min(V, tid * CH), v1 = min(V, v0 + CH);
  constexpr int CHMAX = (SAMPLE_VMAX + SV_T - 1) / SV_T;

  // Block-wide integer count and float sum, the same on every thread: a
  // shuffle tree within each wave (each pairwise sum is symmetric, so every
  // lane ends with the same bits), then the 16 wave totals in order.
  auto block_count = [&](int c) -> int {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if (lane == 0) wcnt[par][wv] = c;
    __syncthreads();
    int t = 0;
    for (int w = 0; w < SV_T / 64; ++w) t += wcnt[par][w];
    par ^= 1;
    return t;
  };
  auto block_fsum = [&](float x) -> float {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    if (lane == 0) wtot[par][wv] = x;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < SV_T / 64; ++w) t += wtot[par][w];
    par ^= 1;
    return t;
  };
  // exclusive prefix over the threads (vocabulary order) of x
  auto block_exscan = [&](float x) -> float {
    float y = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(y, o, 64);
      if (lane >= o) y += t;
    }
    if (lane == 63) wtot[par][wv] = y;
    __syncthreads();
    float before = 0.f;
    for (int w = 0; w < wv; ++w) before += wtot[par][w];
    par ^= 1;
    return before + (y - x);
  };
  auto block_exscan_i = [&](int x) -> int {
    int y = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(y, o, 64);
      if (lane >= o) y += t;
    }
    if (lane == 63) wcnt[par][wv] = y;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wcnt[par][w];
    par ^= 1;
    return before + (y - x);
  };
  // Top-K / top-P cut of e[] (the row's logits `lg`): tokens are ranked by
  // logit, higher first, ties to the lower id.  Thresholds are found bit by
  // bit on an order-preserving integer key of the logit; the tokens tied at
  // the threshold are taken in id order (the thread slices are in id order).
  auto restrict_cut = [&](const float* lg) {
    // order-preserving keys of the slice's logits; keys past the slice are
    // 0, below every finite logit's key and below every threshold the
    // searches try (those are >= 1), so the searches need no range test
    uint32_t kk[CHMAX];
#pragma unroll
    for (int j = 0; j < CHMAX; ++j) {
      const uint32_t u = v0 + j < v1 ? __float_as_uint(lg[v0 + j]) : 0u;
      kk[j] = v0 + j < v1 ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
    }
    auto in = [&](int j) { return v0 + j < v1; };
    if (io.top_k > 0) {
      // the top_k-th largest key: the largest t with #{key >= t} >= top_k
      // (each wave counts its keys >= c by ballots: one compare per key and
      // a scalar popcount, no lane exchange; integer counts in any order)
      uint32_t t = 0;
      for (int b = 31; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        int n = 0;
#pragma unroll
        for (int j = 0; j < CHMAX; ++j) n += __popcll(__ballot(kk[j] >= c));
        if (lane == 0) wcnt[par][wv] = n;
        __syncthreads();
        int tot = 0;
        for (int w = 0; w < SV_T / 64; ++w) tot += wcnt[par][w];
        par ^= 1;
        if (tot >= io.top_k) t = c;
      }
      int ngt = 0, neq = 0;
#pragma unroll
      for (int j = 0; j < CHMAX; ++j) {
        ngt += in(j) && kk[j] > t;
        neq += in(j) && kk[j] == t;
      }
      const int need = io.top_k - block_count(ngt);  // tied tokens kept, lowest ids
      int seen = block_exscan_i(neq);
#pragma unroll
      for (int j = 0; j < CHMAX; ++j) {
        if (!in(j)) continue;
        if (kk[j] < t) e[v0 + j] = 0.f;
        else if (kk[j] == t) {
          if (seen >= need) e[v0 + j] = 0.f;
          ++seen;
        }
      }
      __syncthreads();
    }
    if (io.top_p < 1.f) {
      // this thread's weights (its own slice of e[], after the top-K cut)
      float ev[CHMAX];
#pragma unroll
      for (int j = 0; j < CHMAX; ++j) ev[j] = in(j) ? e[v0 + j] : 0.f;
      float loc = 0.f;  // (+0 for the keys past the slice: the same sum)
#pragma unroll
      for (int j = 0; j < CHMAX; ++j) loc += ev[j];
      const float target = io.top_p * block_fsum(loc);
      // the largest key t whose tokens at or above it hold the target
      uint32_t t = 0;
      for (int b = 31; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < CHMAX; ++j) x += kk[j] >= c ? ev[j] : 0.f;
        if (block_fsum(x) >= target) t = c;
      }
      float sgt = 0.f, seq = 0.f;
#pragma unroll
      for (int j = 0; j < CHMAX; ++j) {
        if (!in(j)) continue;
        if (kk[j] > t) sgt += ev[j];
        else if (kk[j] == t) seq += ev[j];
      }
      const float above = block_fsum(sgt);
      float run = above + block_exscan(seq);
      bool full = run >= target;  // the tied tokens of earlier slices reached it
#pragma unroll
      for (int j = 0; j < CHMAX; ++j) {
        if (!in(j)) continue;
        if (kk[j] < t) e[v0 + j] = 0.f;
        else if (kk[j] == t) {
          if (full) e[v0 + j] = 0.f;
          else {
            run += ev[j];
            full = run >= target;
          }
        }
      }
      __syncthreads();
    }
  };

  // load row `row`'s weights into e[], return Z (fixed order)
  auto weights = [&](int row) -> float {
    const float* lg = io.logits + (size_t)row * V;
    float m = -INFINITY;
    for (int v = v0; v < v1; ++v) m = fmaxf(m, lg[v]);
    red[tid] = m;
    __syncthreads();
    for (int s = SV_T / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
      __syncthreads();
    }
    const float mx = red[0];
    __syncthreads();
    float sum = 0.f;
    for (int v = v0; v < v1; ++v) {
      const float w = expf((lg[v] - mx) / io.temp);
      e[v] = w;
      sum += w;
    }
    if (io.top_k > 0 || io.top_p < 1.f) {
      restrict_cut(lg);
      sum = 0.f;
      for (int v = v0; v < v1; ++v) sum += e[v];
    }
    red[tid] = sum;
    __syncthreads();
    for (int s = SV_T / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    const float z = red[0];
    __syncthreads();
    return z;
  };
  const float z = weights(row);
  float* dst = io.sw + (size_t)b * V;
  if ((V & 3) == 0) {
    for (int v = 4 * tid; v < V; v += 4 * SV_T) *(float4*)&dst[v] = *(const float4*)&e[v];
  } else {
    for (int v = tid; v < V; v += SV_T) dst[v] = e[v];
  }
  if (tid == 0) io.sz[b] = z;
}

// One workgroup: the verification itself, over the weights k_sample_weights
// left (copied into LDS for the visited row), the draws in order.
__global__ __launch_bounds__(SV_T) void k_sample_verify(StepIO io, RowLayout L) {
  __shared__ __align__(16) float e[SAMPLE_VMAX];
  __shared__ float wtot[SV_T / 64];
  __shared__ int32_t removed[VMAX_M];
  __shared__ int32_t surv[VMAX_M];
  __shared__ int s_nrem, s_pick, s_nsurv, s_row, s_done_pos;
  __shared__ float s_target;
  __shared__ int32_t emitted[LA_MAX_N];  // accepted tokens, then the drawn one
  DevState* st = io.st;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n1 = L.N - 1, V = io.V;
  const int vbase = 1 + L.W * n1;
  const int CH = (V + SV_T - 1) / SV_T;
  const int v0 = min(V, tid * CH), v1 = min(V, v0 + CH);
  const unsigned long long step = (unsigned long long)st->stats[ST_STEPS];
  const int ncand = st->ncand;
  uint32_t k = 0;  // draws used (same on every thread)

  // row `row`'s weights into e[] (coalesced), return Z
  auto weights = [&](int row) -> float {
    const int b = row == 0 ? 0 : row - vbase + 1;
    const float* src = io.sw + (size_t)b * V;
    if ((V & 3) == 0) {
      for (int v = 4 * tid; v < V; v += 4 * SV_T) *(float4*)&e[v] = *(const float4*)&src[v];
    } else {
      for (int v = tid; v < V; v += SV_T) e[v] = src[v];
    }
    __syncthreads();
    return io.sz[b];
  };
  // residual draw: the first token v (index order, not removed) whose
  // running sum of weights reaches u * (sum of the remaining weights)
  auto residual = [&](float u) -> int {
    const int nrem = s_nrem;
    float sum = 0.f;
    for (int v = v0; v < v1; ++v) {
      bool rm = false;
      for (int j = 0; j < nrem; ++j) rm = rm || removed[j] == v;
      if (!rm) sum += e[v];
    }
    // inclusive scan of the slice sums within the wave, then the wave
    // totals in order; a slice covers (excl, incl], and the next slice's
    // excl is this slice's incl, so exactly one slice holds the target
    float x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const float xprev = __shfl_up(x, 1, 64);
    if (lane == 63) wtot[wv] = x;
    if (tid == 0) s_pick = -1;
    __syncthreads();
    float before = 0.f;
    for (int w = 0; w < wv; ++w) before += wtot[w];
    float total = 0.f;
    for (int w = 0; w < SV_T / 64; ++w) total += wtot[w];
    const float incl = before + x;
    const float excl = lane == 0 ? before : before + xprev;
    const float target = u * total;
    if (sum > 0.f && excl < target && incl >= target) {
      float run = excl;
      int pick = -1;
      for (int v = v0; v < v1; ++v) {
        bool rm = false;
        for (int j = 0; j < nrem; ++j) rm = rm || removed[j] == v;
        if (rm) continue;
        run += e[v];
        if (run >= target) { pick = v; break; }
      }
      if (pick < 0) {  // rounding inside the slice: its last positive weight
        for (int v = v1 - 1; v >= v0; --v) {
          bool rm = false;
          for (int j = 0; j < nrem; ++j) rm = rm || removed[j] == v;
          if (!rm && e[v] > 0.f) { pick = v; break; }
        }
      }
      s_pick = pick;
    }
    __syncthreads();
    if (s_pick < 0 && tid == 0) {
      // target beyond the scanned total by rounding: the last positive weight
      for (int v = V - 1; v >= 0; --v) {
        bool rm = false;
        for (int j = 0; j < nrem; ++j) rm = rm || removed[j] == v;
        if (!rm && e[v] > 0.f) { s_pick = v; break; }
      }
    }
    __syncthreads();
    return s_pick;
  };

  if (tid == 0) {
    s_nsurv = ncand;
    s_row = 0;
  }
  for (int g = tid; g < ncand; g += SV_T) surv[g] = g;
  __syncthreads();
  int acc = 0, last = -1;
  for (int i = 1; i <= n1 + 1; ++i) {
    const float z = weights(s_row);
    if (tid == 0) {
      s_nrem = 0;
      s_pick = -1;
      s_done_pos = 1;
      float zr = z;
      if (i <= n1) {
        for (int j = 0; j < s_nsurv; ++j) {
          const int c = io.cand[surv[j] * n1 + i - 1];
          bool seen = false;
          for (int q = 0; q < s_nrem; ++q) seen = seen || removed[q] == c;
          if (seen) continue;
          const float r = draw01(io.seed, step, k++);
          if (r * zr <= e[c]) { s_pick = c; break; }
          removed[s_nrem++] = c;
          zr -= e[c];
        }
      }
      if (s_pick >= 0) {
        // survivors: candidates whose i-th token is the accepted one
        int ns = 0;
        for (int j = 0; j < s_nsurv; ++j)
          if (io.cand[surv[j] * n1 + i - 1] == s_pick) surv[ns++] = surv[j];
        s_nsurv = ns;
        s_row = vbase + surv[0] * n1 + (i - 1);
        s_done_pos = 0;
      } else {
        s_target = draw01(io.seed, step, k++);
      }
    }
    __syncthreads();
    if (!s_done_pos) {
      if (tid == 0) emitted[acc] = s_pick;
      ++acc;
      __syncthreads();
      continue;
    }
    const int t = residual(s_target);
    last = t;
    break;
  }
  if (tid == 0) {
    // commit: row 0 and the accepted candidate rows become cache rows
    st->commit_p = st->P;
    st->commit_n = acc + 1;
    st->commit_rows[0] = 0;
    const int g0 = acc > 0 ? surv[0] : 0;
    for (int j = 1; j <= acc; ++j) st->commit_rows[j] = vbase + g0 * n1 + j - 1;
    st->P += acc + 1;
    emitted[acc] = last;
    const int room = io.max_new - st->total;
    int n = 0, done = 0;
    for (int j = 0; j <= acc && n < room; ++j) {
      st->out[n++] = emitted[j];
      if (io.eos >= 0 && emitted[j] == io.eos) { done = 1; break; }
    }
    st->n_out = n;
    st->total += n;
    if (st->total >= io.max_new) done = 1;
    if (done) st->done = 1;
    st->cur = last;
    st->stats[ST_HIST0 + acc] += 1;
    st->stats[ST_STEPS] += 1;
    st->stats[ST_TOKENS] += n;
  }
}

// Copy the committed block rows' K and V into the cache, 16 bytes per
// thread and step (a 16-byte piece never crosses a head: hd is a multiple
// of 8).
template <typename T>
__global__ __launch_bounds__(256) void k_kv_commit(KvCommit c) {
  constexpr int EP = 16 / (int)sizeof(T);  // elements per 16-byte piece
  const int l = blockIdx.x, j = blockIdx.y;
  const int n = c.st->commit_n;
  if (j >= n) return;
  const int row = c.st->commit_rows[j];
  const int p = c.st->commit_p + j;
  const int nk = c.Hkv * c.hd;
  const T* kb = (const T*)c.kb + ((size_t)l * c.M + row) * nk;
  const T* vb = (const T*)c.vb + ((size_t)l * c.M + row) * nk;
  T* kc = (T*)c.kc + (size_t)l * c.Hkv * c.ld_ctx * c.hd;
  T* vc = (T*)c.vc + (size_t)l * c.Hkv * c.ld_ctx * c.hd;
  for (int u = threadIdx.x * EP; u < nk; u += blockDim.x * EP) {
    const int kvh = u / c.hd, i = u - kvh * c.hd;
    const size_t dst = ((size_t)kvh * c.ld_ctx + p) * c.hd + i;
    *(u32x4_t*)(kc + dst) = *(const u32x4_t*)(kb + u);
    *(u32x4_t*)(vc + dst) = *(const u32x4_t*)(vb + u);
  }
}

// Prompt as reference: insert prompt[j .. j+N-1] for j = 0 .. n-N in order.
__global__ void k_pool_seed(PoolDesc pool, DevState* st, const int32_t* prompt, int n) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  InsertCounts c = {0, 0, 0, 0, 0};
  for (int j = 0; j + pool.n1 < n; ++j)
    pool_insert(pool, prompt[j], prompt + j + 1, j > 0 ? prompt[j - 1] : -1, c);
  st->stats[ST_INSERTS] += c.ins;
  st->stats[ST_DUPS] += c.dup;
  st->stats[ST_EVICT] += c.ev;
  st->stats[ST_NGRAMS] += c.ngr;
  st->stats[ST_KEYS] += c.keys;
}

__global__ void k_fill_i32(int32_t* p, int32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Streaming read: wave w of the grid XORs the 16-byte words of slice w
// (ceil(n16 / waves) rounded up to whole 1 KB wave-loads; the last slices may
// be short or empty); the per-block XOR goes to out[block] so the loads are
// not dead.
__global__ __launch_bounds__(256) void k_probe_read(const uint4* __restrict__ buf, size_t n16,
                                                    uint32_t* out) {
  // each wave streams one contiguous slice of 1 KB wave-loads (16 bytes a
  // lane, non-temporal) and keeps PD of them in flight: a load is reissued
  // as soon as its value has been folded into the checksum
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  constexpr int PD = 32;
  const int lane = threadIdx.x & 63;
  const size_t waves = (size_t)gridDim.x * 4;
  const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t per = ((n16 + waves - 1) / waves + 63) / 64 * 64;
  const size_t lo = w * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  const size_t nk = hi > lo ? (hi - lo + 63) / 64 : 0;  // wave-loads of this slice
  auto load = [&](size_t k) -> u4v {
    const size_t j = lo + k * 64 + lane;
    return k < nk && j < hi ? __builtin_nontemporal_load((const u4v*)(buf + j)) : u4v{0u, 0u, 0u, 0u};
  };
  u4v r[PD];
#pragma unroll
  for (int u = 0; u < PD; ++u) r[u] = load(u);
  uint32_t acc = 0;
  for (size_t k0 = 0; k0 < nk; k0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
      r[u] = load(k0 + PD + u);
    }
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t st) {
  la_launch(k_probe_read, dim3(LA_PROBE_BLOCKS), dim3(256), 0, st, (const uint4*)buf, bytes / 16,
            out);
  return hipGetLastError();
}

hipError_t launch_gather(const PoolDesc& pool, const StepIO& io, const RowLayout& lay,
                         hipStream_t st) {
  if (lay.G > GATHER_MAX_G) return hipErrorInvalidValue;
  la_launch(k_gather, dim3(1), dim3(256), 0, st, pool, io, lay);
  return hipGetLastError();
}

hipError_t launch_verify(const PoolDesc& pool, const StepIO& io, const RowLayout& lay,
                         hipStream_t st) {
  if (lay.M > VMAX_M || lay.G > 1024) return hipErrorInvalidValue;
  la_launch(k_verify, dim3(1), dim3(VFY_T), 0, st, pool, io, lay);
  return hipGetLastError();
}

hipError_t launch_sample_weights(const StepIO& io, const RowLayout& lay, hipStream_t st) {
  if (lay.M > VMAX_M || io.V > SAMPLE_VMAX || io.V < 1 || !(io.temp > 0.f) || lay.N < 2 ||
      !io.sw || !io.sz)
    return hipErrorInvalidValue;
  la_launch(k_sample_weights, dim3(1 + lay.G * (lay.N - 1)), dim3(SV_T), 0, st, io, lay);
  return hipGetLastError();
}

hipError_t launch_sample_verify(const StepIO& io, const RowLayout& lay, hipStream_t st) {
  if (lay.M > VMAX_M || io.V > SAMPLE_VMAX || io.V < 1 || !(io.temp > 0.f) || !io.sw || !io.sz)
    return hipErrorInvalidValue;
  la_launch(k_sample_verify, dim3(1), dim3(SV_T), 0, st, io, lay);
  return hipGetLastError();
}

hipError_t launch_philox_uniform(unsigned long long seed, unsigned long long step, int n,
                                 float* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  la_launch(k_philox_uniform, dim3((n + 255) / 256), dim3(256), 0, st, seed, step, n,
            out);
  return hipGetLastError();
}

hipError_t launch_kv_commit(const KvCommit& c, int dtype, hipStream_t st) {
  dim3 grid(c.L, c.nmax);
  if (dtype == LA_BF16)
    la_launch(k_kv_commit<bf16_t>, grid, dim3(256), 0, st, c);
  else
    la_launch(k_kv_commit<float>, grid, dim3(256), 0, st, c);
  return hipGetLastError();
}

hipError_t launch_pool_seed(const PoolDesc& pool, DevState* st, const int32_t* prompt, int n,
                            hipStream_t st_) {
  la_launch(k_pool_seed, dim3(1), dim3(64), 0, st_, pool, st, prompt, n);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  la_launch(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

hipError_t launch_fill_bytes0(void* p, size_t n, hipStream_t st) {
  // callers pass 4-byte multiples
  return launch_fill_i32((int32_t*)p, 0, n / 4, st);
}
