/*
 * la.h -- C-ABI of the lookahead decoding step on one AMD MI355X (gfx950).
 *
 * The calls follow the problem as stated in "Break the Sequential Dependency
 * of LLM Inference Using LOOKAHEAD DECODING" (cited [LD]): a prompt x0
 * (§3.4 "Mathematical Reformulation"), the hyperparameters W, N, G (§3.4
 * "The Lookahead Branch", "N-gram selection from the pool"), one step that
 * returns the accepted tokens -- at least one (§3.4 "Greedy verification
 * algorithm (Algorithm 3)") -- and the observable step compression and pool
 * (§3.4 "Scaling Law", §3.4 "N-gram pool update").
 *
 * Conventions for every call:
 *  - Return value: LA_OK (0), LA_DONE (1, la_step only) or a negative
 *    la_status.  On error, la_last_error() returns a thread-local message.
 *    No C++ exception crosses this boundary.
 *  - "device pointer": memory of the current HIP device (e.g. a torch
 *    tensor's data_ptr()); "host pointer": ordinary CPU memory.
 *  - Streams: a hipStream_t passed as void*; NULL means the null stream.
 *    All device work of a model / session is enqueued on its stream.
 *  - The library never frees caller memory and allocates no device memory:
 *    all session state lives in the caller's workspace.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_DONE = 1,       /* la_step: max_new tokens emitted or EOS emitted */
  LA_EINVAL = -1,    /* bad argument (checked before any device work)   */
  LA_ENOMEM = -2,    /* workspace too small                              */
  LA_ECTX = -3,      /* context full: next step would pass max_ctx       */
  LA_EHIP = -4,      /* a HIP call failed; the session is poisoned       */
  LA_ESTATE = -5     /* call not valid in the object's state             */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Upper bound on N (n-gram length). */
#define LA_MAX_N 16

/* Decoder shape (a LLaMA-shaped decoder: RMSNorm, rotate-half RoPE,
 * SiLU-gated MLP, MHA or GQA, untied embedding and LM head).  The pages
 * evaluate LLaMA-2 / CodeLlama ([LD] §5 "Evaluation Methodology"). */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab;
  float rope_theta;  /* RoPE base, e.g. 10000                         */
  float norm_eps;    /* RMSNorm epsilon, e.g. 1e-5                     */
  int32_t dtype;     /* la_dtype of weights, KV cache and activations */
} la_model_desc;

/* Decode parameters.
 * N  n-gram length (2..LA_MAX_N); the window has N-1 levels ([LD] §3.4
 *    "The Lookahead Branch").
 * W  window width (columns), >= 0.
 * G  max verification candidates per step, 0..1024 ([LD] §3.4 "N-gram
 *    selection from the pool").
 * pool_cap   suffixes kept per first token; 0 means G (min 1).
 * max_ctx    KV-cache capacity in positions.
 * max_new    tokens to generate.
 * eos_id     stop after emitting this id; -1 for none.
 * flags      LA_PROMPT_REF: seed the pool with the prompt's n-grams
 *              ([LD] §5 Table 3, prompt as reference).
 *            LA_AR: plain greedy autoregressive decoding through the same
 *              kernels (W = G = 0 internally; one token per step).
 *            LA_NO_GRAPH: launch every step's kernels eagerly instead of
 *              replaying a captured HIP graph.
 *            LA_DEBUG_LOGITS: every step leaves its rows' logits for
 *              la_debug_logits.  Without it a bf16 session keeps them only
 *              when it samples (temperature > 0): its LM head reduces each
 *              row to its argmax and writes no logits (fp32 sessions keep
 *              them always).
 *            LA_POOL_LRU: evict by recency instead of FIFO.  A suffix that
 *              is generated again (from the window or the prompt) becomes
 *              its bucket's newest entry, so a full bucket drops the one
 *              generated least recently.  The pages leave the pool's cap and
 *              eviction policy unablated and name LRU and FIFO as the
 *              policies to compare ([LD] "What is not ablated",
 *              "Memory-efficient n-gram pool management").  Selection (the
 *              newest G of the bucket) and the output tokens are unchanged;
 *              repeats are still counted in dup_skips.
 *            LA_POOL_CONTEXT: select by a longer match.  Every entry keeps
 *              the token just before its n-gram where it was generated (for
 *              a window column the level-0 token of the column to its left,
 *              or the step's current token; for a prompt n-gram the prompt
 *              token before it).  The G candidates are then the newest
 *              entries whose context equals the token before the current
 *              one, then the newest of the rest, in the bucket's order.  The
 *              pages contrast first-token matching with longer prefixes
 *              ([LD] Table 3, "What is not ablated").  Output tokens are
 *              unchanged; it matters only when pool_cap > G.
 *            LA_ADAPTIVE_G: a step's verification branch holds only the
 *              candidate rows its GEMM row tiles need: the step after one
 *              that found g candidates for its next token processes
 *              1 + (W + G')(N-1) rows, G' the most candidates (at most G)
 *              that fit the same 16-row tiles as g (the pages verify "up to
 *              G" candidates, [LD] §3.4 "N-gram selection from the pool").
 *              Candidate rows past the pool's candidates are padding that
 *              can never be accepted, so tokens, steps and every pool
 *              counter equal those of the fixed-G step; only the rows
 *              computed change (rows_total in la_pool_stats_t).  Graph mode
 *              captures one step per row-tile count as it is first needed.
 * temperature  0: greedy verification ([LD] §3.4 "Greedy verification
 *              algorithm (Algorithm 3)").  > 0: sampling verification
 *              ([LD] §3.4 "Sampling verification (Algorithm 4)") against
 *              softmax(logits / temperature); the lookahead branch stays
 *              greedy.  Needs vocab <= 32768.  With LA_AR: plain sampling.
 * top_k      with temperature > 0: only the top_k tokens by logit (ties to
 *              the lower id) keep their weight; 0 means all, and so does a
 *              value >= vocab.  Must be >= 0.
 * top_p      with temperature > 0: of those, only the shortest leading run
 *              (same order) whose weights reach top_p times their sum; 0 or
 *              1 means no cut, otherwise 0 < top_p < 1.  top-K and top-P are
 *              the pages' examples of a sampling target ([LD] §3.4
 *              "Sampling verification"); Algorithm 4 runs on the cut weights.
 *              Both are ignored when temperature is 0.
 * seed       key of the step's draws (Philox4x32-10, counter = (step, draw
 *              index); see la_philox_uniform).
 * reserved   must be 0.
 * A zero-initialised struct with N, max_ctx and max_new set is valid. */
typedef struct {
  int32_t N, W, G, pool_cap, max_ctx, max_new, eos_id;
  uint32_t flags;
  float temperature;
  int32_t top_k;
  uint64_t seed;
  float top_p;
  uint32_t reserved;
} la_decode_params;

#define LA_PROMPT_REF 1u
#define LA_AR 2u
#define LA_DEBUG_LOGITS 4u
#define LA_NO_GRAPH 8u
#define LA_POOL_LRU 16u
#define LA_POOL_CONTEXT 32u
#define LA_ADAPTIVE_G 64u

/* Statistics since prefill ([LD] §3.4 "Scaling Law": S = tokens / steps). */
typedef struct {
  int64_t steps, tokens;
  int64_t accept_hist[LA_MAX_N + 1]; /* steps that accepted j candidate tokens */
  int64_t pool_ngrams, pool_keys_nonempty;
  int64_t inserts, dup_skips, evictions;
  int64_t gathers_nonempty, cand_total;
  int64_t rows_total; /* block rows the steps' forward passes processed */
} la_pool_stats_t;

typedef struct la_model la_model;
typedef struct la_session la_session;

/* Packed bf16 weight layout (what la_model_load and la_kernel_gemm take for
 * the projection and LM-head matrices of bf16 models).  A row-major
 * W[N][K] (K a multiple of 64) is cut into S = ceil(N/16) stripes of 16 rows
 * and into column blocks of 8 stripes (128 rows; the last block holds the
 * ns(b) = min(8, S - 8b) stripes left).  For block b, K chunk c (of 64) and
 * stripe t < ns(b) of the block (stripe s = 8b + t), 2048 bytes hold
 *   element (j, lane, e) = W[16s + lane%16][64c + 32j + 8(lane/16) + e]
 * at byte offset (b*(K/64)*8 + c*ns(b) + t)*2048 + j*1024 + lane*16 + e*2,
 * for j in {0,1}, lane in [0,64), e in [0,8); rows >= N are zero.  Every
 * 1 KB is one MFMA B operand of 64 lanes.  A (block, chunk) unit is one
 * contiguous run, and units follow in block-major order, the order in which
 * the GEMM deals them to its workgroups, so each workgroup reads one
 * contiguous range.  Total ceil(N/16)*16*K*2 bytes. */
size_t la_packed_bytes(int32_t N, int32_t K);
/* Pack a row-major bf16 W[N][K] (device) into `dst` (device, la_packed_bytes
 * bytes).  Enqueued on `hip_stream`. */
int la_pack_weight(const void* src, int32_t N, int32_t K, void* dst, void* hip_stream);

/* Register a model.  `dev_weights` holds n_weights = 3 + 9*n_layers device
 * pointers, owned by the caller, in this order:
 *   emb [vocab][d], then per layer: attn_norm [d], wq [H*hd][d],
 *   wk [Hkv*hd][d], wv [Hkv*hd][d], wo [d][H*hd], mlp_norm [d],
 *   wg [d_ff][d], wu [d_ff][d], wd [d][d_ff], then final_norm [d],
 *   lm_head [vocab][d].
 * fp32 models: matrices row-major [out][in].  bf16 models: wq, wk, wv, wo,
 * wg, wu, wd and lm_head in the packed layout above (la_pack_weight); emb
 * and the norm gains row-major.  They must stay valid until la_model_free.
 * Every model needs d a multiple of 64 (at most 16384), head_dim 16, 32, 64
 * or 128, and H a multiple of Hkv; bf16 models also need H*hd, Hkv*hd and
 * d_ff multiples of 128.  LA_EINVAL otherwise.  *out receives a
 * library-owned handle. */
int la_model_load(const la_model_desc* d, const void* const* dev_weights, int n_weights,
                  void* hip_stream, la_model** out);
void la_model_free(la_model* m);

/* Device workspace bytes a session with these parameters needs (pure host
 * computation; no device call). */
int la_session_bytes(const la_model* m, const la_decode_params* p, size_t* bytes);

/* Prefill ([LD] §3.4: the prompt x0 is the verified prefix).
 * prompt: host pointer, n_prompt >= 1 tokens in [0, vocab).  The first
 *   n_prompt-1 tokens are run causally into the KV cache; the last becomes
 *   the current token.
 * init_window: host pointer to (N-1)*W ids, level-major (level 0 = oldest),
 *   or NULL for all zeros.  Ignored with LA_AR.
 * dev_workspace: device pointer of ws_bytes >= la_session_bytes(); owned by
 *   the caller, must outlive the session, and must not be shared by two
 *   live sessions.
 * Host arrays are copied before return.  The call returns after the prefill
 * has been enqueued and (unless LA_NO_GRAPH) the step graph captured; it
 * synchronises the stream.  *out receives a library-owned session. */
int la_prefill(la_model* m, const la_decode_params* p, const int32_t* prompt, int32_t n_prompt,
               const int32_t* init_window, void* dev_workspace, size_t ws_bytes,
               void* hip_stream, la_session** out);

/* One lookahead decoding step: candidate gather, one forward pass over
 * M = 1 + (W+G)(N-1) rows under the lookahead mask ([LD] §3.4 "The custom
 * attention mask (Figure 2)"), greedy verification (Algorithm 3) or, with a
 * temperature, sampling verification (Algorithm 4), KV commit, window slide
 * and pool insert.  Blocks until the emitted tokens
 * are on the host.
 * out_tokens: host pointer with room for out_cap >= N ids.
 * *n_out: tokens written (1..N while decoding; fewer on the last step).
 * Returns LA_OK, LA_DONE (budget or EOS reached by this or an earlier
 * step; *n_out may be > 0), LA_ECTX (no device work done), or an error. */
int la_step(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out);

/* Per-kernel-class timing of one step (benchmark hook). */
enum {
  LA_PROF_GEMM = 0,   /* QKV, O, gate/up, down projections            */
  LA_PROF_LMHEAD,     /* LM-head GEMM                                 */
  LA_PROF_ATTN,       /* lookahead attention                          */
  LA_PROF_NORM,       /* RMSNorm, embedding                           */
  LA_PROF_EPI,        /* split-K reduce / RoPE / SiLU / residual      */
  LA_PROF_ARGMAX,     /* per-row argmax                               */
  LA_PROF_BOOK,       /* gather, verify + window + pool, KV commit    */
  LA_PROF_KINDS
};
typedef struct {
  int32_t launches[LA_PROF_KINDS];
  double ms[LA_PROF_KINDS];     /* summed kernel durations (device clock) */
  double bytes[LA_PROF_KINDS];  /* algorithmic HBM bytes of those launches */
  double flops[LA_PROF_KINDS];  /* algorithmic FLOPs of those launches     */
} la_profile_t;

/* la_step with every kernel launched eagerly, each launch's kernels timed by
 * a pair of hipEvents bound to their own start and end (hipExtLaunchKernel),
 * so gaps between launches are not counted; *prof receives the per-class
 * sums.  Same kernels, grids and arguments as the graph replay.  Algorithmic bytes:
 * GEMM = weights + input rows + fp32 output rows; attention = committed K/V
 * read once per KV head + block K/V + q + output. */
int la_step_profile(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out,
                    la_profile_t* prof);

/* Counters since prefill; synchronises the session's stream. */
int la_pool_stats(const la_session* s, la_pool_stats_t* out);

/* fp32 logits of the last step's M rows (rows <= M), row-major [rows][vocab],
 * copied to the host pointer `out`.  Test hook.  LA_ESTATE for a bf16 session
 * without LA_DEBUG_LOGITS that does not sample (it keeps no logits). */
int la_debug_logits(const la_session* s, float* out, int32_t rows);

/* One step, as la_step, run eagerly with a copy of every intermediate of
 * the forward pass appended to the device buffer `dev_trace` (test hook:
 * lets a checker re-run each layer from the engine's own inputs).  Layout,
 * contiguous, with es = 2 (bf16) or 4 (fp32), M rows, "dt" = model dtype:
 *   int32 header[16] = {P, M, max_ctx, L, d, H, Hkv, hd, d_ff, vocab, dtype}
 *   int32 ids[M], int32 pos[M]                    row tokens and positions
 *   K cache, V cache before the step, each [L][Hkv][max_ctx][hd] dt
 *   per layer l: x_in f32[M][d], h1 dt[M][d], q dt[M][H*hd] (after RoPE),
 *                attn_out dt[M][H*hd], x_mid f32[M][d], h2 dt[M][d],
 *                act dt[M][d_ff]
 *   x_final f32[M][d], h_final dt[M][d]
 *   block K, block V, each [L][M][Hkv][hd] dt (after RoPE for K)
 *   logits f32[M][vocab]
 * The buffer is caller-owned device memory of at least
 * la_step_trace_bytes() bytes (LA_ENOMEM otherwise).  Returns as la_step. */
int la_step_trace(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out,
                  void* dev_trace, size_t bytes);
int la_step_trace_bytes(const la_session* s, size_t* bytes);

/* Rows in one step (M = 1 + (W+G)(N-1)) of this session; with LA_ADAPTIVE_G
 * the most rows a step processes. */
int la_session_rows(const la_session* s, int32_t* rows);

void la_session_free(la_session* s);

const char* la_last_error(void);

/* The step's attention on its own (test / benchmark hook), for one layer:
 * every block row q attends to the committed prefix [0, P) and to the block
 * rows the lookahead mask lets it see.
 *   q       [M][H*hd]          device, dtype
 *   k_cache, v_cache [Hkv][ld_ctx][hd]  device, dtype; positions [0, P) used
 *   k_blk, v_blk     [M][Hkv*hd]        device, dtype
 *   out     [M][H*hd]          device, dtype (written)
 * with M = 1 + (W+G)(N-1), formed in 64-bit arithmetic; LA_EINVAL unless
 * 1 <= M <= 2048.  Row positions are P + offset (row layout of la_step).
 * ws: device scratch of ws_bytes >= la_kernel_attention_ws_bytes.
 * Enqueued on `hip_stream`; does not synchronise. */
int la_kernel_attention(const void* q, const void* k_cache, const void* v_cache, int32_t P,
                        int32_t ld_ctx, const void* k_blk, const void* v_blk, void* out,
                        int32_t H, int32_t Hkv, int32_t hd, int32_t N, int32_t W, int32_t G,
                        int32_t dtype, void* ws, size_t ws_bytes, void* hip_stream);
/* Device scratch bytes la_kernel_attention needs (partial softmax states of
 * the committed-prefix chunks); 0 when it needs none or when the arguments
 * are out of range (1 + (W+G)(N-1) outside [1, 2048], N outside [2, 16]). */
size_t la_kernel_attention_ws_bytes(int32_t ld_ctx, int32_t H, int32_t hd, int32_t N, int32_t W,
                                    int32_t G, int32_t dtype);

/* The projection GEMM on its own (test / benchmark hook):
 * y[m][n] = sum_k x[m][k] * w[n][k] in fp32, with the same split and
 * summation order the step uses for an N x K weight.
 *   x [M][K] device, dtype; w device: packed (bf16) or [N][K] (fp32);
 *   y [M][N] device fp32 (written);
 *   ws device scratch of ws_bytes >= la_kernel_gemm_ws_bytes(M, K, N).
 * M >= 1; K a multiple of 64 for bf16.  Enqueued on `hip_stream`. */
int la_kernel_gemm(const void* x, int32_t M, int32_t K, const void* w, int32_t N, float* y,
                   int32_t dtype, void* ws, size_t ws_bytes, void* hip_stream);
size_t la_kernel_gemm_ws_bytes(int32_t M, int32_t K, int32_t N);

/* la_kernel_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same product, split and summation order, so y is bit-identical to
 * la_kernel_gemm's, but its partial sums live in a scratch array the library
 * holds in every GPU's memory for the life of the process
 * (LA_NOALLOC_SCRATCH_BYTES per GPU).  It allocates nothing: no hipMalloc,
 * hipFree or allocating library call; the caller passes x, w and y as for
 * la_kernel_gemm.  LA_ENOMEM when la_kernel_gemm_ws_bytes(M, K, N) exceeds
 * LA_NOALLOC_SCRATCH_BYTES; LA_EINVAL on bad arguments; LA_EHIP when the
 * scratch array cannot be located on the current device.  Every call on one
 * GPU uses that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  The array
 * keeps the last call's partial sums.  Enqueued on `hip_stream`. */
#define LA_NOALLOC_SCRATCH_BYTES 33554432
int la_kernel_gemm_noalloc(const void* x, int32_t M, int32_t K, const void* w, int32_t N, float* y,
                           int32_t dtype, void* hip_stream);

/* The draws of sampling verification (test hook): out[i] = draw i of step
 * `step` under `seed`, i < n: word 0 of Philox4x32-10 (Salmon et al., "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC 2011) at counter (step mod 2^32,
 * step >> 32, i, 0) and key (seed mod 2^32, seed >> 32), mapped to
 * ((word >> 8) + 1) / 2^24 in (0, 1].  out: device, n floats.  Enqueued on
 * `hip_stream`. */
int la_philox_uniform(uint64_t seed, uint64_t step, int32_t n, float* out, void* hip_stream);

/* HBM read probe (benchmark hook): reads `bytes` (a multiple of 16) from the
 * device buffer `buf` across the whole chip (each wave one contiguous slice,
 * 16-byte non-temporal loads, 32 KB in flight per wave) and writes one XOR
 * checksum word per workgroup to `out` (device, LA_PROBE_BLOCKS uint32);
 * measures the achievable read bandwidth.  Enqueued on `hip_stream`. */
#define LA_PROBE_BLOCKS 256
int la_probe_read(const void* buf, size_t bytes, uint32_t* out, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
