// C-ABI and host engine of the lookahead decoding step (see include/la.h).
//
// A session's whole state -- KV cache, block K/V, activations, the n-gram
// pool, the window, the RoPE table and the decoding state -- lives in the
// caller's device workspace.  One step is a fixed kernel sequence whose sizes
// depend only on the decode parameters (the committed length P and the
// current token are read on the device), so the sequence is captured once
// into a HIP graph and replayed per step; the only device->host traffic per
// step is the few emitted tokens.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "la_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define LA_HIP(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(LA_EHIP, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

bool debug_sync() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("LA_DEBUG_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

struct LayerW {
  const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *wg, *wu, *wd;
};

size_t dtype_size(int dt) { return dt == LA_BF16 ? 2 : 4; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Scratch of la_kernel_gemm_noalloc: one copy in every GPU's memory for the
// life of the process.  Host code never uses the array's name as an address
// (on the host it is a stand-in, not device memory): it takes the device
// address that hipGetSymbolAddress returns, once per device, with that
// device current.
static __device__ __align__(256) char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LA_EHIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LA_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LA_OK;
}

}  // namespace

struct la_model {
  la_model_desc d;
  const void* emb;
  std::vector<LayerW> layers;
  const void* final_norm;
  const void* lm_head;
  hipStream_t stream;
};

namespace {

// Workspace carve-up, shared by la_session_bytes (sizes only) and la_prefill.
struct WsPlan {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

struct Views {
  size_t x, h, q, att, att_part, act, part, logits, amax, amax_keys, sw, sz, kc, vc, kb, vb, rope,
      pool_tok, pool_cnt, pool_head, pool_ctx, win, cand, ids, pos, prompt, st, total;
};

struct Shape {
  int L, d, H, Hkv, hd, F, V, dt;
  int M, rows_cap, ld_ctx;
  int N, W, G, cap, lru, by_ctx;
  int sampling;  // temperature > 0: the sampling weights buffers exist
  SplitPlan sp_qkv, sp_o, sp_gu, sp_d, sp_lm;
  double pc_qkv, pc_o, pc_gu, pc_d;  // mean pieces per column block (profile bytes)
  int att_mfma, att_nsplit;  // MFMA-attention prefix chunks (0 = per-row kernel only)
};

Shape make_shape(const la_model* m, const la_decode_params* p) {
  Shape s;
  const la_model_desc& d = m->d;
  s.L = d.n_layers; s.d = d.d_model; s.H = d.n_heads; s.Hkv = d.n_kv_heads; s.hd = d.head_dim;
  s.F = d.d_ff; s.V = d.vocab; s.dt = d.dtype;
  const bool ar = (p->flags & LA_AR) != 0;
  s.N = p->N;
  s.W = ar ? 0 : p->W;
  s.G = ar ? 0 : p->G;
  s.cap = p->pool_cap > 0 ? p->pool_cap : (s.G > 0 ? s.G : 1);
  s.lru = (p->flags & LA_POOL_LRU) != 0;
  s.by_ctx = (p->flags & LA_POOL_CONTEXT) != 0;
  s.sampling = p->temperature > 0.f;
  s.M = 1 + (s.W + s.G) * (s.N - 1);
  s.ld_ctx = p->max_ctx;
  s.rows_cap = s.M > p->max_ctx ? s.M : p->max_ctx;
  const int nqkv = (s.H + 2 * s.Hkv) * s.hd;
  s.sp_qkv = gemm_plan(nqkv, s.d, s.dt);
  s.sp_o = gemm_plan(s.d, s.H * s.hd, s.dt);
  s.sp_gu = gemm_plan(2 * s.F, s.d, s.dt);
  s.sp_d = gemm_plan(s.d, s.F, s.dt);
  // the LM head writes the logits directly: whole column blocks, one piece
  s.sp_lm = gemm_plan_whole(s.V, s.d);
  auto mean_pieces = [](const SplitPlan& p) {
    double t = 0;
    for (int b = 0; b < p.nblk; ++b) t += p.np > 1 ? plan_pieces(p, b) : 1;
    return t / p.nblk;
  };
  s.pc_qkv = mean_pieces(s.sp_qkv);
  s.pc_o = mean_pieces(s.sp_o);
  s.pc_gu = mean_pieces(s.sp_gu);
  s.pc_d = mean_pieces(s.sp_d);
  s.att_mfma = attn_uses_mfma(s.dt, s.hd);
  s.att_nsplit = s.att_mfma ? attn_nchunks(s.ld_ctx) : 0;
  return s;
}

Views plan_views(const Shape& s) {
  WsPlan w;
  Views v;
  const size_t es = dtype_size(s.dt);
  const size_t R = (size_t)s.rows_cap;
  const int nqkv = (s.H + 2 * s.Hkv) * s.hd;
  size_t part = 0;
  auto upd = [&](const SplitPlan& sp, int N) {
    const size_t b = (size_t)sp.np * R * N * 4;
    if (b > part) part = b;
  };
  upd(s.sp_qkv, nqkv);
  upd(s.sp_o, s.d);
  upd(s.sp_gu, 2 * s.F);
  upd(s.sp_d, s.d);
  v.x = w.take(R * s.d * 4);
  v.h = w.take(R * s.d * es);
  v.q = w.take(R * s.H * s.hd * es);
  v.att = w.take(R * s.H * s.hd * es);
  v.att_part = w.take((s.att_mfma ? attn_part_floats(s.att_nsplit, (int)R, s.H, s.hd) : 1) * 4);
  v.act = w.take(R * s.F * es);
  v.part = w.take(part);
  v.logits = w.take((size_t)s.M * s.V * 4);
  v.amax = w.take((size_t)s.M * 4);
  v.amax_keys = w.take((size_t)s.M * s.sp_lm.nblk * 8);
  // sampling weights of row 0 and the verification rows (sampling sessions)
  const size_t nsw = s.sampling ? 1 + (size_t)s.G * (s.N - 1) : 0;
  v.sw = w.take(nsw * s.V * 4);
  v.sz = w.take(nsw * 4);
  const size_t kvb = (size_t)s.L * s.Hkv * s.ld_ctx * s.hd * es;
  v.kc = w.take(kvb);
  v.vc = w.take(kvb);
  const size_t blk = (size_t)s.L * s.M * s.Hkv * s.hd * es;
  v.kb = w.take(blk);
  v.vb = w.take(blk);
  v.rope = w.take((size_t)s.ld_ctx * (s.hd / 2) * sizeof(float2));
  const int n1 = s.N - 1;
  v.pool_tok = w.take((size_t)s.V * s.cap * n1 * 4);
  v.pool_cnt = w.take((size_t)s.V * 4);
  v.pool_head = w.take((size_t)s.V * 4);
  v.pool_ctx = w.take((size_t)s.V * s.cap * 4);
  v.win = w.take((size_t)(s.W * n1 > 0 ? s.W * n1 : 1) * 4);
  v.cand = w.take((size_t)(s.G * n1 > 0 ? s.G * n1 : 1) * 4);
  v.ids = w.take(R * 4);
  v.pos = w.take(R * 4);
  v.prompt = w.take(R * 4 + 4);
  v.st = w.take(sizeof(DevState));
  v.total = w.off;
  return v;
}

int check_params(const la_model* m, const la_decode_params* p) {
  if (!m || !p) return fail(LA_EINVAL, "null model or params");
  const bool ar = (p->flags & LA_AR) != 0;
  if (p->N < 2 || p->N > LA_MAX_N) return fail(LA_EINVAL, "N must be in [2, 16]");
  if (!ar && (p->W < 0 || p->G < 0)) return fail(LA_EINVAL, "W and G must be >= 0");
  if (p->pool_cap < 0 || p->pool_cap > 4096) return fail(LA_EINVAL, "pool_cap out of range");
  if (!ar && p->G > 1024) return fail(LA_EINVAL, "G must be <= 1024");
  if (p->max_ctx < 2) return fail(LA_EINVAL, "max_ctx must be >= 2");
  if (p->max_new < 1) return fail(LA_EINVAL, "max_new must be >= 1");
  if (p->eos_id >= m->d.vocab) return fail(LA_EINVAL, "eos_id out of range");
  if (p->flags & ~(LA_PROMPT_REF | LA_AR | LA_NO_GRAPH | LA_POOL_LRU | LA_POOL_CONTEXT |
                   LA_ADAPTIVE_G | LA_DEBUG_LOGITS))
    return fail(LA_EINVAL, "unknown flags");
  const long long W = ar ? 0 : p->W, G = ar ? 0 : p->G;
  const long long M = 1 + (W + G) * (p->N - 1);
  if (M > 2048) return fail(LA_EINVAL, "1 + (W+G)(N-1) must be <= 2048");
  if (p->reserved != 0) return fail(LA_EINVAL, "reserved must be 0");
  if (p->top_k < 0) return fail(LA_EINVAL, "top_k must be >= 0");
  if (!(p->top_p >= 0.f && p->top_p <= 1.f)) return fail(LA_EINVAL, "top_p must be in [0, 1]");
  if (!(p->temperature >= 0.f) || !std::isfinite(p->temperature))
    return fail(LA_EINVAL, "temperature must be finite and >= 0");
  if (p->temperature > 0.f && m->d.vocab > SAMPLE_VMAX)
    return fail(LA_EINVAL, "sampling needs vocab <= 32768");
  return LA_OK;
}

}  // namespace

struct la_session {
  la_model* m = nullptr;
  la_decode_params p{};
  Shape s{};
  Views v{};
  char* base = nullptr;
  hipStream_t stream = nullptr;
  RowLayout lay{};  // layout of the step being enqueued
  // captured steps, one per verification width G' (all G' = G without
  // LA_ADAPTIVE_G)
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  long long rows_total = 0;
  DevState* host_st = nullptr;  // pinned
  // per-launch event timing (la_step_profile)
  struct ProfRec {
    int kind;
    hipEvent_t a, b;
    double bytes, flops;
  };
  bool prof_on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> evs;
  size_t ev_next = 0;
  hipEvent_t next_event() {
    if (ev_next == evs.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      evs.push_back(e);
    }
    return evs[ev_next++];
  }
  // la_step_trace: destination of the per-layer copies, null otherwise
  char* trace = nullptr;
  size_t trace_off = 0;
  int P_host = 0;
  double sum_off = 0;  // sum over block rows of (position - P)
  int total = 0;
  bool done = false;
  bool poisoned = false;

  template <typename T = void>
  T* at(size_t off) const { return (T*)(base + off); }
};

KernelTimer& kernel_timer() {
  static thread_local KernelTimer t;
  return t;
}

namespace {

// Whether every step leaves the logits in the workspace (la_debug_logits).
bool session_keeps_logits(const la_session* ss) {
  return ss->s.dt != LA_BF16 || (ss->p.flags & LA_DEBUG_LOGITS) || ss->p.temperature > 0.f;
}

hipError_t launch_checked(hipError_t e, const char* what, hipStream_t st) {
  if (e != hipSuccess) return e;
  if (debug_sync()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipStreamIsCapturing(st, &cs);
    if (cs == hipStreamCaptureStatusNone) {
      e = hipStreamSynchronize(st);
      if (e != hipSuccess) fprintf(stderr, "[la] %s: %s\n", what, hipGetErrorString(e));
    }
  }
  return e;
}

#define LA_K(expr, what)                                                          \
  do {                                                                            \
    hipError_t e_ = launch_checked((expr), what, st);                             \
    if (e_ != hipSuccess)                                                         \
      return fail(LA_EHIP, std::string(what) + ": " + hipGetErrorString(e_));     \
  } while (0)

// LA_K with the kernels of the launch timed by events bound to them when the
// session profiles (KernelTimer); a launch that ran no kernel is not counted.
#define LA_KP(kind, bytes, flops, expr, what)                                     \
  do {                                                                            \
    KernelTimer& kt_ = kernel_timer();                                            \
    if (ss->prof_on) {                                                            \
      kt_.start = ss->next_event();                                               \
      kt_.stop = ss->next_event();                                                \
      kt_.started = false;                                                        \
      if (!kt_.start || !kt_.stop) {                                              \
        kt_ = KernelTimer{};                                                      \
        return fail(LA_EHIP, "hipEventCreate failed");                            \
      }                                                                           \
    }                                                                             \
    const hipEvent_t a_ = kt_.start, b_ = kt_.stop;                               \
    const hipError_t e_ = launch_checked((expr), what, st);                       \
    const bool timed_ = kt_.started;                                              \
    kt_ = KernelTimer{};                                                          \
    if (e_ != hipSuccess)                                                         \
      return fail(LA_EHIP, std::string(what) + ": " + hipGetErrorString(e_));     \
    if (ss->prof_on && timed_)                                                    \
      ss->recs.push_back({kind, a_, b_, (double)(bytes), (double)(flops)});       \
  } while (0)

// la_step_trace: append `bytes` from device memory `src` to the trace.
hipError_t trace_copy(la_session* ss, const void* src, size_t bytes) {
  if (!ss->trace) return hipSuccess;
  hipError_t e = hipMemcpyAsync(ss->trace + ss->trace_off, src, bytes, hipMemcpyDeviceToDevice,
                                ss->stream);
  ss->trace_off += bytes;
  return e;
}

// The decoder forward over `rows` rows whose token ids and positions are on
// the device.  mode_prefill: K/V are written straight to the cache at each
// row's position and attention is causal over the cache; otherwise K/V go to
// the block buffers and attention follows the lookahead mask.
int enqueue_forward(la_session* ss, int rows, bool mode_prefill) {
  const Shape& s = ss->s;
  const la_model* m = ss->m;
  hipStream_t st = ss->stream;
  const int dt = s.dt;
  const size_t es = dtype_size(dt);
  float* x = ss->at<float>(ss->v.x);
  void* h = ss->at(ss->v.h);
  void* q = ss->at(ss->v.q);
  void* att = ss->at(ss->v.att);
  void* act = ss->at(ss->v.act);
  float* part = ss->at<float>(ss->v.part);
  const int32_t* ids = ss->at<int32_t>(ss->v.ids);
  const int32_t* pos = ss->at<int32_t>(ss->v.pos);
  const int nqkv = (s.H + 2 * s.Hkv) * s.hd;
  const float eps = m->d.norm_eps;

  const double R = rows, D = s.d, ES = (double)es;
  auto gemm_bytes = [&](double N, double K) { return (N * K + R * K) * ES + R * N * 4.0; };
  // attention: committed keys visible to every row, plus per-row offsets
  double P_att = mode_prefill ? 0.0 : (double)ss->P_host;
  double kv_pos = mode_prefill ? R : P_att;
  double att_keys = mode_prefill ? R * (R + 1) / 2 : R * (P_att + 1) + ss->sum_off;
  const double att_bytes = 2.0 * kv_pos * s.Hkv * s.hd * ES +
                           (mode_prefill ? 0.0 : 2.0 * R * s.Hkv * s.hd * ES) +
                           2.0 * R * s.H * s.hd * ES;
  const double att_flops = 4.0 * s.H * s.hd * att_keys;
  LA_KP(LA_PROF_NORM, R * D * (ES + 4.0), 0, launch_embed(ids, m->emb, x, rows, s.d, dt, st),
        "embed");
  LA_KP(LA_PROF_NORM, R * D * (ES + 4.0), 0,
        launch_rmsnorm(x, m->layers[0].attn_norm, h, rows, s.d, eps, dt, st), "rmsnorm_attn");
  const size_t xrow = (size_t)rows * s.d * 4, hrow = (size_t)rows * s.d * es;
  const size_t qrow = (size_t)rows * s.H * s.hd * es;
  for (int l = 0; l < s.L; ++l) {
    LA_K(trace_copy(ss, x, xrow), "trace");
    LA_K(trace_copy(ss, h, hrow), "trace");
    const LayerW& w = m->layers[l];
    char* kc = ss->at<char>(ss->v.kc) + (size_t)l * s.Hkv * s.ld_ctx * s.hd * es;
    char* vc = ss->at<char>(ss->v.vc) + (size_t)l * s.Hkv * s.ld_ctx * s.hd * es;
    char* kb = ss->at<char>(ss->v.kb) + (size_t)l * s.M * s.Hkv * s.hd * es;
    char* vb = ss->at<char>(ss->v.vb) + (size_t)l * s.M * s.Hkv * s.hd * es;

    GemmDesc g{};
    g.x = h; g.rows = rows; g.rows_pad = rows; g.K = s.d; g.nseg = 3;
    g.seg[0] = {w.wq, s.H * s.hd};
    g.seg[1] = {w.wk, s.Hkv * s.hd};
    g.seg[2] = {w.wv, s.Hkv * s.hd};
    g.N = nqkv; g.sp = s.sp_qkv; g.part = part;
    LA_KP(LA_PROF_GEMM, gemm_bytes(nqkv, s.d), 2.0 * R * nqkv * s.d, launch_gemm(g, dt, st),
          "gemm_qkv");
    QkvEpi e{};
    e.part = part; e.sp = s.sp_qkv; e.rows_pad = rows; e.N = nqkv; e.rows = rows;
    e.H = s.H; e.Hkv = s.Hkv; e.hd = s.hd; e.pos = pos;
    e.rope = ss->at<float2>(ss->v.rope); e.q = q;
    e.kdst = mode_prefill ? (void*)kc : (void*)kb;
    e.vdst = mode_prefill ? (void*)vc : (void*)vb;
    e.dest = mode_prefill ? QKV_TO_CACHE : QKV_TO_BLOCK;
    e.ld_ctx = s.ld_ctx;
    LA_KP(LA_PROF_EPI, R * nqkv * (4.0 * s.pc_qkv + ES), 0, launch_qkv_epi(e, dt, st), "qkv_epi");
    LA_K(trace_copy(ss, q, qrow), "trace");

    AttnDesc a{};
    a.q = q; a.kc = kc; a.vc = vc; a.kb = kb; a.vb = vb; a.out = att; a.pos = pos;
    a.Pdev = mode_prefill ? nullptr : &ss->at<DevState>(ss->v.st)->P;
    a.P_host = 0;
    a.rows = rows; a.H = s.H; a.Hkv = s.Hkv; a.hd = s.hd; a.ld_ctx = s.ld_ctx;
    a.causal_cache = mode_prefill ? 1 : 0;
    a.lay = ss->lay;
    a.D = s.N - 1;
    a.mfma = s.att_mfma;
    a.nsplit = s.att_nsplit;
    if (a.mfma) {
      a.part_o = ss->at<float>(ss->v.att_part);
      a.part_ml = a.part_o + (size_t)a.nsplit * rows * s.H * s.hd;
    }
    LA_KP(LA_PROF_ATTN, att_bytes, att_flops, launch_attention(a, dt, st), "attention");
    LA_K(trace_copy(ss, att, qrow), "trace");

    g = GemmDesc{};
    g.x = att; g.rows = rows; g.rows_pad = rows; g.K = s.H * s.hd; g.nseg = 1;
    g.seg[0] = {w.wo, s.d}; g.N = s.d; g.sp = s.sp_o; g.part = part;
    LA_KP(LA_PROF_GEMM, gemm_bytes(s.d, s.H * s.hd), 2.0 * R * s.d * s.H * s.hd,
          launch_gemm(g, dt, st), "gemm_o");
    LA_KP(LA_PROF_EPI, R * D * (4.0 * s.pc_o + 8.0 + ES), 0,
          launch_resid_norm(part, s.sp_o, rows, s.d, rows, x, w.mlp_norm, h, eps, dt, st),
          "resid_o_norm");
    LA_K(trace_copy(ss, x, xrow), "trace");
    LA_K(trace_copy(ss, h, hrow), "trace");

    g = GemmDesc{};
    g.x = h; g.rows = rows; g.rows_pad = rows; g.K = s.d; g.nseg = 2;
    g.seg[0] = {w.wg, s.F}; g.seg[1] = {w.wu, s.F};
    g.N = 2 * s.F; g.sp = s.sp_gu; g.part = part;
    LA_KP(LA_PROF_GEMM, gemm_bytes(2.0 * s.F, s.d), 2.0 * R * 2.0 * s.F * s.d,
          launch_gemm(g, dt, st), "gemm_gate_up");
    LA_KP(LA_PROF_EPI, R * s.F * (8.0 * s.pc_gu + ES), 0,
          launch_silu_epi(part, s.sp_gu, rows, s.F, rows, act, dt, st), "silu_epi");
    LA_K(trace_copy(ss, act, (size_t)rows * s.F * es), "trace");

    g = GemmDesc{};
    g.x = act; g.rows = rows; g.rows_pad = rows; g.K = s.F; g.nseg = 1;
    g.seg[0] = {w.wd, s.d}; g.N = s.d; g.sp = s.sp_d; g.part = part;
    LA_KP(LA_PROF_GEMM, gemm_bytes(s.d, s.F), 2.0 * R * s.d * s.F, launch_gemm(g, dt, st),
          "gemm_down");
    // the next layer's attention norm, or the final norm after the last layer
    const void* gnext = l + 1 < s.L ? m->layers[l + 1].attn_norm : m->final_norm;
    LA_KP(LA_PROF_EPI, R * D * (4.0 * s.pc_d + 8.0 + ES), 0,
          launch_resid_norm(part, s.sp_d, rows, s.d, rows, x, gnext, h, eps, dt, st),
          "resid_down_norm");
  }
  LA_K(trace_copy(ss, x, xrow), "trace");
  LA_K(trace_copy(ss, h, hrow), "trace");
  return LA_OK;
}

int enqueue_step(la_session* ss) {
  const Shape& s = ss->s;
  hipStream_t st = ss->stream;
  const int dt = s.dt;
  PoolDesc pool{ss->at<int32_t>(ss->v.pool_tok), ss->at<int32_t>(ss->v.pool_cnt),
                ss->at<int32_t>(ss->v.pool_head), s.V, s.cap, s.N - 1, s.lru,
                ss->at<int32_t>(ss->v.pool_ctx), s.by_ctx};
  StepIO io{};
  io.st = ss->at<DevState>(ss->v.st);
  io.win = ss->at<int32_t>(ss->v.win);
  io.cand = ss->at<int32_t>(ss->v.cand);
  io.ids = ss->at<int32_t>(ss->v.ids);
  io.pos = ss->at<int32_t>(ss->v.pos);
  io.amax = ss->at<int32_t>(ss->v.amax);
  io.max_new = ss->p.max_new;
  io.eos = ss->p.eos_id;
  io.gmax = s.G;
  io.logits = ss->at<float>(ss->v.logits);
  io.sw = ss->at<float>(ss->v.sw);
  io.sz = ss->at<float>(ss->v.sz);
  io.V = s.V;
  io.temp = ss->p.temperature;
  io.seed = (unsigned long long)ss->p.seed;
  io.top_k = ss->p.top_k < s.V ? ss->p.top_k : 0;
  io.top_p = ss->p.top_p > 0.f && ss->p.top_p < 1.f ? ss->p.top_p : 1.f;

  const int Mc = ss->lay.M;  // rows of this step (the layout's G may be below s.G)
  const double R = Mc, ES = (double)dtype_size(dt);
  LA_KP(LA_PROF_BOOK, 0, 0, launch_gather(pool, io, ss->lay, st), "gather");
  const size_t es = dtype_size(dt);
  const size_t cache_bytes = (size_t)s.L * s.Hkv * s.ld_ctx * s.hd * es;
  const size_t blk_bytes = (size_t)s.L * s.M * s.Hkv * s.hd * es;
  if (ss->trace) {
    int32_t hdr[16] = {ss->P_host, s.M, s.ld_ctx, s.L, s.d, s.H, s.Hkv, s.hd, s.F, s.V, dt};
    LA_K(hipMemcpyAsync(ss->trace, hdr, sizeof(hdr), hipMemcpyHostToDevice, st), "trace");
    LA_K(hipStreamSynchronize(st), "trace");  // hdr is a stack array
    ss->trace_off = sizeof(hdr);
  }
  LA_K(trace_copy(ss, io.ids, (size_t)s.M * 4), "trace");
  LA_K(trace_copy(ss, io.pos, (size_t)s.M * 4), "trace");
  LA_K(trace_copy(ss, ss->at(ss->v.kc), cache_bytes), "trace");
  LA_K(trace_copy(ss, ss->at(ss->v.vc), cache_bytes), "trace");
  int rc = enqueue_forward(ss, Mc, false);
  if (rc != LA_OK) return rc;
  LA_K(trace_copy(ss, ss->at(ss->v.kb), blk_bytes), "trace");
  LA_K(trace_copy(ss, ss->at(ss->v.vb), blk_bytes), "trace");
  const la_model* m = ss->m;
  float* x = ss->at<float>(ss->v.x);
  void* h = ss->at(ss->v.h);
  GemmDesc g{};
  g.x = h; g.rows = Mc; g.rows_pad = Mc; g.K = s.d; g.nseg = 1;
  g.seg[0] = {m->lm_head, s.V}; g.N = s.V; g.sp = s.sp_lm;
  // bf16: the LM head leaves each row's argmax as one key per 128-column
  // block, and writes the logits only when they are wanted (sampling
  // verification reads them; LA_DEBUG_LOGITS and the trace keep them)
  const bool keys = dt == LA_BF16;
  const bool logits = !keys || session_keeps_logits(ss) || ss->trace;
  g.part = logits ? ss->at<float>(ss->v.logits) : nullptr;
  g.amax_keys = keys ? ss->at<unsigned long long>(ss->v.amax_keys) : nullptr;
  LA_KP(LA_PROF_LMHEAD, ((double)s.V * s.d + R * s.d) * ES + (logits ? R * s.V * 4.0 : 0.0),
        2.0 * R * s.V * s.d, launch_gemm(g, dt, st), "gemm_lm_head");
  LA_K(trace_copy(ss, ss->at(ss->v.logits), (size_t)s.M * s.V * 4), "trace");
  if (keys)
    LA_KP(LA_PROF_ARGMAX, R * s.sp_lm.nblk * 8.0, 0,
          launch_argmax_keys(ss->at<unsigned long long>(ss->v.amax_keys), Mc, s.sp_lm.nblk,
                             ss->at<int32_t>(ss->v.amax), st),
          "argmax");
  else
    LA_KP(LA_PROF_ARGMAX, R * s.V * 4.0, 0,
          launch_argmax(ss->at<float>(ss->v.logits), Mc, s.V, ss->at<int32_t>(ss->v.amax), st),
          "argmax");
  if (io.temp > 0.f) {
    LA_KP(LA_PROF_BOOK, 0, 0, launch_sample_weights(io, ss->lay, st), "sample_weights");
    LA_KP(LA_PROF_BOOK, 0, 0, launch_sample_verify(io, ss->lay, st), "sample_verify");
  }
  LA_KP(LA_PROF_BOOK, 0, 0, launch_verify(pool, io, ss->lay, st), "verify");
  KvCommit c{};
  c.st = io.st;
  c.kb = ss->at(ss->v.kb); c.vb = ss->at(ss->v.vb);
  c.kc = ss->at(ss->v.kc); c.vc = ss->at(ss->v.vc);
  c.L = s.L; c.M = s.M; c.Hkv = s.Hkv; c.hd = s.hd; c.ld_ctx = s.ld_ctx; c.nmax = s.N;
  LA_KP(LA_PROF_BOOK, 0, 0, launch_kv_commit(c, dt, st), "kv_commit");
  return LA_OK;
}

#undef LA_K

int max_offset(const Shape& s) {
  // largest row position relative to P: lookahead rows reach N+W-2, candidate
  // rows N-1
  int off = s.N - 1;
  if (s.W > 0 && s.N + s.W - 2 > off) off = s.N + s.W - 2;
  if (s.G == 0 && s.W == 0) off = 0;
  return off;
}

}  // namespace

extern "C" {

const char* la_last_error(void) { return g_err.c_str(); }

int la_model_load(const la_model_desc* d, const void* const* dev_weights, int n_weights,
                  void* hip_stream, la_model** out) {
  if (!d || !dev_weights || !out) return fail(LA_EINVAL, "null argument");
  *out = nullptr;
  if (d->dtype != LA_F32 && d->dtype != LA_BF16) return fail(LA_EINVAL, "dtype must be LA_F32 or LA_BF16");
  if (d->n_layers < 1 || d->d_model < 1 || d->n_heads < 1 || d->n_kv_heads < 1 || d->d_ff < 1 ||
      d->vocab < 1)
    return fail(LA_EINVAL, "shape fields must be >= 1");
  if (d->n_heads % d->n_kv_heads) return fail(LA_EINVAL, "n_heads must be a multiple of n_kv_heads");
  const int hd = d->head_dim;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return fail(LA_EINVAL, "head_dim must be 16, 32, 64 or 128");
  if (!(d->norm_eps > 0.f) || !(d->rope_theta > 0.f)) return fail(LA_EINVAL, "norm_eps and rope_theta must be > 0");
  // the residual + RMSNorm epilogue gives each row whole waves of columns
  if (d->d_model % 64 || d->d_model > 16384)
    return fail(LA_EINVAL, "d_model must be a multiple of 64, at most 16384");
  if (d->dtype == LA_BF16) {
    const int hq = d->n_heads * hd, hk = d->n_kv_heads * hd;
    if (d->d_model % 64 || hq % 128 || hk % 128 || d->d_ff % 128)
      return fail(LA_EINVAL, "bf16 needs d_model % 64 == 0 and H*hd, Hkv*hd, d_ff multiples of 128");
  }
  if (n_weights != 3 + 9 * d->n_layers) return fail(LA_EINVAL, "n_weights must be 3 + 9*n_layers");
  for (int i = 0; i < n_weights; ++i)
    if (!dev_weights[i]) return fail(LA_EINVAL, "null weight pointer " + std::to_string(i));
  la_model* m = new (std::nothrow) la_model();
  if (!m) return fail(LA_ENOMEM, "host allocation failed");
  m->d = *d;
  m->emb = dev_weights[0];
  m->layers.resize(d->n_layers);
  for (int l = 0; l < d->n_layers; ++l) {
    const void* const* w = dev_weights + 1 + 9 * l;
    m->layers[l] = LayerW{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7], w[8]};
  }
  m->final_norm = dev_weights[1 + 9 * d->n_layers];
  m->lm_head = dev_weights[2 + 9 * d->n_layers];
  m->stream = (hipStream_t)hip_stream;
  *out = m;
  return LA_OK;
}

void la_model_free(la_model* m) { delete m; }

int la_session_bytes(const la_model* m, const la_decode_params* p, size_t* bytes) {
  if (!bytes) return fail(LA_EINVAL, "null bytes");
  int rc = check_params(m, p);
  if (rc != LA_OK) return rc;
  *bytes = plan_views(make_shape(m, p)).total;
  return LA_OK;
}

int la_session_rows(const la_session* s, int32_t* rows) {
  if (!s || !rows) return fail(LA_EINVAL, "null argument");
  *rows = s->s.M;
  return LA_OK;
}

static void session_destroy(la_session* s) {
  if (!s) return;
  for (hipGraphExec_t e : s->execs)
    if (e) hipGraphExecDestroy(e);
  for (hipGraph_t g : s->graphs)
    if (g) hipGraphDestroy(g);
  if (s->host_st) hipHostFree(s->host_st);
  for (hipEvent_t e : s->evs) hipEventDestroy(e);
  delete s;
}

void la_session_free(la_session* s) { session_destroy(s); }

// Capture the step at the session's current layout into a graph (once per
// verification width).
static int capture_step(la_session* ss) {
  const int g = ss->lay.G;
  if (ss->execs[g]) return LA_OK;
  hipStream_t st = ss->stream;
  hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(LA_EHIP, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
  const int rc = enqueue_step(ss);
  hipGraph_t gr = nullptr;
  e = hipStreamEndCapture(st, &gr);
  if (rc != LA_OK) {
    if (gr) hipGraphDestroy(gr);
    return rc;
  }
  if (e != hipSuccess) return fail(LA_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  ss->graphs[g] = gr;
  e = hipGraphInstantiate(&ss->execs[g], gr, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    ss->execs[g] = nullptr;
    return fail(LA_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
  }
  return LA_OK;
}

// Verification width of a step whose gather will take g candidates: the
// most candidates (at most G) whose rows fit the same 16-row tiles.
static int adaptive_width(const Shape& s, int g) {
  const int n1 = s.N - 1;
  const int tiles = (1 + (s.W + g) * n1 + 15) / 16;
  int w = (16 * tiles - 1) / n1 - s.W;
  if (w > s.G) w = s.G;
  return w < g ? g : w;
}

int la_prefill(la_model* m, const la_decode_params* p, const int32_t* prompt, int32_t n_prompt,
               const int32_t* init_window, void* dev_workspace, size_t ws_bytes, void* hip_stream,
               la_session** out) {
  if (!out) return fail(LA_EINVAL, "null out");
  *out = nullptr;
  int rc = check_params(m, p);
  if (rc != LA_OK) return rc;
  if (!prompt || n_prompt < 1) return fail(LA_EINVAL, "prompt must hold >= 1 token");
  if (!dev_workspace) return fail(LA_EINVAL, "null workspace");
  for (int i = 0; i < n_prompt; ++i)
    if (prompt[i] < 0 || prompt[i] >= m->d.vocab) return fail(LA_EINVAL, "prompt token out of range");
  const bool graph = (p->flags & LA_NO_GRAPH) == 0;
  if (graph && !hip_stream) return fail(LA_EINVAL, "graph mode needs a non-null stream");
  Shape s = make_shape(m, p);
  Views v = plan_views(s);
  if (ws_bytes < v.total) return fail(LA_ENOMEM, "workspace too small: need " + std::to_string(v.total));
  if (n_prompt - 1 + max_offset(s) + 1 > p->max_ctx)
    return fail(LA_ECTX, "prompt does not fit max_ctx");
  const int n1 = s.N - 1;
  if (init_window && s.W > 0)
    for (int i = 0; i < s.W * n1; ++i)
      if (init_window[i] < 0 || init_window[i] >= s.V) return fail(LA_EINVAL, "window token out of range");

  la_session* ss = new (std::nothrow) la_session();
  if (!ss) return fail(LA_ENOMEM, "host allocation failed");
  ss->m = m; ss->p = *p; ss->s = s; ss->v = v;
  ss->base = (char*)dev_workspace;
  ss->stream = (hipStream_t)hip_stream;
  ss->lay = RowLayout{s.N, s.W, s.G, s.M};
  for (int l = 0; l < n1; ++l)
    for (int k = 0; k < s.W; ++k) ss->sum_off += 1 + l + k;
  ss->sum_off += (double)s.G * n1 * (n1 + 1) / 2;
  hipStream_t st = ss->stream;

  auto bail = [&](int code) {
    session_destroy(ss);
    return code;
  };
#define LA_PF(expr)                                                                         \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return bail(fail(LA_EHIP, std::string(#expr) + " failed: " + hipGetErrorString(e_))); \
  } while (0)

  LA_PF(hipHostMalloc((void**)&ss->host_st, sizeof(DevState), hipHostMallocDefault));

  // host-side tables and initial state
  std::vector<float2> rope((size_t)s.ld_ctx * (s.hd / 2));
  for (int ps = 0; ps < s.ld_ctx; ++ps)
    for (int i = 0; i < s.hd / 2; ++i) {
      const double inv = std::pow((double)m->d.rope_theta, -2.0 * i / s.hd);
      const double ang = (double)ps * inv;
      rope[(size_t)ps * (s.hd / 2) + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  std::vector<int32_t> iota(n_prompt > 1 ? n_prompt - 1 : 1);
  for (int i = 0; i < (int)iota.size(); ++i) iota[i] = i;
  std::vector<int32_t> win((size_t)(s.W * n1 > 0 ? s.W * n1 : 1), 0);
  if (init_window && s.W > 0) memcpy(win.data(), init_window, (size_t)s.W * n1 * 4);
  DevState h0;
  memset(&h0, 0, sizeof(h0));
  h0.P = n_prompt - 1;
  h0.cur = prompt[n_prompt - 1];
  h0.prev = n_prompt >= 2 ? prompt[n_prompt - 2] : -1;

  LA_PF(hipMemcpyAsync(ss->at(v.rope), rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice, st));
  LA_PF(hipMemcpyAsync(ss->at(v.prompt), prompt, (size_t)n_prompt * 4, hipMemcpyHostToDevice, st));
  LA_PF(hipMemcpyAsync(ss->at(v.ids), prompt, (size_t)(n_prompt > 1 ? n_prompt - 1 : 1) * 4, hipMemcpyHostToDevice, st));
  LA_PF(hipMemcpyAsync(ss->at(v.pos), iota.data(), iota.size() * 4, hipMemcpyHostToDevice, st));
  LA_PF(hipMemcpyAsync(ss->at(v.win), win.data(), win.size() * 4, hipMemcpyHostToDevice, st));
  LA_PF(hipMemcpyAsync(ss->at(v.st), &h0, sizeof(h0), hipMemcpyHostToDevice, st));
  LA_PF(launch_fill_i32(ss->at<int32_t>(v.pool_cnt), 0, (size_t)s.V, st));
  LA_PF(launch_fill_i32(ss->at<int32_t>(v.pool_head), 0, (size_t)s.V, st));
  // the host arrays above are stack/heap locals: finish the copies now
  LA_PF(hipStreamSynchronize(st));

  if (n_prompt > 1) {
    rc = enqueue_forward(ss, n_prompt - 1, true);
    if (rc != LA_OK) return bail(rc);
  }
  if ((p->flags & LA_PROMPT_REF) && s.G > 0 && n_prompt >= s.N) {
    PoolDesc pool{ss->at<int32_t>(v.pool_tok), ss->at<int32_t>(v.pool_cnt),
                  ss->at<int32_t>(v.pool_head), s.V, s.cap, n1, s.lru,
                  ss->at<int32_t>(v.pool_ctx), s.by_ctx};
    LA_PF(launch_pool_seed(pool, ss->at<DevState>(v.st), ss->at<int32_t>(v.prompt), n_prompt, st));
  }
  LA_PF(hipStreamSynchronize(st));

  ss->graphs.assign((size_t)s.G + 1, nullptr);
  ss->execs.assign((size_t)s.G + 1, nullptr);
  if (graph) {
    // every width a step can take, captured now so that no step pays for a
    // capture (with LA_ADAPTIVE_G one per 16-row tile count)
    const bool adaptive = (p->flags & LA_ADAPTIVE_G) != 0;
    for (int g = adaptive ? 0 : s.G; g <= s.G; ++g) {
      const int w = adaptive ? adaptive_width(s, g) : s.G;
      ss->lay = RowLayout{s.N, s.W, w, 1 + (s.W + w) * n1};
      rc = capture_step(ss);
      if (rc != LA_OK) return bail(rc);
    }
    ss->lay = RowLayout{s.N, s.W, s.G, s.M};
  }
  ss->P_host = n_prompt - 1;
  *out = ss;
#undef LA_PF
  return LA_OK;
}

static size_t trace_bytes(const Shape& s) {
  const size_t es = dtype_size(s.dt), M = (size_t)s.M;
  const size_t xrow = M * s.d * 4, hrow = M * s.d * es, qrow = M * s.H * s.hd * es;
  size_t b = 16 * 4 + 2 * M * 4;
  b += 2 * (size_t)s.L * s.Hkv * s.ld_ctx * s.hd * es;
  b += (size_t)s.L * (2 * xrow + 2 * hrow + 2 * qrow + M * s.F * es);
  b += xrow + hrow;
  b += 2 * (size_t)s.L * M * s.Hkv * s.hd * es;
  b += M * s.V * 4;
  return b;
}

static int step_impl(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out,
                     la_profile_t* prof, char* trace = nullptr) {
  if (!s || !out_tokens || !n_out) return fail(LA_EINVAL, "null argument");
  *n_out = 0;
  if (s->poisoned) return fail(LA_ESTATE, "session poisoned by an earlier HIP error");
  if (out_cap < s->s.N) return fail(LA_EINVAL, "out_cap must be >= N");
  if (s->done) return LA_DONE;
  if (s->P_host + max_offset(s->s) + 1 > s->p.max_ctx)
    return fail(LA_ECTX, "context full: step would pass max_ctx");
  int rc = LA_OK;
  // the step's layout: the full width, or with LA_ADAPTIVE_G the width the
  // candidates found for this step's token need (the previous step counted
  // them; the first step takes the full width)
  int gw = s->s.G;
  if ((s->p.flags & LA_ADAPTIVE_G) && !prof && !trace && s->rows_total > 0)
    gw = adaptive_width(s->s, s->host_st->next_g);
  s->lay = RowLayout{s->s.N, s->s.W, gw, 1 + (s->s.W + gw) * (s->s.N - 1)};
  if (prof) {
    s->prof_on = true;
    s->recs.clear();
    s->ev_next = 0;
    rc = enqueue_step(s);
    s->prof_on = false;
  } else if (trace) {
    s->trace = trace;
    s->trace_off = 0;
    rc = enqueue_step(s);
    s->trace = nullptr;
  } else if (!(s->p.flags & LA_NO_GRAPH)) {
    rc = capture_step(s);  // a width not seen yet (LA_ADAPTIVE_G) is captured now
    if (rc == LA_OK) {
      hipError_t e = hipGraphLaunch(s->execs[gw], s->stream);
      if (e != hipSuccess) rc = fail(LA_EHIP, std::string("hipGraphLaunch: ") + hipGetErrorString(e));
    }
  } else {
    rc = enqueue_step(s);
  }
  if (rc == LA_OK) {
    DevState* dst = s->at<DevState>(s->v.st);
    hipError_t e = hipMemcpyAsync(s->host_st, dst, offsetof(DevState, ncand), hipMemcpyDeviceToHost,
                                  s->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(s->stream);
    if (e != hipSuccess) rc = fail(LA_EHIP, std::string("step sync: ") + hipGetErrorString(e));
  }
  if (rc != LA_OK) {
    s->poisoned = true;
    return rc;
  }
  if (prof) {
    memset(prof, 0, sizeof(*prof));
    for (const auto& r : s->recs) {
      float ms = 0.f;
      hipError_t e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e != hipSuccess) {
        s->poisoned = true;
        return fail(LA_EHIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
      }
      prof->launches[r.kind] += 1;
      prof->ms[r.kind] += ms;
      prof->bytes[r.kind] += r.bytes;
      prof->flops[r.kind] += r.flops;
    }
  }
  s->rows_total += s->lay.M;
  const int n = s->host_st->n_out;
  for (int i = 0; i < n; ++i) out_tokens[i] = s->host_st->out[i];
  *n_out = n;
  s->total += n;
  s->P_host = s->host_st->P;
  s->done = s->host_st->done != 0;
  return s->done ? LA_DONE : LA_OK;
}

int la_step(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out) {
  return step_impl(s, out_tokens, out_cap, n_out, nullptr);
}

int la_step_profile(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out,
                    la_profile_t* prof) {
  if (!prof) return fail(LA_EINVAL, "null prof");
  return step_impl(s, out_tokens, out_cap, n_out, prof);
}

int la_step_trace_bytes(const la_session* s, size_t* bytes) {
  if (!s || !bytes) return fail(LA_EINVAL, "null argument");
  *bytes = trace_bytes(s->s);
  return LA_OK;
}

int la_step_trace(la_session* s, int32_t* out_tokens, int32_t out_cap, int32_t* n_out,
                  void* dev_trace, size_t bytes) {
  if (!dev_trace) return fail(LA_EINVAL, "null trace buffer");
  if (!s) return fail(LA_EINVAL, "null session");
  if (bytes < trace_bytes(s->s))
    return fail(LA_ENOMEM, "trace buffer too small: need " + std::to_string(trace_bytes(s->s)));
  return step_impl(s, out_tokens, out_cap, n_out, nullptr, (char*)dev_trace);
}

int la_pool_stats(const la_session* s, la_pool_stats_t* out) {
  if (!s || !out) return fail(LA_EINVAL, "null argument");
  DevState h;
  LA_HIP(hipStreamSynchronize(s->stream));
  LA_HIP(hipMemcpy(&h, s->at<DevState>(s->v.st), sizeof(h), hipMemcpyDeviceToHost));
  memset(out, 0, sizeof(*out));
  out->steps = h.stats[ST_STEPS];
  out->tokens = h.stats[ST_TOKENS];
  for (int i = 0; i <= LA_MAX_N; ++i) out->accept_hist[i] = h.stats[ST_HIST0 + i];
  out->pool_ngrams = h.stats[ST_NGRAMS];
  out->pool_keys_nonempty = h.stats[ST_KEYS];
  out->inserts = h.stats[ST_INSERTS];
  out->dup_skips = h.stats[ST_DUPS];
  out->evictions = h.stats[ST_EVICT];
  out->gathers_nonempty = h.stats[ST_GATHER_NE];
  out->cand_total = h.stats[ST_CAND_TOTAL];
  out->rows_total = s->rows_total;
  return LA_OK;
}

int la_debug_logits(const la_session* s, float* out, int32_t rows) {
  if (!s || !out) return fail(LA_EINVAL, "null argument");
  if (rows < 1 || rows > s->s.M) return fail(LA_EINVAL, "rows must be in [1, M]");
  if (!session_keeps_logits(s))
    return fail(LA_ESTATE, "the session keeps no logits: prefill it with LA_DEBUG_LOGITS");
  LA_HIP(hipStreamSynchronize(s->stream));
  LA_HIP(hipMemcpy(out, s->at(s->v.logits), (size_t)rows * s->s.V * 4, hipMemcpyDeviceToHost));
  return LA_OK;
}

size_t la_kernel_attention_ws_bytes(int32_t ld_ctx, int32_t H, int32_t hd, int32_t N, int32_t W,
                                    int32_t G, int32_t dtype) {
  if (ld_ctx < 0 || H < 1 || N < 2 || N > LA_MAX_N || W < 0 || G < 0) return 0;
  if (!attn_uses_mfma(dtype, hd)) return 0;
  // widen before adding: W + G may not fit an int
  const long long M = 1 + ((long long)W + G) * (N - 1);
  if (M < 1 || M > 2048) return 0;
  const int nsplit = attn_nchunks(ld_ctx);
  return attn_part_floats(nsplit > 0 ? nsplit : 1, (int)M, H, hd) * 4;
}

int la_kernel_attention(const void* q, const void* k_cache, const void* v_cache, int32_t P,
                        int32_t ld_ctx, const void* k_blk, const void* v_blk, void* out, int32_t H,
                        int32_t Hkv, int32_t hd, int32_t N, int32_t W, int32_t G, int32_t dtype,
                        void* ws, size_t ws_bytes, void* hip_stream) {
  if (!q || !k_blk || !v_blk || !out) return fail(LA_EINVAL, "null pointer");
  if (P > 0 && (!k_cache || !v_cache)) return fail(LA_EINVAL, "null cache");
  if (P < 0 || ld_ctx < P) return fail(LA_EINVAL, "need 0 <= P <= ld_ctx");
  if (H < 1 || Hkv < 1 || H % Hkv) return fail(LA_EINVAL, "bad head counts");
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return fail(LA_EINVAL, "bad head_dim");
  if (N < 2 || N > LA_MAX_N || W < 0 || G < 0) return fail(LA_EINVAL, "bad N, W, G");
  if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_EINVAL, "bad dtype");
  const long long M = 1 + ((long long)W + G) * (N - 1);
  if (M < 1 || M > 2048) return fail(LA_EINVAL, "1 + (W+G)(N-1) must be in [1, 2048]");
  AttnDesc a{};
  a.q = q; a.kc = k_cache ? k_cache : k_blk; a.vc = v_cache ? v_cache : v_blk;
  a.kb = k_blk; a.vb = v_blk; a.out = out;
  a.pos = nullptr; a.Pdev = nullptr; a.P_host = P;
  a.rows = (int)M; a.H = H; a.Hkv = Hkv; a.hd = hd; a.ld_ctx = ld_ctx;
  a.causal_cache = 0;
  a.lay = RowLayout{N, W, G, (int)M};
  a.D = N - 1;
  a.mfma = attn_uses_mfma(dtype, hd);
  if (a.mfma) {
    a.nsplit = attn_nchunks(ld_ctx);
    if (a.nsplit < 1) a.nsplit = 1;
    const size_t need = attn_part_floats(a.nsplit, (int)M, H, hd) * 4;
    if (!ws || ws_bytes < need) return fail(LA_ENOMEM, "attention workspace too small");
    a.part_o = (float*)ws;
    a.part_ml = a.part_o + (size_t)a.nsplit * M * H * hd;
  }
  LA_HIP(launch_attention(a, dtype, (hipStream_t)hip_stream));
  return LA_OK;
}

int la_philox_uniform(uint64_t seed, uint64_t step, int32_t n, float* out, void* hip_stream) {
  if (n < 0 || (n > 0 && !out)) return fail(LA_EINVAL, "bad argument");
  LA_HIP(launch_philox_uniform(seed, step, n, out, (hipStream_t)hip_stream));
  return LA_OK;
}

int la_probe_read(const void* buf, size_t bytes, uint32_t* out, void* hip_stream) {
  if (!buf || !out || bytes % 16) return fail(LA_EINVAL, "need buffers and bytes % 16 == 0");
  LA_HIP(launch_probe_read(buf, bytes, out, (hipStream_t)hip_stream));
  return LA_OK;
}

size_t la_packed_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 64 || K % 64) return 0;
  return packed_bytes(N, K);
}

int la_pack_weight(const void* src, int32_t N, int32_t K, void* dst, void* hip_stream) {
  if (!src || !dst) return fail(LA_EINVAL, "null pointer");
  if (N < 1 || K < 64 || K % 64) return fail(LA_EINVAL, "need N >= 1 and K a multiple of 64");
  LA_HIP(launch_pack(src, N, K, dst, (hipStream_t)hip_stream));
  return LA_OK;
}

size_t la_kernel_gemm_ws_bytes(int32_t M, int32_t K, int32_t N) {
  if (M < 1 || K < 1 || N < 1) return 0;
  const SplitPlan sp = gemm_plan(N, K, LA_BF16);
  return sp.np > 1 ? (size_t)sp.np * M * N * 4 : 0;
}

int la_kernel_gemm_noalloc(const void* x, int32_t M, int32_t K, const void* w, int32_t N, float* y,
                           int32_t dtype, void* hip_stream) {
  if (!x || !w || !y) return fail(LA_EINVAL, "null pointer");
  if (M < 1 || K < 1 || N < 1) return fail(LA_EINVAL, "sizes must be >= 1");
  if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_EINVAL, "bad dtype");
  if (dtype == LA_BF16 && K % 64) return fail(LA_EINVAL, "bf16 needs K % 64 == 0");
  const SplitPlan sp = gemm_plan(N, K, dtype);
  const size_t need = sp.np > 1 ? (size_t)sp.np * M * N * 4 : 0;
  if (need > (size_t)LA_NOALLOC_SCRATCH_BYTES)
    return fail(LA_ENOMEM, "partial sums need " + std::to_string(need) +
                               " bytes, beyond the static scratch of " +
                               std::to_string(LA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need) {
    const int rc = scratch_address(&ws);
    if (rc != LA_OK) return rc;
  }
  return la_kernel_gemm(x, M, K, w, N, y, dtype, ws, need, hip_stream);
}

int la_kernel_gemm(const void* x, int32_t M, int32_t K, const void* w, int32_t N, float* y,
                   int32_t dtype, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!x || !w || !y) return fail(LA_EINVAL, "null pointer");
  if (M < 1 || K < 1 || N < 1) return fail(LA_EINVAL, "sizes must be >= 1");
  if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_EINVAL, "bad dtype");
  if (dtype == LA_BF16 && K % 64) return fail(LA_EINVAL, "bf16 needs K % 64 == 0");
  const SplitPlan sp = gemm_plan(N, K, dtype);
  const size_t need = sp.np > 1 ? (size_t)sp.np * M * N * 4 : 0;
  if (ws_bytes < need || (need && !ws)) return fail(LA_ENOMEM, "workspace too small");
  hipStream_t st = (hipStream_t)hip_stream;
  GemmDesc g{};
  g.x = x; g.rows = M; g.rows_pad = M; g.K = K; g.nseg = 1; g.seg[0] = {w, N};
  g.N = N; g.sp = sp; g.part = sp.np > 1 ? (float*)ws : y;
  LA_HIP(launch_gemm(g, dtype, st));
  if (sp.np > 1) LA_HIP(launch_sum_epi((float*)ws, sp, M, N, M, y, st));
  return LA_OK;
}

}  // extern "C"
