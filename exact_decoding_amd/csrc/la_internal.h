// Internal declarations shared by the HIP kernels and the engine.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "la.h"

typedef uint16_t bf16_t;
// native 16-byte vector: HIP's uint4 is a struct whose copies the compiler can
// leave in private memory
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// scalar storage types: fp32 or bf16 (round to nearest even on store)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const bf16_t* p) {
  return __uint_as_float(((uint32_t)*p) << 16);
}
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // finite inputs only
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ void st_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_f(bf16_t* p, float v) { *p = f2bf(v); }

// ---------------------------------------------------------------------------
// kernel launches, with optional per-kernel timing (la_step_profile)
// ---------------------------------------------------------------------------
// While `stop` is set on the calling thread, launches through la_launch bind
// the events to the kernels' own start and end (hipExtLaunchKernelGGL):
// `start` to the first kernel launched, `stop` to the last one, so the
// elapsed time between them is what the kernels took on the device, without
// the gaps that event records between eager launches would add.
struct KernelTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool started = false;
};
KernelTimer& kernel_timer();  // the calling thread's

template <typename F, typename... A>
inline void la_launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, A... args) {
  KernelTimer& t = kernel_timer();
  if (t.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, t.started ? nullptr : t.start, t.stop, 0,
                          args...);
    t.started = true;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  }
}

// ---------------------------------------------------------------------------
// device-resident decoding state (one per session, in the workspace)
// ---------------------------------------------------------------------------
enum {
  ST_INSERTS = 0, ST_DUPS, ST_EVICT, ST_GATHER_NE, ST_CAND_TOTAL, ST_STEPS, ST_TOKENS,
  ST_NGRAMS, ST_KEYS, ST_HIST0, ST_COUNT = ST_HIST0 + LA_MAX_N + 1
};

struct DevState {
  int32_t P;           // committed tokens in the KV cache
  int32_t cur;         // current (last emitted, uncached) token
  int32_t total;       // tokens emitted so far
  int32_t done;        // 1 once max_new or EOS is reached
  int32_t n_out;       // tokens emitted by the last step
  int32_t out[LA_MAX_N];
  int32_t next_g;      // candidates the next step will gather (min(bucket of cur, G))
  int32_t ncand;       // candidates gathered this step
  int32_t commit_p;    // P before the last step's commit
  int32_t commit_n;    // rows committed by the last step
  int32_t commit_rows[LA_MAX_N];
  int32_t prev;        // the token before cur (-1: none)
  int32_t pad_[2];
  long long stats[ST_COUNT];
};

// Static description of a step's block-row layout.
struct RowLayout {
  int N, W, G;   // W = G = 0 for plain autoregressive decoding
  int M;         // 1 + (W + G) * (N - 1)
};

// ---------------------------------------------------------------------------
// GEMM: y_part[p][m][n] = sum over the K range of piece p of x[m][k] * w[n][k]
// ---------------------------------------------------------------------------
// How one product's work is dealt out.  Its units are (column block of 128,
// K chunk of 64) pairs in block-major order, U = nblk * nch of them; workgroup
// w takes units [floor(w U / G), floor((w+1) U / G)), at most nch of them, so
// it covers the tail of one column block and possibly the head of the next.
// The pieces a column block is cut into are summed in K order by the
// epilogue.  The plan depends on (N, K) only, never on the row count, so a
// row gets the same sums at any M.
constexpr int GEMM_NWG = 128;  // output columns of one GEMM column block

struct SplitPlan {
  int nch;   // K / 64
  int nblk;  // column blocks of 128
  int G;     // workgroups per 128-row block
  int np;    // most pieces any column block is cut into (1: no partial sums)
};

// workgroup holding unit u, and the pieces of column block b
__host__ __device__ inline int plan_wg_of(const SplitPlan& p, int u) {
  return (int)(((unsigned)(u + 1) * (unsigned)p.G - 1u) / (unsigned)(p.nblk * p.nch));
}
__host__ __device__ inline int plan_first_wg(const SplitPlan& p, int b) {
  return plan_wg_of(p, b * p.nch);
}
__host__ __device__ inline int plan_pieces(const SplitPlan& p, int b) {
  return plan_wg_of(p, (b + 1) * p.nch - 1) - plan_first_wg(p, b) + 1;
}

struct GemmSeg {
  const void* w;  // [n][K] row-major
  int n;          // rows of this segment
};

struct GemmDesc {
  const void* x;  // [rows][K] row-major (rows padded to a multiple of 128 for bf16)
  int rows;       // valid rows
  int K;
  int nseg;
  GemmSeg seg[3];
  int N;          // total columns (sum of segment rows)
  SplitPlan sp;   // how the (column block, K chunk) units are dealt out
  float* part;    // [sp.np][rows_pad][N]; the output itself when sp.np == 1
                  // (null: no output, with amax_keys)
  int rows_pad;   // leading row count of part
  // whole-block plans (sp.np == 1, bf16): each column block's row maxima as
  // argmax keys, [rows][sp.nblk] (argmax_key); null: none
  unsigned long long* amax_keys;
};

// Order-preserving 64-bit argmax key of logit v at column col: the larger
// key has the larger value, and of equal values the lower column (the
// argmax's ties go to the lowest id); -0 counts as +0.
__host__ __device__ inline unsigned long long argmax_key(float v, int col) {
  unsigned int u;
  __builtin_memcpy(&u, &v, 4);
  if ((u << 1) == 0u) u = 0u;
  const unsigned int ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (unsigned int)col);
}
hipError_t launch_argmax_keys(const unsigned long long* keys, int rows, int nblk, int32_t* out,
                              hipStream_t st);

SplitPlan gemm_plan(int N, int K, int dtype);
SplitPlan gemm_plan_whole(int N, int K);  // one workgroup per column block
size_t packed_bytes(int N, int K);
hipError_t launch_pack(const void* src, int N, int K, void* dst, hipStream_t st);
hipError_t launch_gemm(const GemmDesc& g, int dtype, hipStream_t st);

// epilogues of the split GEMM
enum QkvDest { QKV_TO_BLOCK = 0, QKV_TO_CACHE = 1 };
struct QkvEpi {
  const float* part; SplitPlan sp; int rows_pad; int N;
  int rows, H, Hkv, hd;
  const int32_t* pos;      // absolute position of each row
  const float2* rope;      // [max_ctx][hd/2] (cos, sin)
  void* q;                 // [rows][H*hd]
  void* kdst; void* vdst;  // block: [rows][Hkv*hd]; cache: [Hkv][ld_ctx][hd]
  int dest; int ld_ctx;
};
hipError_t launch_qkv_epi(const QkvEpi& e, int dtype, hipStream_t st);
hipError_t launch_resid_norm(const float* part, const SplitPlan& sp, int rows_pad, int d,
                             int rows, float* x, const void* g, void* h, float eps, int dtype,
                             hipStream_t st);
hipError_t launch_silu_epi(const float* part, const SplitPlan& sp, int rows_pad, int F, int rows,
                           void* act, int dtype, hipStream_t st);
hipError_t launch_sum_epi(const float* part, const SplitPlan& sp, int rows_pad, int N, int rows,
                          float* y, hipStream_t st);

// norm / embedding / argmax
hipError_t launch_rmsnorm(const float* x, const void* g, void* y, int rows, int d, float eps,
                          int dtype, hipStream_t st);
hipError_t launch_embed(const int32_t* ids, const void* emb, float* x, int rows, int d,
                        int dtype, hipStream_t st);
hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* out, hipStream_t st);

// attention
struct AttnDesc {
  const void* q;       // [rows][H*hd]
  const void* kc;      // [Hkv][ld_ctx][hd]
  const void* vc;
  const void* kb;      // [M][Hkv*hd] block rows (step mode)
  const void* vb;
  void* out;           // [rows][H*hd]
  const int32_t* pos;  // absolute position per row
  const int32_t* Pdev; // committed length P on the device (step mode), or null
  int P_host;          // used when Pdev is null
  int rows, H, Hkv, hd, ld_ctx;
  int causal_cache;    // 1: every key 0..pos(row) is in the cache (prefill)
  RowLayout lay;
  // Split of each row's keys: the committed tiles [0, F) go through the MFMA
  // kernel in the chunks of attn_chunk_start, [F, pos] through the per-row
  // kernel; F = min(floor((pos - D) / 16) * 16, floor(P / 16) * 16).
  // mfma == 0: no MFMA part (F = 0).
  int D;
  int mfma;
  int nsplit;          // chunks allocated in part_* (grid of the MFMA kernel)
  float* part_o;       // [nsplit][rows][H][hd] unnormalised outputs
  float* part_ml;      // [nsplit][rows][H][2] running max, sum
};
hipError_t launch_attention(const AttnDesc& a, int dtype, hipStream_t st);
// Whether the MFMA kernel takes the shared prefix (bf16, head_dim 128).
int attn_uses_mfma(int dtype, int hd);
// The shared prefix of a row is split into chunks on a fixed partition of
// absolute positions (64 wide below 512, 128 below 1024, 256 below 4096, 512
// after: short prefixes spread over more workgroups, long ones keep the
// number of partials down), so a row's arithmetic depends on its position
// only, never on the session's context capacity.
__host__ __device__ inline int attn_chunk_start(int s) {
  return s <= 8 ? 64 * s
       : s <= 12 ? 512 + 128 * (s - 8)
       : s <= 24 ? 1024 + 256 * (s - 12)
                 : 4096 + 512 * (s - 24);
}
__host__ __device__ inline int attn_nchunks(int L) {  // chunks meeting [0, L)
  if (L <= 0) return 0;
  if (L <= 512) return (L + 63) / 64;
  if (L <= 1024) return 8 + (L - 512 + 127) / 128;
  if (L <= 4096) return 12 + (L - 1024 + 255) / 256;
  return 24 + (L - 4096 + 511) / 512;
}
size_t attn_part_floats(int nsplit, int rows, int H, int hd);

// lookahead bookkeeping kernels
struct PoolDesc {
  int32_t* tok;   // [V][cap][N-1]
  int32_t* cnt;   // [V]
  int32_t* head;  // [V]
  int V, cap, n1; // n1 = N - 1
  int lru;        // 1: a repeated suffix becomes the bucket's newest entry
  int32_t* ctx;   // [V][cap] the token before each entry's n-gram (-1: none)
  int by_ctx;     // 1: select entries whose context is the token before cur first
};
struct StepIO {
  DevState* st;
  int32_t* win;   // [(N-1)][W]
  int32_t* cand;  // [G][N-1]
  int32_t* ids;   // [M]
  int32_t* pos;   // [M]
  const int32_t* amax;  // [M]
  int max_new, eos;
  int gmax;       // the session's G (the layout's G may be smaller, LA_ADAPTIVE_G)
  // sampling verification ([LD] §3.4 "Sampling verification (Algorithm 4)");
  // temp == 0: greedy verification
  const float* logits;  // [M][V]
  int V;
  float temp;
  unsigned long long seed;
  int top_k;      // 0: no top-K cut (else 1 <= top_k < V)
  float top_p;    // 1: no top-P cut (else 0 < top_p < 1)
  // the sampling weights of row 0 and of every verification row (block b:
  // row 0 for b = 0, verification row b - 1 after), [1 + G(N-1)][V], and
  // their sums
  float* sw;
  float* sz;
};
hipError_t launch_gather(const PoolDesc& pool, const StepIO& io, const RowLayout& lay,
                         hipStream_t st);
hipError_t launch_verify(const PoolDesc& pool, const StepIO& io, const RowLayout& lay,
                         hipStream_t st);
// Largest vocabulary the sampling verification keeps in LDS.
constexpr int SAMPLE_VMAX = 32768;
hipError_t launch_sample_weights(const StepIO& io, const RowLayout& lay, hipStream_t st);
hipError_t launch_sample_verify(const StepIO& io, const RowLayout& lay, hipStream_t st);
hipError_t launch_philox_uniform(unsigned long long seed, unsigned long long step, int n,
                                 float* out, hipStream_t st);
struct KvCommit {
  const DevState* st;
  const void* kb; const void* vb;  // [L][M][Hkv*hd]
  void* kc; void* vc;              // [L][Hkv][ld_ctx][hd]
  int L, M, Hkv, hd, ld_ctx, nmax;
};
hipError_t launch_kv_commit(const KvCommit& c, int dtype, hipStream_t st);
hipError_t launch_pool_seed(const PoolDesc& pool, DevState* st, const int32_t* prompt, int n,
                            hipStream_t st_);
hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t st);
hipError_t launch_fill_bytes0(void* p, size_t n, hipStream_t st);
