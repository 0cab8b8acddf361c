// Projection GEMMs of the decoder forward: y = x W^T at M = 1 + (W+G)(N-1)
// rows (the pages' "FLOPs per step ∝ (W+G)(N-1)", [LD] §3.4 "Scaling Law").
// At these M the GEMMs stream weights from HBM (intensity ~M FLOP/byte, below
// the bf16 MFMA ridge), so every weight byte is read once, in whole 128-byte
// lines, with several chunks in flight per wave.
//
// Batch invariance: the sum for one output element runs over the same MFMA
// sequence (64-wide K chunks, fixed K split chosen from (N, K) alone, splits
// added in split order) whatever the number of rows or the row's place in the
// tile.  A row therefore gets bit-identical results at M = 1 (autoregressive)
// and at M = 121 (lookahead), which the token-for-token equality of the two
// decodes relies on.
#include "la_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int NWG = 128;      // output columns per workgroup (4 waves x 2 tiles x 16)
constexpr int KC = 64;        // K per chunk: two 16x16x32 MFMA steps
#ifndef LA_GEMM_PF
#define LA_GEMM_PF 4
#endif
#ifndef LA_GEMM_TARGET_WG
#define LA_GEMM_TARGET_WG 256
#endif
constexpr int PF = LA_GEMM_PF;  // weight chunks in flight per wave

union U4B { u32x4_t u; bf16x8_t v; };

// Workgroup barrier that waits only for this wave's LDS traffic
// (lgkmcnt(0)), not for its outstanding global loads: __syncthreads() also
// drains vmcnt, which would empty the weight prefetch pipeline at every chunk.
// s_waitcnt imm on gfx9: vmcnt[3:0]|[15:14] = 63, expcnt[6:4] = 7, lgkmcnt[11:8] = 0.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One workgroup: rows [mb*128, mb*128 + 16*MT) x columns [nb*128, nb*128+128)
// over the K chunks of split `blockIdx.y`, with five waves:
//  * waves 0-3 (consumers) own 32 columns each (two 16-column MFMA tiles) for
//    all MT row tiles; each keeps PF chunks of its weight rows in flight in
//    registers and issues no other global load, so its in-order load counter
//    never makes it wait on anything but the chunk it is about to use;
//  * wave 4 (producer) stages the x tile of each chunk into a ring of XR LDS
//    stages, XR-1 chunks ahead of the consumers, from a 2-deep register ring.
// One barrier per chunk; the producer writes the stage the consumers left
// at the previous barrier.
//
// Weights come in the packed layout (see la.h): MFMA step j of chunk c of a
// 16-row stripe is one contiguous KB holding, for lane (q = lane/16,
// r = lane%16), k in [64c + 32j + 8q, +8) of row r; the x tile is read with
// the same k order.  A wave therefore streams each of its two stripes
// sequentially.  LDS x rows are 128 bytes with the 16-byte pieces
// XOR-swizzled by (row/2) mod 8 so the A-fragment reads hit distinct banks.
constexpr int XR = 3;  // LDS stages of the x tile

__device__ __forceinline__ int xswz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

template <int MT>
__global__ __launch_bounds__(320) void k_gemm_bf16(GemmDesc g) {
  constexpr int XSTAGE = MT * 16 * 64;  // bf16 per x stage
  __shared__ __align__(16) bf16_t xs[XR * XSTAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int nb = blockIdx.x, split = blockIdx.y, mb = blockIdx.z;
  const int K = g.K;
  const int nch = K / KC;
  const int c0 = (int)((long long)split * nch / g.S);
  const int c1 = (int)((long long)(split + 1) * nch / g.S);
  const int row0 = mb * 128;
  const int xrows = g.rows - row0;  // valid rows in this row block

  if (wave == 4) {
    // ---------------- producer: x tiles -> LDS ring ----------------
    constexpr int NP = MT * 2;  // 16-byte pieces per lane per chunk
    const bf16_t* X = (const bf16_t*)g.x;
    const bf16_t* xp[NP];
    int lo[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int pi = lane + 64 * j;
      const int row = pi >> 3, pc = pi & 7;
      const int rc = row < xrows ? row : xrows - 1;
      xp[j] = X + (size_t)(row0 + rc) * K + pc * 8;
      lo[j] = row * 64 + xswz(row, pc) * 8;
    }
    u32x4_t ring[2][NP];
    auto load = [&](int c, u32x4_t (&dst)[NP]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NP; ++j) dst[j] = *(const u32x4_t*)(xp[j] + (size_t)c * KC);
    };
    auto store = [&](int c, const u32x4_t (&src)[NP]) __attribute__((always_inline)) {
      bf16_t* st = xs + ((c - c0) % XR) * XSTAGE;
#pragma unroll
      for (int j = 0; j < NP; ++j) *(u32x4_t*)(st + lo[j]) = src[j];
    };
    // prologue: stages for chunks c0 .. c0+XR-2, ring for the next two
    for (int c = c0; c < c1 && c < c0 + XR - 1; ++c) {
      load(c, ring[0]);
      store(c, ring[0]);
    }
    load(min(c0 + XR - 1, c1 - 1), ring[(XR - 1) & 1]);
    load(min(c0 + XR, c1 - 1), ring[XR & 1]);
    int c = c0;
    // steady state: store chunk c+XR-1, load chunk c+XR+1 (same ring slot)
    for (; c + XR + 3 <= c1; c += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        lds_barrier();
        const int slot = (XR - 1 + u) & 1;
        store(c + u + XR - 1, ring[slot]);
        load(c + u + XR + 1, ring[slot]);
      }
    }
    for (; c < c1; ++c) {
      lds_barrier();
      const int slot = (c - c0 + XR - 1) & 1;
      if (c + XR - 1 < c1) {
        if (slot == 0) store(c + XR - 1, ring[0]); else store(c + XR - 1, ring[1]);
      }
      if (c + XR + 1 < c1) {
        if (slot == 0) load(c + XR + 1, ring[0]); else load(c + XR + 1, ring[1]);
      }
    }
    return;
  }

  // ---------------- consumers: weights + MFMA ----------------
  const int col0 = nb * NWG;
  int si = 0, sbase = 0;
  while (si < g.nseg - 1 && col0 >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
  const bf16_t* W = (const bf16_t*)g.seg[si].w;
  const int segn = g.seg[si].n;
  const int nl = col0 - sbase + wave * 32;  // first local weight row of this wave

  // a column past the segment reads row 0; its output is discarded at the
  // store.  Unpredicated loads let the compiler count outstanding loads
  // exactly instead of draining them at branch joins.
  // packed stripes: stripe of 16 rows, K/64 blocks of 2 KB, 1 KB per MFMA
  // step; a stripe past the segment reads stripe 0 (its output is discarded)
  const bf16_t* wrow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int stripe = (nl + t * 16) >> 4;
    const int ok = nl + t * 16 < segn;
    wrow[t] = W + (size_t)(ok ? stripe : 0) * nch * 1024 + lane * 8;
  }

  f32x4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t wr[PF][2][2];
  auto load_w = [&](int c, u32x4_t (&dst)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16_t* p = wrow[t] + (size_t)c * 1024;
      dst[t][0] = *(const u32x4_t*)p;
      dst[t][1] = *(const u32x4_t*)(p + 512);
    }
  };
  // A-fragment offsets (bf16) in a stage: row i*16 + r, k 32j + 8q .. +8
  // (16-byte piece 4j + q)
  int aoff[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) aoff[i][j] = (i * 16 + r) * 64 + xswz(i * 16 + r, 4 * j + q) * 8;

  auto chunk = [&](int c, u32x4_t (&w)[2][2], bool more_w) __attribute__((always_inline)) {
    lds_barrier();
    const bf16_t* st = xs + ((c - c0) % XR) * XSTAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      U4B b0, b1;
      b0.u = w[0][j];
      b1.u = w[1][j];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        U4B a;
        a.u = *(const u32x4_t*)(st + aoff[i][j]);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b0.v, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b1.v, acc[i][1], 0, 0, 0);
      }
    }
    if (more_w) load_w(c + PF, w);
  };

  // prologue: unconditional (a stage past the split reloads the last chunk
  // and is never used), so the loop sees a fixed count of loads in flight
#pragma unroll
  for (int s = 0; s < PF; ++s) load_w(min(c0 + s, c1 - 1), wr[s]);
  int cb = c0;
  for (; cb + 2 * PF <= c1; cb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) chunk(cb + s, wr[s], true);
  }
  for (; cb < c1; cb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int c = cb + s;
      if (c < c1) chunk(c, wr[s], c + PF < c1);
    }
  }

  // D layout of 16x16 MFMA: lane holds rows 4q..4q+3 of column r
  float* out = g.part + (size_t)split * g.rows_pad * g.N;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nloc = nl + t * 16 + r;
    if (nloc >= segn) continue;
    const int col = sbase + nloc;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + i * 16 + q * 4 + e;
        if (row < g.rows) out[(size_t)row * g.N + col] = acc[i][t][e];
      }
    }
  }
}

// fp32 models: one thread per output element, K summed in order.
__global__ __launch_bounds__(64) void k_gemm_f32(GemmDesc g) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= g.N || m >= g.rows) return;
  int si = 0, sbase = 0;
  while (si < g.nseg - 1 && n >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
  const float* w = (const float*)g.seg[si].w + (size_t)(n - sbase) * g.K;
  const float* x = (const float*)g.x + (size_t)m * g.K;
  float acc = 0.f;
  for (int k = 0; k < g.K; ++k) acc = fmaf(x[k], w[k], acc);
  g.part[(size_t)m * g.N + n] = acc;
}

// Sum of the split partials of one output element, splits in order.  S is a
// compile-time constant so the S loads are issued together.
template <int S>
__device__ __forceinline__ float sum_splits(const float* __restrict__ part, int rows_pad, int N,
                                            int m, int col) {
  float p[S];
#pragma unroll
  for (int s = 0; s < S; ++s) p[s] = part[((size_t)s * rows_pad + m) * N + col];
  float v = p[0];
#pragma unroll
  for (int s = 1; s < S; ++s) v += p[s];
  return v;
}

#define LA_SPLIT_DISPATCH(S_, CALL) \
  switch (S_) {                     \
    case 1: CALL(1); break;         \
    case 2: CALL(2); break;         \
    case 4: CALL(4); break;         \
    case 8: CALL(8); break;         \
    case 16: CALL(16); break;       \
    default: return hipErrorInvalidValue; \
  }

// Sum the K splits of the fused QKV product, rotate q and k (RoPE at the
// row's position, pairs (i, i + hd/2)) and store q, k, v.  One thread per
// rotated pair of q/k or per element of v.
template <typename T, int S>
__global__ __launch_bounds__(256) void k_qkv_epi(QkvEpi e) {
  const int m = blockIdx.y;
  const int u = blockIdx.x * 256 + threadIdx.x;
  const int hd = e.hd, half = hd >> 1;
  const int nq = e.H * hd, nk = e.Hkv * hd;
  const int npair = (e.H + e.Hkv) * half;
  if (u >= npair + nk) return;
  const int pos = e.pos[m];
  if (u < npair) {
    const int hh = u / half, i = u - hh * half;
    const int col = hh * hd + i;
    const float x1 = sum_splits<S>(e.part, e.rows_pad, e.N, m, col);
    const float x2 = sum_splits<S>(e.part, e.rows_pad, e.N, m, col + half);
    const float2 cs = e.rope[(size_t)pos * half + i];
    const float y1 = x1 * cs.x - x2 * cs.y;
    const float y2 = x1 * cs.y + x2 * cs.x;
    if (hh < e.H) {
      T* q = (T*)e.q + (size_t)m * nq + hh * hd;
      st_f(q + i, y1);
      st_f(q + i + half, y2);
    } else {
      const int kvh = hh - e.H;
      T* kd = (T*)e.kdst;
      T* dst = e.dest == QKV_TO_BLOCK ? kd + (size_t)m * nk + kvh * hd
                                      : kd + ((size_t)kvh * e.ld_ctx + pos) * hd;
      st_f(dst + i, y1);
      st_f(dst + i + half, y2);
    }
  } else {
    const int vi = u - npair;
    const float v = sum_splits<S>(e.part, e.rows_pad, e.N, m, nq + nk + vi);
    const int kvh = vi / hd, i = vi - kvh * hd;
    T* vd = (T*)e.vdst;
    T* dst = e.dest == QKV_TO_BLOCK ? vd + (size_t)m * nk + vi
                                    : vd + ((size_t)kvh * e.ld_ctx + pos) * hd + i;
    st_f(dst, v);
  }
}

template <int S>
__global__ __launch_bounds__(256) void k_resid_epi(const float* part, int rows_pad, int N,
                                                   float* x) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  x[(size_t)m * N + n] += sum_splits<S>(part, rows_pad, N, m, n);
}

// x[m] += sum of the split partials; then h[m] = x[m] / sqrt(mean(x^2) + eps) * g
// (the residual add fused with the next RMSNorm).  Thread t owns columns
// t, t+256, ...; the sum of squares is reduced in a fixed tree.
// x[m] += sum of the split partials (in split order); then
// h[m] = x[m] / sqrt(mean(x^2) + eps) * g: the residual add fused with the
// next RMSNorm.  One workgroup of d/NC threads per row; thread t owns columns
// t + j*blockDim; the sum of squares is reduced in a fixed order (within a
// wave by xor-shuffles, then across waves in wave order).
template <typename T, int S, int NC>
__global__ __launch_bounds__(1024) void k_resid_norm(const float* __restrict__ part, int rows_pad,
                                                     int d, float* __restrict__ x,
                                                     const T* __restrict__ g, T* __restrict__ h,
                                                     float eps) {
  __shared__ float red[16];
  const int m = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  float* xr = x + (size_t)m * d;
  float v[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) v[j] = sum_splits<S>(part, rows_pad, d, m, tid + j * nt);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    v[j] = xr[tid + j * nt] + v[j];
    xr[tid + j * nt] = v[j];
    ss = fmaf(v[j], v[j], ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (nt >> 6); ++w) tot += red[w];
  const float rs = 1.0f / sqrtf(tot / (float)d + eps);
  T* hr = h + (size_t)m * d;
#pragma unroll
  for (int j = 0; j < NC; ++j) st_f(hr + tid + j * nt, v[j] * rs * ld_f(g + tid + j * nt));
}

template <int S>
__global__ __launch_bounds__(256) void k_sum_epi(const float* part, int rows_pad, int N,
                                                 float* y) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  y[(size_t)m * N + n] = sum_splits<S>(part, rows_pad, N, m, n);
}

template <typename T, int S>
__global__ __launch_bounds__(256) void k_silu_epi(const float* part, int rows_pad, int F,
                                                  T* act) {
  const int m = blockIdx.y;
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const float gt = sum_splits<S>(part, rows_pad, 2 * F, m, f);
  const float up = sum_splits<S>(part, rows_pad, 2 * F, m, F + f);
  const float sg = gt / (1.0f + expf(-gt));
  st_f(act + (size_t)m * F + f, sg * up);
}

// dst block (stripe s, chunk c): element (j, lane, e) = W[16s + lane%16][64c + 32j + 8(lane/16) + e]
__global__ __launch_bounds__(128) void k_pack_bf16(const bf16_t* __restrict__ src, int N, int K,
                                                   bf16_t* __restrict__ dst) {
  const int s = blockIdx.y, c = blockIdx.x;
  const int nch = K / KC;
  const int j = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = 16 * s + (lane & 15);
  const int k = 64 * c + 32 * j + 8 * (lane >> 4);
  u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
  if (row < N) v = *(const u32x4_t*)(src + (size_t)row * K + k);
  *(u32x4_t*)(dst + (((size_t)s * nch + c) * 2 + j) * 512 + lane * 8) = v;
}

}  // namespace

size_t packed_bytes(int N, int K) { return (size_t)((N + 15) / 16) * 16 * K * 2; }

hipError_t launch_pack(const void* src, int N, int K, void* dst, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_bf16, dim3(K / KC, (N + 15) / 16), dim3(128), 0, st,
                     (const bf16_t*)src, N, K, (bf16_t*)dst);
  return hipGetLastError();
}

int gemm_splits(int N, int K, int dtype) {
  if (dtype != LA_BF16) return 1;
  const int nblk = (N + NWG - 1) / NWG;
  const int nch = K / KC;
  int S = 1;
  // the largest power-of-two split that keeps the grid within one round of
  // LA_GEMM_TARGET_WG workgroups (one per CU), with >= 4 chunks per split
  while (nblk * S * 2 <= LA_GEMM_TARGET_WG && (S * 2) * 4 <= nch && S < 16) S *= 2;
  return S;
}

hipError_t launch_gemm(const GemmDesc& g, int dtype, hipStream_t st) {
  if (dtype == LA_F32) {
    dim3 grid((g.N + 63) / 64, g.rows);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(64), 0, st, g);
    return hipGetLastError();
  }
  const int nblk = (g.N + NWG - 1) / NWG;
  const int mblk = (g.rows + 127) / 128;
  const int rows_last = g.rows - (mblk - 1) * 128;
  // the row-tile count only changes how many rows one workgroup carries, not
  // the arithmetic of any row
  const int mt = mblk > 1 ? 8 : (rows_last + 15) / 16;
  dim3 grid(nblk, g.S, mblk);
  const dim3 blk(320);
  switch (mt) {
    case 1: hipLaunchKernelGGL(k_gemm_bf16<1>, grid, blk, 0, st, g); break;
    case 2: hipLaunchKernelGGL(k_gemm_bf16<2>, grid, blk, 0, st, g); break;
    case 3: hipLaunchKernelGGL(k_gemm_bf16<3>, grid, blk, 0, st, g); break;
    case 4: hipLaunchKernelGGL(k_gemm_bf16<4>, grid, blk, 0, st, g); break;
    case 5: hipLaunchKernelGGL(k_gemm_bf16<5>, grid, blk, 0, st, g); break;
    case 6: hipLaunchKernelGGL(k_gemm_bf16<6>, grid, blk, 0, st, g); break;
    case 7: hipLaunchKernelGGL(k_gemm_bf16<7>, grid, blk, 0, st, g); break;
    default: hipLaunchKernelGGL(k_gemm_bf16<8>, grid, blk, 0, st, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_qkv_epi(const QkvEpi& e, int dtype, hipStream_t st) {
  const int units = (e.H + e.Hkv) * (e.hd / 2) + e.Hkv * e.hd;
  dim3 grid((units + 255) / 256, e.rows);
#define LA_QKV(S_)                                                              \
  if (dtype == LA_BF16)                                                         \
    hipLaunchKernelGGL((k_qkv_epi<bf16_t, S_>), grid, dim3(256), 0, st, e);     \
  else                                                                          \
    hipLaunchKernelGGL((k_qkv_epi<float, S_>), grid, dim3(256), 0, st, e);
  LA_SPLIT_DISPATCH(e.S, LA_QKV)
#undef LA_QKV
  return hipGetLastError();
}

hipError_t launch_resid_epi(const float* part, int S, int rows_pad, int N, int rows, float* x,
                            hipStream_t st) {
#define LA_RE(S_) \
  hipLaunchKernelGGL((k_resid_epi<S_>), dim3((N + 255) / 256, rows), dim3(256), 0, st, part, rows_pad, N, x);
  LA_SPLIT_DISPATCH(S, LA_RE)
#undef LA_RE
  return hipGetLastError();
}

// columns per thread for a row of d values in one workgroup (<= 1024 threads)
static int norm_nc(int d) {
  for (int nc = 1; nc <= 16; ++nc)
    if (d % nc == 0 && d / nc <= 1024 && (d / nc) % 64 == 0) return nc;
  return 0;
}

hipError_t launch_resid_norm(const float* part, int S, int rows_pad, int d, int rows, float* x,
                             const void* g, void* h, float eps, int dtype, hipStream_t st) {
  const int nc = norm_nc(d);
  if (!nc) return hipErrorInvalidValue;
  const dim3 blk(d / nc);
#define LA_RN2(S_, NC_)                                                                        \
  if (dtype == LA_BF16)                                                                        \
    hipLaunchKernelGGL((k_resid_norm<bf16_t, S_, NC_>), dim3(rows), blk, 0, st, part, rows_pad, \
                       d, x, (const bf16_t*)g, (bf16_t*)h, eps);                               \
  else                                                                                         \
    hipLaunchKernelGGL((k_resid_norm<float, S_, NC_>), dim3(rows), blk, 0, st, part, rows_pad,  \
                       d, x, (const float*)g, (float*)h, eps);
#define LA_RN(S_)                                                       \
  switch (nc) {                                                         \
    case 1: LA_RN2(S_, 1) break;                                        \
    case 2: LA_RN2(S_, 2) break;                                        \
    case 4: LA_RN2(S_, 4) break;                                        \
    case 5: LA_RN2(S_, 5) break;                                        \
    case 8: LA_RN2(S_, 8) break;                                        \
    case 16: LA_RN2(S_, 16) break;                                      \
    default: return hipErrorInvalidValue;                               \
  }
  LA_SPLIT_DISPATCH(S, LA_RN)
#undef LA_RN
#undef LA_RN2
  return hipGetLastError();
}

hipError_t launch_sum_epi(const float* part, int S, int rows_pad, int N, int rows, float* y,
                          hipStream_t st) {
#define LA_SE(S_) \
  hipLaunchKernelGGL((k_sum_epi<S_>), dim3((N + 255) / 256, rows), dim3(256), 0, st, part, rows_pad, N, y);
  LA_SPLIT_DISPATCH(S, LA_SE)
#undef LA_SE
  return hipGetLastError();
}

hipError_t launch_silu_epi(const float* part, int S, int rows_pad, int F, int rows, void* act,
                           int dtype, hipStream_t st) {
#define LA_SI(S_)                                                                              \
  if (dtype == LA_BF16)                                                                        \
    hipLaunchKernelGGL((k_silu_epi<bf16_t, S_>), dim3((F + 255) / 256, rows), dim3(256), 0, st, \
                       part, rows_pad, F, (bf16_t*)act);                                       \
  else                                                                                         \
    hipLaunchKernelGGL((k_silu_epi<float, S_>), dim3((F + 255) / 256, rows), dim3(256), 0, st,  \
                       part, rows_pad, F, (float*)act);
  LA_SPLIT_DISPATCH(S, LA_SI)
#undef LA_SI
  return hipGetLastError();
}
