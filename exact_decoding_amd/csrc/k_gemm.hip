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
constexpr int PF = 4;         // weight chunks in flight per wave
constexpr int XS = KC + 8;    // LDS row stride (bf16) for the x tile, padded against bank conflicts

union U4B { uint4 u; bf16x8_t v; };

// One workgroup: rows [mb*128, mb*128 + 16*MT) x columns [nb*128, nb*128+128)
// over the K chunks of split `blockIdx.y`.  Wave w owns columns w*32..w*32+31
// (two 16-column MFMA tiles) for all MT row tiles.
//
// K permutation inside a 64-chunk: lane group q = lane/16 supplies k in
// [16q + 8j, 16q + 8j + 8) to MFMA step j, in both operands, so a lane reads
// 32 contiguous bytes of its weight row per chunk and four lanes cover one
// 128-byte line.
template <int MT>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmDesc g) {
  __shared__ __align__(16) bf16_t xs[2][MT * 16 * XS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int nb = blockIdx.x, split = blockIdx.y, mb = blockIdx.z;
  const int K = g.K;
  const int nch = K / KC;
  const int c0 = (int)((long long)split * nch / g.S);
  const int c1 = (int)((long long)(split + 1) * nch / g.S);

  // weight segment holding this workgroup's columns
  const int col0 = nb * NWG;
  int si = 0, sbase = 0;
  while (si < g.nseg - 1 && col0 >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
  const bf16_t* W = (const bf16_t*)g.seg[si].w;
  const int segn = g.seg[si].n;
  const int nl = col0 - sbase + wave * 32;  // first local weight row of this wave

  const bf16_t* wrow[2];
  bool wok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = nl + t * 16 + r;
    wok[t] = n < segn;
    wrow[t] = W + (size_t)(wok[t] ? n : 0) * K + q * 16;
  }

  const bf16_t* X = (const bf16_t*)g.x;
  const int row0 = mb * 128;
  const int xrows = g.rows - row0;  // valid rows in this row block

  f32x4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wr[PF][2][2];
  auto load_w = [&](int c, uint4 (&dst)[2][2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (wok[t]) {
        const uint4* p = (const uint4*)(wrow[t] + (size_t)c * KC);
        dst[t][0] = p[0];
        dst[t][1] = p[1];
      } else {
        dst[t][0] = make_uint4(0, 0, 0, 0);
        dst[t][1] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // x tile: MT*16 rows x 64 k = MT*128 pieces of 16 bytes
  constexpr int XP = (MT * 128 + 255) / 256;
  uint4 xr[XP];
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < XP; ++j) {
      const int p = tid + j * 256;
      if (p < MT * 128) {
        const int rr = p >> 3, cc = p & 7;
        if (rr < xrows)
          xr[j] = *(const uint4*)(X + (size_t)(row0 + rr) * K + (size_t)c * KC + cc * 8);
        else
          xr[j] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XP; ++j) {
      const int p = tid + j * 256;
      if (p < MT * 128) {
        const int rr = p >> 3, cc = p & 7;
        *(uint4*)(&xs[buf][rr * XS + cc * 8]) = xr[j];
      }
    }
  };

  if (c0 < c1) {
#pragma unroll
    for (int s = 0; s < PF; ++s)
      if (c0 + s < c1) load_w(c0 + s, wr[s]);
    load_x(c0);
    store_x(0);
    __syncthreads();
  }

  for (int cb = c0; cb < c1; cb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int c = cb + s;
      if (c < c1) {
        const int buf = (c - c0) & 1;
        if (c + 1 < c1) load_x(c + 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          U4B b0, b1;
          b0.u = wr[s][0][j];
          b1.u = wr[s][1][j];
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            U4B a;
            a.u = *(const uint4*)(&xs[buf][(i * 16 + r) * XS + q * 16 + j * 8]);
            acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b0.v, acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b1.v, acc[i][1], 0, 0, 0);
          }
        }
        if (c + PF < c1) load_w(c + PF, wr[s]);
        if (c + 1 < c1) store_x(buf ^ 1);
        __syncthreads();
      }
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

__device__ __forceinline__ float sum_splits(const float* part, int S, int rows_pad, int N, int m,
                                            int col) {
  float v = part[(size_t)m * N + col];
  for (int s = 1; s < S; ++s) v += part[((size_t)s * rows_pad + m) * N + col];
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void k_qkv_epi(QkvEpi e) {
  const int m = blockIdx.x;
  if (m >= e.rows) return;
  const int hd = e.hd, half = hd >> 1;
  const int nq = e.H * hd, nk = e.Hkv * hd;
  const int pos = e.pos[m];
  T* q = (T*)e.q + (size_t)m * nq;
  T* kd = (T*)e.kdst;
  T* vd = (T*)e.vdst;
  const float2* rope = e.rope + (size_t)pos * half;
  for (int u = threadIdx.x; u < (e.H + e.Hkv) * half; u += blockDim.x) {
    const int hh = u / half, i = u - hh * half;
    const int col = hh * hd + i;
    const float x1 = sum_splits(e.part, e.S, e.rows_pad, e.N, m, col);
    const float x2 = sum_splits(e.part, e.S, e.rows_pad, e.N, m, col + half);
    const float2 cs = rope[i];
    const float y1 = x1 * cs.x - x2 * cs.y;
    const float y2 = x1 * cs.y + x2 * cs.x;
    if (hh < e.H) {
      st_f(q + hh * hd + i, y1);
      st_f(q + hh * hd + i + half, y2);
    } else {
      const int kvh = hh - e.H;
      T* dst = e.dest == QKV_TO_BLOCK ? kd + (size_t)m * nk + kvh * hd
                                      : kd + ((size_t)kvh * e.ld_ctx + pos) * hd;
      st_f(dst + i, y1);
      st_f(dst + i + half, y2);
    }
  }
  for (int u = threadIdx.x; u < nk; u += blockDim.x) {
    const float v = sum_splits(e.part, e.S, e.rows_pad, e.N, m, nq + nk + u);
    const int kvh = u / hd, i = u - kvh * hd;
    T* dst = e.dest == QKV_TO_BLOCK ? vd + (size_t)m * nk + u
                                    : vd + ((size_t)kvh * e.ld_ctx + pos) * hd + i;
    st_f(dst, v);
  }
}

__global__ __launch_bounds__(256) void k_resid_epi(const float* part, int S, int rows_pad, int N,
                                                   float* x) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  x[(size_t)m * N + n] += sum_splits(part, S, rows_pad, N, m, n);
}

__global__ __launch_bounds__(256) void k_sum_epi(const float* part, int S, int rows_pad, int N,
                                                 float* y) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  y[(size_t)m * N + n] = sum_splits(part, S, rows_pad, N, m, n);
}

template <typename T>
__global__ __launch_bounds__(256) void k_silu_epi(const float* part, int S, int rows_pad, int F,
                                                  T* act) {
  const int m = blockIdx.y;
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const float gt = sum_splits(part, S, rows_pad, 2 * F, m, f);
  const float up = sum_splits(part, S, rows_pad, 2 * F, m, F + f);
  const float sg = gt / (1.0f + expf(-gt));
  st_f(act + (size_t)m * F + f, sg * up);
}

}  // namespace

int gemm_splits(int N, int K, int dtype) {
  if (dtype != LA_BF16) return 1;
  const int nblk = (N + NWG - 1) / NWG;
  const int nch = K / KC;
  int S = 1;
  // enough workgroups to cover the 256 CUs, keeping >= 4 chunks per split
  while (nblk * S < 256 && (S * 2) * 4 <= nch) S *= 2;
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
  switch (mt) {
    case 1: hipLaunchKernelGGL(k_gemm_bf16<1>, grid, dim3(256), 0, st, g); break;
    case 2: hipLaunchKernelGGL(k_gemm_bf16<2>, grid, dim3(256), 0, st, g); break;
    case 3: hipLaunchKernelGGL(k_gemm_bf16<3>, grid, dim3(256), 0, st, g); break;
    case 4: hipLaunchKernelGGL(k_gemm_bf16<4>, grid, dim3(256), 0, st, g); break;
    case 5: hipLaunchKernelGGL(k_gemm_bf16<5>, grid, dim3(256), 0, st, g); break;
    case 6: hipLaunchKernelGGL(k_gemm_bf16<6>, grid, dim3(256), 0, st, g); break;
    case 7: hipLaunchKernelGGL(k_gemm_bf16<7>, grid, dim3(256), 0, st, g); break;
    default: hipLaunchKernelGGL(k_gemm_bf16<8>, grid, dim3(256), 0, st, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_qkv_epi(const QkvEpi& e, int dtype, hipStream_t st) {
  if (dtype == LA_BF16)
    hipLaunchKernelGGL(k_qkv_epi<bf16_t>, dim3(e.rows), dim3(256), 0, st, e);
  else
    hipLaunchKernelGGL(k_qkv_epi<float>, dim3(e.rows), dim3(256), 0, st, e);
  return hipGetLastError();
}

hipError_t launch_resid_epi(const float* part, int S, int rows_pad, int N, int rows, float* x,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_resid_epi, dim3((N + 255) / 256, rows), dim3(256), 0, st, part, S,
                     rows_pad, N, x);
  return hipGetLastError();
}

hipError_t launch_sum_epi(const float* part, int S, int rows_pad, int N, int rows, float* y,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_sum_epi, dim3((N + 255) / 256, rows), dim3(256), 0, st, part, S,
                     rows_pad, N, y);
  return hipGetLastError();
}

hipError_t launch_silu_epi(const float* part, int S, int rows_pad, int F, int rows, void* act,
                           int dtype, hipStream_t st) {
  if (dtype == LA_BF16)
    hipLaunchKernelGGL(k_silu_epi<bf16_t>, dim3((F + 255) / 256, rows), dim3(256), 0, st, part,
                       S, rows_pad, F, (bf16_t*)act);
  else
    hipLaunchKernelGGL(k_silu_epi<float>, dim3((F + 255) / 256, rows), dim3(256), 0, st, part, S,
                       rows_pad, F, (float*)act);
  return hipGetLastError();
}
