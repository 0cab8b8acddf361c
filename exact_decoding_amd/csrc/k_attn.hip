// Lookahead attention, RMSNorm, embedding gather and per-row argmax.
//
// Attention follows the lookahead mask of [LD] §3.4 "The custom attention
// mask (Figure 2)" without materialising it.  Under the row layout of a step
// (row 0 = current token at P; lookahead row 1+l*W+k at P+1+l+k;
// verification row 1+W(N-1)+g(N-1)+(i-1) at P+i) every row sees exactly one
// key at each position 0..pos(row): committed positions < P come from the KV
// cache, and position P+j comes from the block row `chain_row(row, j)`.
//
// Each row's keys are visited in absolute-position tiles of 64 with a fixed
// summation order, so a row's result depends only on the keys it sees, not on
// whether they sit in the cache or in the block, nor on the other rows: the
// verification row that reproduces an autoregressive step gets the bits of
// that step.
#include "la_internal.h"

namespace {

// Block row holding the key at position P + j for block row `r` (0 <= j <=
// pos(r) - P).
__device__ __forceinline__ int chain_row(int r, int j, const RowLayout& L) {
  if (j == 0 || r == 0) return 0;
  const int n1 = L.N - 1;
  int rr = r - 1;
  if (rr < L.W * n1) {           // lookahead row (level l, column k)
    const int l = rr / L.W, k = rr - l * L.W;
    (void)l;
    if (j <= k) return 1 + (j - 1);          // level 0, column j-1
    return 1 + (j - 1 - k) * L.W + k;        // own column, level j-1-k
  }
  rr -= L.W * n1;                // verification row (candidate g)
  const int g = rr / n1;
  return 1 + L.W * n1 + g * n1 + (j - 1);
}

// Position of block row r relative to P (the row layout above).
__device__ __forceinline__ int row_offset(int r, const RowLayout& L) {
  if (r == 0) return 0;
  const int n1 = L.N - 1;
  int rr = r - 1;
  if (rr < L.W * n1) {
    const int l = rr / L.W, k = rr - l * L.W;
    return 1 + l + k;
  }
  rr -= L.W * n1;
  return rr % n1 + 1;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// dot(q, k) over HD in order d = 0..HD-1 (16-byte loads of k)
template <int HD>
__device__ __forceinline__ float dot_q(const float* qs, const bf16_t* k) {
  float acc = 0.f;
#pragma unroll
  for (int d0 = 0; d0 < HD; d0 += 8) {
    const uint4 u = *(const uint4*)(k + d0);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(qs[d0 + 2 * e], __uint_as_float(w[e] << 16), acc);
      acc = fmaf(qs[d0 + 2 * e + 1], __uint_as_float(w[e] & 0xFFFF0000u), acc);
    }
  }
  return acc;
}
template <int HD>
__device__ __forceinline__ float dot_q(const float* qs, const float* k) {
  float acc = 0.f;
#pragma unroll
  for (int d0 = 0; d0 < HD; d0 += 4) {
    const float4 u = *(const float4*)(k + d0);
    acc = fmaf(qs[d0], u.x, acc);
    acc = fmaf(qs[d0 + 1], u.y, acc);
    acc = fmaf(qs[d0 + 2], u.z, acc);
    acc = fmaf(qs[d0 + 3], u.w, acc);
  }
  return acc;
}

// One wave per (head, row).  Lane j of a tile scores the key at position
// 64t + j; lanes own output dimensions lane, lane+64 for the P.V sum.
template <typename T, int HD>
__global__ __launch_bounds__(64) void k_attn(AttnDesc a) {
  constexpr int NPL = (HD + 63) / 64;  // output dims per lane
  __shared__ float qs[HD];
  __shared__ float ps[64];
  const int h = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const int kvh = h * a.Hkv / a.H;
  const int Pc = a.Pdev ? *a.Pdev : a.P_host;
  const int pos = a.pos ? a.pos[r] : Pc + row_offset(r, a.lay);
  const int P = a.causal_cache ? pos + 1 : Pc;
  const int ldb = a.Hkv * HD;
  const T* q = (const T*)a.q + (size_t)r * a.H * HD + h * HD;
  const T* kc = (const T*)a.kc + (size_t)kvh * a.ld_ctx * HD;
  const T* vc = (const T*)a.vc + (size_t)kvh * a.ld_ctx * HD;
  const T* kb = (const T*)a.kb + kvh * HD;
  const T* vb = (const T*)a.vb + kvh * HD;
  for (int i = lane; i < HD; i += 64) qs[i] = ld_f(q + i);
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)HD);

  float m_run = -INFINITY, l_run = 0.f;
  float o[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) o[j] = 0.f;

  const int ntiles = pos / 64 + 1;
  for (int t = 0; t < ntiles; ++t) {
    const int p = t * 64 + lane;
    float s = -INFINITY;
    if (p <= pos) {
      const T* kp = p < P ? kc + (size_t)p * HD
                          : kb + (size_t)chain_row(r, p - P, a.lay) * ldb;
      s = dot_q<HD>(qs, kp) * scale;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = expf(m_run - m_new);
    const float pj = p <= pos ? expf(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(pj);
    m_run = m_new;
    ps[lane] = pj;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NPL; ++j) o[j] *= alpha;
    const int jmax = min(63, pos - t * 64);
    for (int jj = 0; jj <= jmax; ++jj) {
      const int pp = t * 64 + jj;
      const T* vp = pp < P ? vc + (size_t)pp * HD
                           : vb + (size_t)chain_row(r, pp - P, a.lay) * ldb;
      const float w = ps[jj];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int d = lane + 64 * j;
        if (d < HD) o[j] = fmaf(w, ld_f(vp + d), o[j]);
      }
    }
    __syncthreads();
  }
  T* out = (T*)a.out + (size_t)r * a.H * HD + h * HD;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int d = lane + 64 * j;
    if (d < HD) st_f(out + d, o[j] * inv);
  }
}

// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, one workgroup per row, fixed
// reduction order.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, const T* g, T* y, int d,
                                                 float eps) {
  __shared__ float red[256];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int i = tid; i < d; i += 256) ss = fmaf(xr[i], xr[i], ss);
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float rs = 1.0f / sqrtf(red[0] / (float)d + eps);
  T* yr = y + (size_t)m * d;
  for (int i = tid; i < d; i += 256) st_f(yr + i, xr[i] * rs * ld_f(g + i));
}

template <typename T>
__global__ __launch_bounds__(256) void k_embed(const int32_t* ids, const T* emb, float* x, int d) {
  const int m = blockIdx.x;
  const T* e = emb + (size_t)ids[m] * d;
  for (int i = threadIdx.x; i < d; i += 256) x[(size_t)m * d + i] = ld_f(e + i);
}

// Row argmax with ties to the lowest id: the winner is the maximum of
// (value, -id), which no reduction order can change.
__global__ __launch_bounds__(256) void k_argmax(const float* logits, int V, int32_t* out) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (size_t)m * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int n = tid; n < V; n += 256) {
    const float v = row[n];
    if (v > bv) { bv = v; bi = n; }
  }
  sv[tid] = bv;
  si[tid] = bi;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      const float v2 = sv[tid + s];
      const int i2 = si[tid + s];
      if (v2 > sv[tid] || (v2 == sv[tid] && i2 < si[tid])) { sv[tid] = v2; si[tid] = i2; }
    }
    __syncthreads();
  }
  if (tid == 0) out[m] = si[0];
}

}  // namespace

hipError_t launch_attention(const AttnDesc& a, int dtype, hipStream_t st) {
  dim3 grid(a.H, a.rows);
#define LA_ATTN_CASE(T, HD)                                                  \
  if (a.hd == HD) {                                                          \
    hipLaunchKernelGGL((k_attn<T, HD>), grid, dim3(64), 0, st, a);           \
    return hipGetLastError();                                                \
  }
  if (dtype == LA_BF16) {
    LA_ATTN_CASE(bf16_t, 128)
    LA_ATTN_CASE(bf16_t, 64)
    LA_ATTN_CASE(bf16_t, 32)
    LA_ATTN_CASE(bf16_t, 16)
  } else {
    LA_ATTN_CASE(float, 128)
    LA_ATTN_CASE(float, 64)
    LA_ATTN_CASE(float, 32)
    LA_ATTN_CASE(float, 16)
  }
#undef LA_ATTN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_rmsnorm(const float* x, const void* g, void* y, int rows, int d, float eps,
                          int dtype, hipStream_t st) {
  if (dtype == LA_BF16)
    hipLaunchKernelGGL(k_rmsnorm<bf16_t>, dim3(rows), dim3(256), 0, st, x, (const bf16_t*)g,
                       (bf16_t*)y, d, eps);
  else
    hipLaunchKernelGGL(k_rmsnorm<float>, dim3(rows), dim3(256), 0, st, x, (const float*)g,
                       (float*)y, d, eps);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* ids, const void* emb, float* x, int rows, int d, int dtype,
                        hipStream_t st) {
  if (dtype == LA_BF16)
    hipLaunchKernelGGL(k_embed<bf16_t>, dim3(rows), dim3(256), 0, st, ids, (const bf16_t*)emb, x,
                       d);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(rows), dim3(256), 0, st, ids, (const float*)emb, x, d);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(rows), dim3(256), 0, st, logits, V, out);
  return hipGetLastError();
}
