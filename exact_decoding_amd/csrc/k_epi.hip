// Epilogues of the split projection GEMM: each sums the K pieces of an
// output element in K order (the piece count of its column block comes from
// the split plan) and applies what the decoder does next: RoPE and the q, k,
// v stores (k_qkv_epi), the residual add fused with the next RMSNorm
// (k_resid_norm), SiLU(gate) * up (k_silu_epi), or a plain sum (k_sum_epi,
// the GEMM test hook).  The *4 variants handle four consecutive columns per
// thread with 16-byte loads; the others serve widths that do not fill a
// wave that way.
#include "la_internal.h"

typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int NWG = GEMM_NWG;

// Sum of the pieces of one output element, in K order.  NP is a
// compile-time bound (>= the plan's np) so the loads are issued together.
template <int NP>
__device__ __forceinline__ float sum_pieces(const float* __restrict__ part, const SplitPlan& sp,
                                            int rows_pad, int N, int m, int col) {
  if (NP == 1) return part[(size_t)m * N + col];
  const int np = plan_pieces(sp, col / NWG);
  float p[NP];
#pragma unroll
  for (int s = 0; s < NP; ++s) p[s] = s < np ? part[((size_t)s * rows_pad + m) * N + col] : 0.f;
  float v = p[0];
#pragma unroll
  for (int s = 1; s < NP; ++s)
    if (s < np) v += p[s];
  return v;
}

// The same sum for four consecutive columns (col a multiple of 4, N too; the
// four share a column block), with 16-byte loads.  The pieces are read once:
// the loads carry the streaming hint, so they do not push the x tiles, KV
// rows and other reused data out of the L2.
template <int NP>
__device__ __forceinline__ f32x4_t sum_pieces4(const float* __restrict__ part, const SplitPlan& sp,
                                               int rows_pad, int N, int m, int col) {
  if (NP == 1) return __builtin_nontemporal_load((const f32x4_t*)(part + (size_t)m * N + col));
  const int np = plan_pieces(sp, col / NWG);
  f32x4_t p[NP];
#pragma unroll
  for (int s = 0; s < NP; ++s)
    p[s] = s < np ? __builtin_nontemporal_load((const f32x4_t*)(part + ((size_t)s * rows_pad + m) * N + col))
                  : f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t v = p[0];
#pragma unroll
  for (int s = 1; s < NP; ++s)
    if (s < np) v += p[s];
  return v;
}

// four values of the model dtype at p (4-element aligned)
__device__ __forceinline__ f32x4_t ld4(const bf16_t* p) {
  const u32x2_t u = *(const u32x2_t*)p;
  return f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
}
__device__ __forceinline__ f32x4_t ld4(const float* p) { return *(const f32x4_t*)p; }
__device__ __forceinline__ void st4(bf16_t* p, f32x4_t v) {
  const uint32_t a = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
  const uint32_t b = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
  *(u32x2_t*)p = u32x2_t{a, b};
}
__device__ __forceinline__ void st4(float* p, f32x4_t v) { *(f32x4_t*)p = v; }

#define LA_SPLIT_DISPATCH(NP_, CALL)          \
  if ((NP_) <= 1) { CALL(1); }                \
  else if ((NP_) <= 2) { CALL(2); }           \
  else if ((NP_) <= 4) { CALL(4); }           \
  else if ((NP_) <= 8) { CALL(8); }           \
  else if ((NP_) <= 16) { CALL(16); }         \
  else return hipErrorInvalidValue;

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
    const float x1 = sum_pieces<S>(e.part, e.sp, e.rows_pad, e.N, m, col);
    const float x2 = sum_pieces<S>(e.part, e.sp, e.rows_pad, e.N, m, col + half);
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
    const float v = sum_pieces<S>(e.part, e.sp, e.rows_pad, e.N, m, nq + nk + vi);
    const int kvh = vi / hd, i = vi - kvh * hd;
    T* vd = (T*)e.vdst;
    T* dst = e.dest == QKV_TO_BLOCK ? vd + (size_t)m * nk + vi
                                    : vd + ((size_t)kvh * e.ld_ctx + pos) * hd + i;
    st_f(dst, v);
  }
}

// k_qkv_epi with four consecutive pairs (or v elements) per thread.
template <typename T, int S>
__global__ __launch_bounds__(256) void k_qkv_epi4(QkvEpi e) {
  const int m = blockIdx.y;
  const int u = blockIdx.x * 256 + threadIdx.x;
  const int hd = e.hd, half = hd >> 1, hq = half >> 2;
  const int nq = e.H * hd, nk = e.Hkv * hd;
  const int npair = (e.H + e.Hkv) * hq;
  if (u >= npair + (nk >> 2)) return;
  const int pos = e.pos[m];
  if (u < npair) {
    const int hh = u / hq, i = (u - hh * hq) * 4;
    const int col = hh * hd + i;
    const f32x4_t x1 = sum_pieces4<S>(e.part, e.sp, e.rows_pad, e.N, m, col);
    const f32x4_t x2 = sum_pieces4<S>(e.part, e.sp, e.rows_pad, e.N, m, col + half);
    const f32x4_t* cs = (const f32x4_t*)(e.rope + (size_t)pos * half + i);  // (c, s) pairs
    const f32x4_t c01 = cs[0], c23 = cs[1];
    const f32x4_t c = {c01.x, c01.z, c23.x, c23.z}, sn = {c01.y, c01.w, c23.y, c23.w};
    const f32x4_t y1 = x1 * c - x2 * sn;
    const f32x4_t y2 = x1 * sn + x2 * c;
    T* dst;
    if (hh < e.H) {
      dst = (T*)e.q + (size_t)m * nq + hh * hd + i;
    } else {
      const int kvh = hh - e.H;
      T* kd = (T*)e.kdst;
      dst = e.dest == QKV_TO_BLOCK ? kd + (size_t)m * nk + kvh * hd + i
                                   : kd + ((size_t)kvh * e.ld_ctx + pos) * hd + i;
    }
    st4(dst, y1);
    st4(dst + half, y2);
  } else {
    const int vi = (u - npair) * 4;
    const f32x4_t v = sum_pieces4<S>(e.part, e.sp, e.rows_pad, e.N, m, nq + nk + vi);
    const int kvh = vi / hd, i = vi - kvh * hd;
    T* vd = (T*)e.vdst;
    T* dst = e.dest == QKV_TO_BLOCK ? vd + (size_t)m * nk + vi
                                    : vd + ((size_t)kvh * e.ld_ctx + pos) * hd + i;
    st4(dst, v);
  }
}

// k_resid_norm with four consecutive columns per thread: thread t owns
// columns 4(t + j*blockDim) .. +3, j < NC; the sum of squares is reduced in
// a fixed order (per thread, then xor-shuffles within a wave, then across
// waves in wave order).
template <typename T, int S, int NC>
__global__ __launch_bounds__(1024) void k_resid_norm4(const float* __restrict__ part, SplitPlan sp,
                                                      int rows_pad, int d, float* __restrict__ x,
                                                      const T* __restrict__ g, T* __restrict__ h,
                                                      float eps) {
  __shared__ float red[16];
  const int m = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  float* xr = x + (size_t)m * d;
  f32x4_t v[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) v[j] = sum_pieces4<S>(part, sp, rows_pad, d, m, 4 * (tid + j * nt));
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    f32x4_t* xp = (f32x4_t*)(xr + 4 * (tid + j * nt));
    v[j] = *xp + v[j];
    *xp = v[j];
    ss = fmaf(v[j].x, v[j].x, ss);
    ss = fmaf(v[j].y, v[j].y, ss);
    ss = fmaf(v[j].z, v[j].z, ss);
    ss = fmaf(v[j].w, v[j].w, ss);
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
  for (int j = 0; j < NC; ++j) {
    const int c = 4 * (tid + j * nt);
    st4(hr + c, v[j] * rs * ld4(g + c));
  }
}

// k_silu_epi with four consecutive features per thread.
template <typename T, int S>
__global__ __launch_bounds__(256) void k_silu_epi4(const float* part, SplitPlan sp, int rows_pad,
                                                   int F, T* act) {
  const int m = blockIdx.y;
  const int f = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (f >= F) return;
  const f32x4_t gt = sum_pieces4<S>(part, sp, rows_pad, 2 * F, m, f);
  const f32x4_t up = sum_pieces4<S>(part, sp, rows_pad, 2 * F, m, F + f);
  f32x4_t y;
#pragma unroll
  for (int k = 0; k < 4; ++k) y[k] = gt[k] / (1.0f + expf(-gt[k])) * up[k];
  st4(act + (size_t)m * F + f, y);
}

// x[m] += sum of the pieces (in K order); then
// h[m] = x[m] / sqrt(mean(x^2) + eps) * g: the residual add fused with the
// next RMSNorm.  One workgroup of d/NC threads per row; thread t owns columns
// t + j*blockDim; the sum of squares is reduced in a fixed order (within a
// wave by xor-shuffles, then across waves in wave order).
template <typename T, int S, int NC>
__global__ __launch_bounds__(1024) void k_resid_norm(const float* __restrict__ part, SplitPlan sp,
                                                     int rows_pad,
                                                     int d, float* __restrict__ x,
                                                     const T* __restrict__ g, T* __restrict__ h,
                                                     float eps) {
  __shared__ float red[16];
  const int m = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  float* xr = x + (size_t)m * d;
  float v[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) v[j] = sum_pieces<S>(part, sp, rows_pad, d, m, tid + j * nt);
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
__global__ __launch_bounds__(256) void k_sum_epi(const float* part, SplitPlan sp, int rows_pad,
                                                 int N, float* y) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  y[(size_t)m * N + n] = sum_pieces<S>(part, sp, rows_pad, N, m, n);
}

template <typename T, int S>
__global__ __launch_bounds__(256) void k_silu_epi(const float* part, SplitPlan sp, int rows_pad,
                                                  int F, T* act) {
  const int m = blockIdx.y;
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const float gt = sum_pieces<S>(part, sp, rows_pad, 2 * F, m, f);
  const float up = sum_pieces<S>(part, sp, rows_pad, 2 * F, m, F + f);
  const float sg = gt / (1.0f + expf(-gt));
  st_f(act + (size_t)m * F + f, sg * up);
}

}  // namespace

hipError_t launch_qkv_epi(const QkvEpi& e, int dtype, hipStream_t st) {
  if (e.hd % 8 == 0 && e.N % 4 == 0) {  // four pairs per thread
    const int units = (e.H + e.Hkv) * (e.hd / 8) + e.Hkv * e.hd / 4;
    dim3 grid((units + 255) / 256, e.rows);
#define LA_QKV4(S_)                                                             \
  if (dtype == LA_BF16)                                                         \
    la_launch((k_qkv_epi4<bf16_t, S_>), grid, dim3(256), 0, st, e);             \
  else                                                                          \
    la_launch((k_qkv_epi4<float, S_>), grid, dim3(256), 0, st, e);
    LA_SPLIT_DISPATCH(e.sp.np, LA_QKV4)
#undef LA_QKV4
    return hipGetLastError();
  }
  const int units = (e.H + e.Hkv) * (e.hd / 2) + e.Hkv * e.hd;
  dim3 grid((units + 255) / 256, e.rows);
#define LA_QKV(S_)                                                              \
  if (dtype == LA_BF16)                                                         \
    la_launch((k_qkv_epi<bf16_t, S_>), grid, dim3(256), 0, st, e);              \
  else                                                                          \
    la_launch((k_qkv_epi<float, S_>), grid, dim3(256), 0, st, e);
  LA_SPLIT_DISPATCH(e.sp.np, LA_QKV)
#undef LA_QKV
  return hipGetLastError();
}

// columns per thread for a row of d values in one workgroup (<= 1024 threads)
static int norm_nc(int d) {
  for (int nc = 1; nc <= 16; ++nc)
    if (d % nc == 0 && d / nc <= 1024 && (d / nc) % 64 == 0) return nc;
  return 0;
}

hipError_t launch_resid_norm(const float* part, const SplitPlan& sp, int rows_pad, int d,
                             int rows, float* x, const void* g, void* h, float eps, int dtype,
                             hipStream_t st) {
  const int nc4 = d % 4 == 0 ? norm_nc(d / 4) : 0;
  if (nc4) {  // four columns per thread
    const dim3 blk(d / 4 / nc4);
#define LA_RQ2(S_, NC_)                                                                        \
  if (dtype == LA_BF16)                                                                        \
    la_launch((k_resid_norm4<bf16_t, S_, NC_>), dim3(rows), blk, 0, st, part, sp,              \
              rows_pad, d, x, (const bf16_t*)g, (bf16_t*)h, eps);                              \
  else                                                                                         \
    la_launch((k_resid_norm4<float, S_, NC_>), dim3(rows), blk, 0, st, part, sp,               \
              rows_pad, d, x, (const float*)g, (float*)h, eps);
#define LA_RQ(S_)                                                       \
  switch (nc4) {                                                        \
    case 1: LA_RQ2(S_, 1) break;                                        \
    case 2: LA_RQ2(S_, 2) break;                                        \
    case 4: LA_RQ2(S_, 4) break;                                        \
    case 5: LA_RQ2(S_, 5) break;                                        \
    default: return hipErrorInvalidValue;                               \
  }
    LA_SPLIT_DISPATCH(sp.np, LA_RQ)
#undef LA_RQ
#undef LA_RQ2
    return hipGetLastError();
  }
  const int nc = norm_nc(d);
  if (!nc) return hipErrorInvalidValue;
  const dim3 blk(d / nc);
#define LA_RN2(S_, NC_)                                                                        \
  if (dtype == LA_BF16)                                                                        \
    la_launch((k_resid_norm<bf16_t, S_, NC_>), dim3(rows), blk, 0, st, part, sp,               \
              rows_pad, d, x, (const bf16_t*)g, (bf16_t*)h, eps);                              \
  else                                                                                         \
    la_launch((k_resid_norm<float, S_, NC_>), dim3(rows), blk, 0, st, part, sp,                \
              rows_pad, d, x, (const float*)g, (float*)h, eps);
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
  LA_SPLIT_DISPATCH(sp.np, LA_RN)
#undef LA_RN
#undef LA_RN2
  return hipGetLastError();
}

hipError_t launch_sum_epi(const float* part, const SplitPlan& sp, int rows_pad, int N, int rows,
                          float* y, hipStream_t st) {
#define LA_SE(S_)                                                                           \
  la_launch((k_sum_epi<S_>), dim3((N + 255) / 256, rows), dim3(256), 0, st, part, sp,       \
            rows_pad, N, y);
  LA_SPLIT_DISPATCH(sp.np, LA_SE)
#undef LA_SE
  return hipGetLastError();
}

hipError_t launch_silu_epi(const float* part, const SplitPlan& sp, int rows_pad, int F, int rows,
                           void* act, int dtype, hipStream_t st) {
  if (F % 4 == 0) {  // four features per thread
    const dim3 grid((F / 4 + 255) / 256, rows);
#define LA_SQ(S_)                                                                               \
  if (dtype == LA_BF16)                                                                         \
    la_launch((k_silu_epi4<bf16_t, S_>), grid, dim3(256), 0, st, part, sp, rows_pad,            \
              F, (bf16_t*)act);                                                                 \
  else                                                                                          \
    la_launch((k_silu_epi4<float, S_>), grid, dim3(256), 0, st, part, sp, rows_pad,             \
              F, (float*)act);
    LA_SPLIT_DISPATCH(sp.np, LA_SQ)
#undef LA_SQ
    return hipGetLastError();
  }
#define LA_SI(S_)                                                                              \
  if (dtype == LA_BF16)                                                                        \
    la_launch((k_silu_epi<bf16_t, S_>), dim3((F + 255) / 256, rows), dim3(256), 0, st,         \
              part, sp, rows_pad, F, (bf16_t*)act);                                            \
  else                                                                                         \
    la_launch((k_silu_epi<float, S_>), dim3((F + 255) / 256, rows), dim3(256), 0, st,          \
              part, sp, rows_pad, F, (float*)act);
  LA_SPLIT_DISPATCH(sp.np, LA_SI)
#undef LA_SI
  return hipGetLastError();
}
