// Lookahead attention, RMSNorm, embedding gather and per-row argmax.
//
// Attention follows the lookahead mask of [LD] §3.4 "The custom attention
// mask (Figure 2)" without materialising it.  Under the row layout of a step
// (row 0 = current token at P; lookahead row 1+l*W+k at P+1+l+k;
// verification row 1+W(N-1)+g(N-1)+(i-1) at P+i) every row sees exactly one
// key at each position 0..pos(row): committed positions < P come from the KV
// cache, and position P+j comes from the block row `chain_row(row, j)`.
//
// Each row's keys are visited in absolute-position tiles with a fixed
// summation order, so a row's result depends only on the keys it sees, not on
// whether they sit in the cache or in the block, nor on the other rows: the
// verification row that reproduces an autoregressive step gets the bits of
// that step.
#include "la_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

union U4 {
  u32x4_t u;
  bf16x8_t v;
  bf16_t h[8];
};

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

// e^x through the hardware base-2 exponential (v_exp_f32) of x log2(e):
// about 1 ulp in the range the softmax uses, where the library expf spends a
// dozen instructions on range reduction; the softmax of every attention
// step (and of the autoregressive query it must match) uses it.
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504f); }

// float -> bf16 bits, round to nearest even, by the hardware conversion
// (v_cvt_pk_bf16_f32); equal to the integer rounding for finite values
__device__ __forceinline__ uint16_t bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

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

constexpr int AT = 64;  // attention tile (positions)
constexpr int BT = 16;  // granularity of the MFMA part's end

// End of the MFMA part of a row's keys (a multiple of BT): at least D keys
// before the row's own position stay in the per-row part, and never a block
// position (>= P).  A verification row at P+i (i <= D) and the
// autoregressive query at the same position get the same split.  The MFMA
// kernel masks per key, so the per-row part is at most D + BT keys long for
// a verification row.
__device__ __forceinline__ int bulk_end(int pos, int P, int D) {
  int f = pos - D;
  f = f < 0 ? 0 : (f / BT) * BT;
  const int pf = (P / BT) * BT;
  return f < pf ? f : pf;
}

__device__ __forceinline__ int row_pos(const AttnDesc& a, int r, int Pc) {
  return a.pos ? a.pos[r] : Pc + row_offset(r, a.lay);
}

// Per-row part: one wave per (head, row) over positions [F, pos] in tiles of
// TT = 32 positions starting at F (keys from the cache below P, from the
// block chain above); F is a function of pos, so a tile, and the place of
// each key in it, depend only on the row's position.  With D + BT <= TT the
// part is a single tile.  Key slot j of a tile (position base + j) is held by
// the lane pair 2j, 2j+1, each lane with half of the key's dimensions; the
// pair adds its two half dot products low half first.  For the P.V sum lanes
// own output dimensions.  Writes the normalised output after merging the MFMA
// kernel's (m, l, o) partials of [0, F) in chunk order.
constexpr int TT = 32;  // per-row tile (positions)

// half of dot(q, k): dimensions [h0, h0 + HD/2) in four interleaved partial
// sums, each in increasing order, added as (p0+p1)+(p2+p3).  bf16: q is
// kept as bf16 pairs (word w = dimensions 2w, 2w+1 of the half) and pair p
// goes to partial p mod 4 through the packed dot (v_dot2c_f32_bf16: both
// products and the partial added in one instruction); fp32: dimension d
// to partial d mod 4.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int HD>
__device__ __forceinline__ float dot_half(const float* qs, const u32x4_t (&k)[HD / 16], bf16_t) {
  const u32x4_t* qw = (const u32x4_t*)qs;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < HD / 16; ++c) {
    const u32x4_t qv = qw[c];
    const uint32_t qe[4] = {qv.x, qv.y, qv.z, qv.w};
    const uint32_t w[4] = {k[c].x, k[c].y, k[c].z, k[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qe[e]),
                                             __builtin_bit_cast(bf16x2_t, w[e]), a[e], false);
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}
template <int HD>
__device__ __forceinline__ float dot_half(const float* qs, const u32x4_t (&k)[HD / 8], float) {
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < HD / 8; ++c) {
    a[0] = fmaf(qs[4 * c], __uint_as_float(k[c].x), a[0]);
    a[1] = fmaf(qs[4 * c + 1], __uint_as_float(k[c].y), a[1]);
    a[2] = fmaf(qs[4 * c + 2], __uint_as_float(k[c].z), a[2]);
    a[3] = fmaf(qs[4 * c + 3], __uint_as_float(k[c].w), a[3]);
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// LDS ordering inside one wave: its LDS writes are complete and visible to
// all of its lanes (the per-row part uses wave-private LDS).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int HD>
struct TailLds {
  static constexpr int VSTRIDE = HD + 16 / (int)sizeof(T);  // padded LDS row of V
  float qs[HD];
  float ps[TT];
  T vs[TT * VSTRIDE] __attribute__((aligned(16)));
};

// The MFMA kernel's (m, l, o) partials of the chunks of [0, F), merged in
// chunk order with NPRE chunks' loads in flight, then the row's own part;
// the normalised result goes to the output.
template <int HD>
struct PartRing {
  static constexpr int NPRE = 8;
  static constexpr int DPL = HD >= 64 ? HD / 64 : 1;  // output dims per lane
  float pm[NPRE], pl[NPRE], po[NPRE][DPL];
};

template <int HD>
__device__ __forceinline__ void ring_load(const AttnDesc& a, int h, int r, int nch, int sp, int i,
                                          PartRing<HD>& R, int d0, bool down) {
  if (sp < nch) {
    const size_t pb = ((size_t)sp * a.rows + r) * a.H + h;
    R.pm[i] = a.part_ml[pb * 2];
    R.pl[i] = a.part_ml[pb * 2 + 1];
#pragma unroll
    for (int j = 0; j < PartRing<HD>::DPL; ++j) R.po[i][j] = down ? a.part_o[pb * HD + d0 + j] : 0.f;
  }
}

// (m, l, oo) <- (m, l, oo) merged with a state (ms, ls, os)
template <int DPL>
__device__ __forceinline__ void ml_merge(float& m, float& l, float (&oo)[DPL], float ms, float ls,
                                         const float (&os)[DPL]) {
  const float mn = fmaxf(m, ms);
  const float ca = m == -INFINITY ? 0.f : exp_e(m - mn);
  const float cb = exp_e(ms - mn);
  l = l * ca + ls * cb;
#pragma unroll
  for (int j = 0; j < DPL; ++j) oo[j] = oo[j] * ca + os[j] * cb;
  m = mn;
}

template <typename T, int HD>
__device__ __forceinline__ void merge_out(const AttnDesc& a, int h, int r, int nch, float m_run,
                                          float l_run, const float (&o)[PartRing<HD>::DPL],
                                          PartRing<HD>& R, int d0, bool down) {
  constexpr int NPRE = PartRing<HD>::NPRE, DPL = PartRing<HD>::DPL;
  float m = -INFINITY, l = 0.f, oo[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) oo[j] = 0.f;
  for (int sp0 = 0; sp0 < nch; sp0 += NPRE) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      if (sp0 + i < nch) {
        ml_merge<DPL>(m, l, oo, R.pm[i], R.pl[i], R.po[i]);
        ring_load<HD>(a, h, r, nch, sp0 + i + NPRE, i, R, d0, down);
      }
    }
  }
  ml_merge<DPL>(m, l, oo, m_run, l_run, o);
  T* out = (T*)a.out + (size_t)r * a.H * HD + h * HD;
  const float inv = 1.0f / l;
  if (down)
#pragma unroll
    for (int j = 0; j < DPL; ++j) st_f(out + d0 + j, oo[j] * inv);
}

// The per-row part of row r, head h, by one wave (all 64 lanes) on its own
// TailLds, then the merge with the MFMA partials; writes the row's
// normalised output.
template <typename T, int HD>
__device__ __forceinline__ void tail_row(const AttnDesc& a, int h, int r, TailLds<T, HD>& L) {
  constexpr int NV = HD * (int)sizeof(T) / 16;       // 16-byte words per K / V row
  constexpr int NH = NV / 2;                         // words per half row (one lane)
  constexpr int DPL = PartRing<HD>::DPL;             // output dims per lane (contiguous)
  constexpr int VSTRIDE = TailLds<T, HD>::VSTRIDE;
  static_assert(NV % 2 == 0, "a lane holds half a row");
  float* qs = L.qs;
  float* ps = L.ps;
  T* vs = L.vs;
  const int lane = threadIdx.x & 63;
  const int slot = lane >> 1, half = lane & 1;
  const int kvh = h * a.Hkv / a.H;
  const int Pc = a.Pdev ? *a.Pdev : a.P_host;
  const int pos = row_pos(a, r, Pc);
  const int P = a.causal_cache ? pos + 1 : Pc;
  const int F = a.mfma ? bulk_end(pos, P, a.D) : 0;
  const int ldb = a.Hkv * HD;
  const T* q = (const T*)a.q + (size_t)r * a.H * HD + h * HD;
  const T* kc = (const T*)a.kc + (size_t)kvh * a.ld_ctx * HD + half * (HD / 2);
  const T* vc = (const T*)a.vc + (size_t)kvh * a.ld_ctx * HD + half * (HD / 2);
  const T* kb = (const T*)a.kb + kvh * HD + half * (HD / 2);
  const T* vb = (const T*)a.vb + kvh * HD + half * (HD / 2);
  const float scale = 1.0f / sqrtf((float)HD);
  const int d0 = lane * DPL;
  const bool down = d0 < HD;

  float m_run = -INFINITY, l_run = 0.f;
  float o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;

  // the first NPRE chunk partials, loaded now so their latency overlaps the
  // tile below
  const int nch = a.mfma ? attn_nchunks(F) : 0;
  PartRing<HD> R;
#pragma unroll
  for (int i = 0; i < PartRing<HD>::NPRE; ++i) ring_load<HD>(a, h, r, nch, i, i, R, d0, down);
  if (sizeof(T) == 2) {  // bf16 pairs, one word per two dimensions
    for (int i = lane; i < HD / 2; i += 64) ((uint32_t*)qs)[i] = ((const uint32_t*)q)[i];
  } else {
    for (int i = lane; i < HD; i += 64) qs[i] = ld_f(q + i);
  }

  // tiles of TT positions over [F, pos]
  for (int base = F; base <= pos; base += TT) {
    const int p = base + slot;
    const bool on = p <= pos;
    u32x4_t kr[NH], vr[NH];
    if (on) {
      const int src = p < P ? -1 : chain_row(r, p - P, a.lay);
      const u32x4_t* kp = (const u32x4_t*)(src < 0 ? kc + (size_t)p * HD : kb + (size_t)src * ldb);
      const u32x4_t* vp = (const u32x4_t*)(src < 0 ? vc + (size_t)p * HD : vb + (size_t)src * ldb);
#pragma unroll
      for (int e = 0; e < NH; ++e) kr[e] = kp[e];
#pragma unroll
      for (int e = 0; e < NH; ++e) vr[e] = vp[e];
    }
    if (on) {
#pragma unroll
      for (int e = 0; e < NH; ++e)
        *(u32x4_t*)((char*)(vs + slot * VSTRIDE + half * (HD / 2)) + 16 * e) = vr[e];
    }
    wave_lds_sync();
    const float mine =
        on ? dot_half<HD>(qs + half * (sizeof(T) == 2 ? HD / 4 : HD / 2), kr, T()) : 0.f;
    const float other = __shfl_xor(mine, 1, 64);
    const float sc = on ? ((half ? other : mine) + (half ? mine : other)) * scale : -INFINITY;
    const float mp = wave_max(sc);
    const float pv = on ? exp_e(sc - mp) : 0.f;
    if (!half) ps[slot] = pv;
    const float lp = wave_sum(half ? 0.f : pv);
    wave_lds_sync();
    // P.V over this tile: key j goes to partial j mod 4
    float acc[4][DPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[u][j] = 0.f;
    if (down) {
      const int n = min(TT, pos - base + 1);
      // four keys at a time: their weights and values are read together,
      // then key jj + u is added to partial u (keys past n leave it as is)
      for (int jj = 0; jj < n; jj += 4) {
        const float4 w4 = *(const float4*)(ps + jj);
        const float w[4] = {w4.x, w4.y, w4.z, w4.w};
        float vv[4][DPL];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < DPL; ++j) vv[u][j] = ld_f(vs + (jj + u) * VSTRIDE + d0 + j);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < DPL; ++j)
            acc[u][j] = jj + u < n ? fmaf(w[u], vv[u][j], acc[u][j]) : acc[u][j];
      }
    }
    const float mn = fmaxf(m_run, mp);
    const float ca = m_run == -INFINITY ? 0.f : exp_e(m_run - mn);
    const float cb = exp_e(mp - mn);
    l_run = l_run * ca + lp * cb;
#pragma unroll
    for (int j = 0; j < DPL; ++j)
      o[j] = o[j] * ca + ((acc[0][j] + acc[1][j]) + (acc[2][j] + acc[3][j])) * cb;
    m_run = mn;
    wave_lds_sync();
  }

  merge_out<T, HD>(a, h, r, nch, m_run, l_run, o, R, d0, down);
}

template <typename T, int HD>
__global__ __launch_bounds__(64) void k_attn_tail(AttnDesc a) {
  __shared__ TailLds<T, HD> L;
  tail_row<T, HD>(a, blockIdx.x, blockIdx.y, L);
}

// MFMA part (bf16, head_dim 128): one workgroup per (head, prefix chunk
// committed positions, block of 64 or 128 rows).  Each 64-position tile of
// K and V is staged in LDS once and used by every row of the block; wave w
// handles the 16-row group w, or with 128 rows the groups w and w+4, both on
// each tile (group_tiles<2>).
//
// Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
// A = 16 keys x 32 dims of K, B = 32 dims x 16 rows of Q^T), so a lane holds
// 16 scores of one row (row = lane % 16, keys 16kb + 4(lane/16) + e); the
// row's softmax statistics then need a reduction over 4 lanes only, and the
// probabilities are already in the A-operand layout of P.V: for the 32-key
// step j, MFMA slot (lane/16, s) carries key 32j + 4(lane/16) + s (s < 4) or
// 32j + 16 + 4(lane/16) + s - 4, and V is read transposed from LDS with the
// same key order.  A tile that lies past a row's bulk end leaves that row's
// state unchanged (alpha = 1, p = 0).
constexpr int ATT_WIDE_P = 1024;  // committed length from which a workgroup takes 128 rows
constexpr int KSTR = 128 + 8;  // LDS row stride of K (bf16)
constexpr int VSTR = AT + 8;   // LDS row stride of V^T (bf16)

// One 16-row group: its rows' bulk ends F (lane's row = c16) and Q^T
// fragments (zero for rows past `nrows`).
__device__ __forceinline__ void group_load(const AttnDesc& a, int h, int Pc, int row0, int nrows,
                                           int c16, int q4, int& F, U4 (&qf)[4]) {
  const int r = row0 + c16;
  F = 0;
  if (c16 < nrows) {
    const int pos = row_pos(a, r, Pc);
    const int P = a.causal_cache ? pos + 1 : Pc;
    F = bulk_end(pos, P, a.D);
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (c16 < nrows)
      qf[ks].u = *(const u32x4_t*)((const bf16_t*)a.q + (size_t)r * a.H * 128 + h * 128 +
                                   ks * 32 + q4 * 8);
    else
      qf[ks].u = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// The online-softmax update of NG 16-row groups of one wave from the 64-key
// tile [t0, t0 + 64) staged in Ks / Vt; keys at or past a row's F are
// masked.  With NG = 2 the steps of the two groups interleave (the K
// fragment of each MFMA and the V^T fragment of each P.V step are read from
// LDS once for both, and one group's shuffle and exponential latencies
// overlap the other's); each group's arithmetic is the same for NG = 1 and
// NG = 2, which a verification row (two groups per wave at 121 rows) and the
// autoregressive query at its position (one group) rely on for bit-identical
// outputs.  No fused multiply-adds: otherwise the compiler fuses the score
// scaling into the exponent's subtraction in one instance and not the other.
// A group whose rows all end before the tile takes alpha = 1 and p = 0 for
// every row, which leaves its state bit for bit unchanged.
template <int NG>
__device__ __forceinline__ void group_tiles(const bf16_t* Ks, const bf16_t* Vt, int t0,
                                            const int (&F)[2], const U4 (&qf)[2][4],
                                            f32x4_t (&o)[2][8], float (&m_run)[2],
                                            float (&l_run)[2], int c16, int q4, float scale) {
#pragma clang fp contract(off)
  // keys [t0, F) of the tile are this lane's row's (F a multiple of BT)
  int nv[NG];
  bool any = false;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    nv[gi] = F[gi] - t0;
    any = any || nv[gi] > 0;
  }
  // skip the tile when it is past every row of the groups
  if (!__any(any)) return;
  f32x4_t st[NG][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) st[gi][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      U4 ka;
      ka.u = *(const u32x4_t*)(&Ks[(kb * 16 + c16) * KSTR + ks * 32 + q4 * 8]);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        st[gi][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.v, qf[gi][ks].v, st[gi][kb], 0, 0, 0);
    }
  }
  float mt[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    mt[gi] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = kb * 16 + 4 * q4 + e < nv[gi] ? st[gi][kb][e] * scale : -INFINITY;
        st[gi][kb][e] = sv;
        mt[gi] = fmaxf(mt[gi], sv);
      }
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) mt[gi] = fmaxf(mt[gi], __shfl_xor(mt[gi], 16, 64));
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) mt[gi] = fmaxf(mt[gi], __shfl_xor(mt[gi], 32, 64));
  // p enters the PV product as the sum of two bf16 values, hi = bf16(p)
  // and lo = bf16(p - hi) (p - hi is exact in fp32), so the product
  // carries p to about 2^-17 relative, as an fp32 product would: no
  // rounding of the probabilities beyond the fp32 arithmetic
  float alpha[NG], m_new[NG], ls[NG];
  U4 pa[NG][2], pl[NG][2];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    m_new[gi] = fmaxf(m_run[gi], mt[gi]);
    alpha[gi] = m_new[gi] == -INFINITY ? 1.0f : exp_e(m_run[gi] - m_new[gi]);
    ls[gi] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = kb * 16 + 4 * q4 + e < nv[gi] ? exp_e(st[gi][kb][e] - m_new[gi]) : 0.f;
        ls[gi] += pv;
        const uint16_t hb = bf16_rne(pv);
        pa[gi][kb >> 1].h[(kb & 1) * 4 + e] = hb;
        pl[gi][kb >> 1].h[(kb & 1) * 4 + e] = bf16_rne(pv - __uint_as_float((uint32_t)hb << 16));
      }
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) ls[gi] += __shfl_xor(ls[gi], 16, 64);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) ls[gi] += __shfl_xor(ls[gi], 32, 64);
  // rescale O rows 4*q4 + e by their row's alpha (held by lane 4*q4 + e)
  float al[NG][4];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    l_run[gi] = l_run[gi] * alpha[gi] + ls[gi];
    m_run[gi] = m_new[gi];
#pragma unroll
    for (int e = 0; e < 4; ++e) al[gi][e] = __shfl(alpha[gi], q4 * 4 + e, 64);
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[gi][db][e] *= al[gi][e];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16_t* vr = &Vt[(db * 16 + c16) * VSTR + 32 * j + 4 * q4];
      U4 vb;
      const u32x2_t lo = *(const u32x2_t*)vr;
      const u32x2_t hi = *(const u32x2_t*)(vr + 16);
      vb.u = u32x4_t{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        o[gi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[gi][j].v, vb.v, o[gi][db], 0, 0, 0);
        o[gi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[gi][j].v, vb.v, o[gi][db], 0, 0, 0);
      }
    }
  }
}

// A group's (m, l) and unnormalised O of one chunk -> part_ml / part_o.
__device__ __forceinline__ void group_store(const AttnDesc& a, int split, int h, int row0,
                                            int nrows, const f32x4_t (&o)[8], float m_run,
                                            float l_run, int lane) {
  const int c16 = lane & 15, q4 = lane >> 4;
  if (lane < 16 && c16 < nrows) {
    float* pm = a.part_ml + (((size_t)split * a.rows + row0 + c16) * a.H + h) * 2;
    pm[0] = m_run;
    pm[1] = l_run;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int rl = q4 * 4 + e;
    if (rl >= nrows) continue;
    float* po = a.part_o + (((size_t)split * a.rows + row0 + rl) * a.H + h) * 128;
#pragma unroll
    for (int db = 0; db < 8; ++db) po[db * 16 + c16] = o[db][e];
  }
}

// Register budget of two waves per SIMD (two workgroups per compute unit):
// with one, a long prefix's chunks run in five rounds over the chip, and a
// tile's fetch latency is hidden by nothing but the workgroup's own math.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bulk(AttnDesc a) {
  __shared__ __align__(16) bf16_t Ks[AT * KSTR];
  __shared__ __align__(16) bf16_t Vt[128 * VSTR];
  // chunks grow with position (64 to 512 keys): the largest are dispatched
  // first, so the short ones fill the compute units they leave, instead of
  // the long ones starting last and setting the kernel's end
  const int h = blockIdx.x, split = a.nsplit - 1 - (int)blockIdx.y, rb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, q4 = lane >> 4;
  const int kvh = h * a.Hkv / a.H;
  const int Pc = a.Pdev ? *a.Pdev : a.P_host;
  // The grid has one z index per 64 rows.  Below ATT_WIDE_P committed
  // positions (few chunks, one or two tiles each) each workgroup takes its
  // 64 rows, one 16-row group per wave, so twice as many workgroups share
  // the work; from ATT_WIDE_P on, even z indices take 128 rows (two groups
  // per wave, each K/V tile serving both) and odd ones have nothing to do.
  // A row's arithmetic is the same either way (group_tiles<1> and <2>).
  const bool wide = Pc >= ATT_WIDE_P;
  if (wide && (rb & 1)) return;
  const int row0 = rb * 64;
  const int nrows = min(wide ? 128 : 64, a.rows - row0);
  const int ngroups = (nrows + 15) >> 4;
  const int s0 = attn_chunk_start(split);
  const bf16_t* kc = (const bf16_t*)a.kc + (size_t)kvh * a.ld_ctx * 128;
  const bf16_t* vc = (const bf16_t*)a.vc + (size_t)kvh * a.ld_ctx * 128;
  const float scale = 1.0f / sqrtf(128.0f);

  // this wave's row groups w and w + 4
  int F[2];
  bool gon[2];
  U4 qf[2][4];
  f32x4_t o[2][8];
  float m_run[2], l_run[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int g = wave + 4 * gi;
    gon[gi] = g < ngroups;
    group_load(a, h, Pc, row0 + g * 16, gon[gi] ? min(16, nrows - g * 16) : 0, c16, q4, F[gi],
               qf[gi]);
#pragma unroll
    for (int db = 0; db < 8; ++db) o[gi][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[gi] = -INFINITY;
    l_run[gi] = 0.f;
  }
  // the workgroup's furthest bulk end bounds the tile loop
  __shared__ int s_fmax;
  if (tid == 0) s_fmax = 0;
  __syncthreads();
  atomicMax(&s_fmax, max(F[0], F[1]));
  __syncthreads();
  const int tend = min(attn_chunk_start(split + 1), s_fmax);
  // no row of the workgroup has keys in this chunk: the per-row kernel reads
  // none of its partials
  if (tend <= s0) return;

  // K [key][dim] and V^T [dim][key] of a 64-position tile: each thread holds
  // 32 dims of one key of K and 16 dims of a key pair of V, fetched one tile
  // ahead so the loads of tile t+1 overlap the arithmetic of tile t.  Keys
  // at or past tend (past every row's MFMA part, possibly never written)
  // are staged as zeros: masked rows then add exactly 0 * 0.  The loaded
  // words are only selected at the LDS store, so nothing waits for the
  // loads before the tile's arithmetic.
  const int fkey = tid >> 2, fseg = tid & 3;  // K: 32 dims per thread
  const int fkp = tid & 31, fvs = tid >> 5;   // V: key pair, 16-dim segment
  u32x4_t kf[4], va[2], vb[2];
  bool kok = false, v0ok = false, v1ok = false;
  const u32x4_t z4 = u32x4_t{0u, 0u, 0u, 0u};
  auto fetch = [&](int t0) __attribute__((always_inline)) {
    // addresses clamped to key tend-1 (a tile may reach past the cache's
    // capacity); the words of such keys are replaced by zeros at the store
    const int k0 = t0 + fkey, v0k = t0 + 2 * fkp;
    const int kl = min(k0, tend - 1), v0l = min(v0k, tend - 1), v1l = min(v0k + 1, tend - 1);
    const u32x4_t* src = (const u32x4_t*)(kc + (size_t)kl * 128 + fseg * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) kf[j] = src[j];
    const u32x4_t* v0 = (const u32x4_t*)(vc + (size_t)v0l * 128 + fvs * 16);
    const u32x4_t* v1 = (const u32x4_t*)(vc + (size_t)v1l * 128 + fvs * 16);
    va[0] = v0[0];
    va[1] = v0[1];
    vb[0] = v1[0];
    vb[1] = v1[1];
    kok = k0 < tend;
    v0ok = v0k < tend;
    v1ok = v0k + 1 < tend;
  };
  fetch(s0);
  for (int t0 = s0; t0 < tend; t0 += AT) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4_t*)(&Ks[fkey * KSTR + fseg * 32 + j * 8]) = kok ? kf[j] : z4;
    U4 va0, va1, vb0, vb1;
    va0.u = v0ok ? va[0] : z4;
    va1.u = v0ok ? va[1] : z4;
    vb0.u = v1ok ? vb[0] : z4;
    vb1.u = v1ok ? vb[1] : z4;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      *(uint32_t*)(&Vt[(fvs * 16 + d) * VSTR + 2 * fkp]) =
          (uint32_t)va0.h[d] | ((uint32_t)vb0.h[d] << 16);
      *(uint32_t*)(&Vt[(fvs * 16 + 8 + d) * VSTR + 2 * fkp]) =
          (uint32_t)va1.h[d] | ((uint32_t)vb1.h[d] << 16);
    }
    __syncthreads();
    if (t0 + AT < tend) fetch(t0 + AT);
    if (gon[1])
      group_tiles<2>(Ks, Vt, t0, F, qf, o, m_run, l_run, c16, q4, scale);
    else if (gon[0])
      group_tiles<1>(Ks, Vt, t0, F, qf, o, m_run, l_run, c16, q4, scale);
    __syncthreads();
  }
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int g = wave + 4 * gi;
    if (gon[gi]) group_store(a, split, h, row0 + g * 16, min(16, nrows - g * 16), o[gi], m_run[gi],
                             l_run[gi], lane);
  }
}

// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, one workgroup per row; each
// thread adds the squares of its 4-column groups in order, then the sums
// are added by a fixed shuffle tree per wave and the 4 wave sums in order.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, const T* g, T* y, int d,
                                                 float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int i = tid * 4; i < d; i += 1024) {
    const float4 v = *(const float4*)(xr + i);
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = 1.0f / sqrtf(tot / (float)d + eps);
  T* yr = y + (size_t)m * d;
  for (int i = tid * 4; i < d; i += 1024) {
    const float4 v = *(const float4*)(xr + i);
    st_f(yr + i, v.x * rs * ld_f(g + i));
    st_f(yr + i + 1, v.y * rs * ld_f(g + i + 1));
    st_f(yr + i + 2, v.z * rs * ld_f(g + i + 2));
    st_f(yr + i + 3, v.w * rs * ld_f(g + i + 3));
  }
}

// Embedding gather to the fp32 residual stream, eight columns per thread.
__device__ __forceinline__ void ld8(const bf16_t* p, float (&v)[8]) {
  const u32x4_t u = *(const u32x4_t*)p;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(256) void k_embed(const int32_t* ids, const T* emb, float* x, int d) {
  const int m = blockIdx.x;
  const T* e = emb + (size_t)ids[m] * d;
  float* xr = x + (size_t)m * d;
  for (int i = threadIdx.x * 8; i < d; i += 2048) {
    float v[8];
    ld8(e + i, v);
    *(float4*)(xr + i) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(xr + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Row argmax with ties to the lowest id: the winner is the maximum of
// (value, -id), which no reduction order can change.  1024 threads per row;
// with V a multiple of 4 each thread reads 16-byte groups (a 32000-entry row
// in one pass), eight independent chains per thread, then shuffle and LDS
// combines.
__device__ __forceinline__ void amax_take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

template <bool VEC>
__global__ __launch_bounds__(1024) void k_argmax(const float* logits, int V, int32_t* out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* row = logits + (size_t)m * V;
  float bv8[8];
  int bi8[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) { bv8[u] = -INFINITY; bi8[u] = 0x7fffffff; }
  if (VEC) {
    const int ng = V / 4;
    for (int g0 = tid; g0 < ng; g0 += 8 * 1024) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (g0 + u * 1024 < ng) v[u] = *(const float4*)(row + 4 * (g0 + u * 1024));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = 4 * (g0 + u * 1024);
        if (g0 + u * 1024 < ng) {
          amax_take(bv8[u], bi8[u], v[u].x, i);
          amax_take(bv8[u], bi8[u], v[u].y, i + 1);
          amax_take(bv8[u], bi8[u], v[u].z, i + 2);
          amax_take(bv8[u], bi8[u], v[u].w, i + 3);
        }
      }
    }
  } else {
    for (int n0 = tid; n0 < V; n0 += 8 * 1024) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (n0 + u * 1024 < V) amax_take(bv8[u], bi8[u], row[n0 + u * 1024], n0 + u * 1024);
    }
  }
  float bv = bv8[0];
  int bi = bi8[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) amax_take(bv, bi, bv8[u], bi8[u]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    amax_take(bv, bi, v2, i2);
  }
  if (lane == 0) { sv[wv] = bv; si[wv] = bi; }
  __syncthreads();
  if (tid == 0) {
    float b = sv[0];
    int i = si[0];
    for (int w = 1; w < 16; ++w) amax_take(b, i, sv[w], si[w]);
    out[m] = i;
  }
}

// Row argmax from the LM head's per-block keys: one wave per row, the
// largest key (any order gives it), its column.
__global__ __launch_bounds__(64) void k_argmax_keys(const unsigned long long* keys, int nblk,
                                                    int32_t* out) {
  const int m = blockIdx.x, lane = threadIdx.x;
  const unsigned long long* row = keys + (size_t)m * nblk;
  unsigned long long best = 0;
  for (int b = lane; b < nblk; b += 64) best = row[b] > best ? row[b] : best;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned int lo = __shfl_xor((unsigned int)best, o, 64);
    const unsigned int hi = __shfl_xor((unsigned int)(best >> 32), o, 64);
    const unsigned long long k = ((unsigned long long)hi << 32) | lo;
    best = k > best ? k : best;
  }
  if (lane == 0) out[m] = (int32_t)(0xFFFFFFFFu - (unsigned int)best);
}

}  // namespace

hipError_t launch_argmax_keys(const unsigned long long* keys, int rows, int nblk, int32_t* out,
                              hipStream_t st) {
  la_launch(k_argmax_keys, dim3(rows), dim3(64), 0, st, keys, nblk, out);
  return hipGetLastError();
}

int attn_uses_mfma(int dtype, int hd) { return dtype == LA_BF16 && hd == 128; }

size_t attn_part_floats(int nsplit, int rows, int H, int hd) {
  return (size_t)nsplit * rows * H * (hd + 2);
}

hipError_t launch_attention(const AttnDesc& a, int dtype, hipStream_t st) {
  dim3 grid(a.H, a.rows);
  if (a.mfma) {
    if (dtype != LA_BF16 || a.hd != 128 || a.nsplit < 1)
      return hipErrorInvalidValue;
    la_launch(k_attn_bulk, dim3(a.H, a.nsplit, (a.rows + 63) / 64), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    la_launch((k_attn_tail<bf16_t, 128>), grid, dim3(64), 0, st, a);
    return hipGetLastError();
  }
#define LA_ATTN_CASE(T, HD)                                                  \
  if (a.hd == HD) {                                                          \
    la_launch((k_attn_tail<T, HD>), grid, dim3(64), 0, st, a);               \
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
    la_launch(k_rmsnorm<bf16_t>, dim3(rows), dim3(256), 0, st, x, (const bf16_t*)g,
              (bf16_t*)y, d, eps);
  else
    la_launch(k_rmsnorm<float>, dim3(rows), dim3(256), 0, st, x, (const float*)g,
              (float*)y, d, eps);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* ids, const void* emb, float* x, int rows, int d, int dtype,
                        hipStream_t st) {
  if (dtype == LA_BF16)
    la_launch(k_embed<bf16_t>, dim3(rows), dim3(256), 0, st, ids, (const bf16_t*)emb, x, d);
  else
    la_launch(k_embed<float>, dim3(rows), dim3(256), 0, st, ids, (const float*)emb, x, d);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* out, hipStream_t st) {
  if (V % 4 == 0)
    la_launch(k_argmax<true>, dim3(rows), dim3(1024), 0, st, logits, V, out);
  else
    la_launch(k_argmax<false>, dim3(rows), dim3(1024), 0, st, logits, V, out);
  return hipGetLastError();
}
