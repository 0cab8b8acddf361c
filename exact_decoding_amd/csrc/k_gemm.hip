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

#include <type_traits>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int NWG = GEMM_NWG;  // output columns per workgroup (4 waves x 2 tiles x 16)
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

// One workgroup: rows [mb*128, mb*128 + 16*MT) x the run of (column block,
// K chunk) units that the split plan deals to workgroup blockIdx.x: n <= nch
// chunks, the first nA of them chunks cA.. of column block bA, the rest
// chunks 0.. of block bA + 1.  Five waves:
//  * waves 0-3 (consumers) own 32 columns each (two 16-column MFMA tiles) for
//    all MT row tiles; each keeps PF chunks of its weight rows in flight in
//    registers and issues no other global load until its stores at the end,
//    so its in-order load counter never makes it wait on anything but the
//    chunk it is about to use.  The weight stream runs on across the block
//    boundary; there the accumulators of block bA are parked in LDS (LDS
//    traffic does not touch that counter);
//  * wave 4 (producer) stages the x tile of each chunk into a ring of XR LDS
//    stages, XR-1 chunks ahead of the consumers, from a 2-deep register ring.
// One barrier per chunk; the producer writes the stage the consumers left
// at the previous barrier.
//
// Weights come in the packed layout (see la.h): MFMA step j of chunk c of a
// 16-row stripe is one contiguous KB holding, for lane (q = lane/16,
// r = lane%16), k in [64c + 32j + 8q, +8) of row r; the x tile is read with
// the same k order.  The stripes of one 128-row column block sit side by
// side for each chunk, and the chunks of a block, then the blocks, follow
// each other: the (column block, K chunk) units lie in memory in the order
// the split plan deals them out, so every workgroup streams one contiguous
// range whatever the plan.  LDS x rows are 128 bytes with the 16-byte pieces
// XOR-swizzled by (row/2) mod 8 so the A-fragment reads hit distinct banks.
constexpr int XR = 3;  // LDS stages of the x tile

__device__ __forceinline__ int xswz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// The argmax keys of column block b (one whole block) for rows row0 ..
// row0 + nr - 1, from its values in LDS: row rr, local column c at
// vs[(c / 32) * ld_wave + rr * ld_row + c % 32].  Each row's 128 columns are
// cut into 16 runs of 8 taken by different threads (partial keys in kp,
// LDS, nr * 16 of them), then thread rr takes the largest of its row's 16.
// The caller has synchronised the workgroup after writing vs.
__device__ __forceinline__ void block_row_keys(const GemmDesc& g, const float* vs, int ld_wave,
                                               int ld_row, unsigned long long* kp, int b,
                                               int row0, int nr) {
  const int col0 = b * NWG;
  for (int t = threadIdx.x; t < nr * 16; t += blockDim.x) {
    const int rr = t >> 4, c0 = (t & 15) * 8;
    unsigned long long best = 0;
#pragma unroll
    for (int c = c0; c < c0 + 8; ++c) {
      if (col0 + c < g.N) {
        const unsigned long long k =
            argmax_key(vs[(c >> 5) * ld_wave + rr * ld_row + (c & 31)], col0 + c);
        best = k > best ? k : best;
      }
    }
    kp[t] = best;
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < nr; rr += blockDim.x) {
    unsigned long long best = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) best = kp[rr * 16 + j] > best ? kp[rr * 16 + j] : best;
    g.amax_keys[(size_t)(row0 + rr) * g.sp.nblk + b] = best;
  }
}

template <int MT>
__global__ __launch_bounds__(320) void k_gemm_bf16(GemmDesc g) {
  constexpr int XSTAGE = MT * 16 * 64;  // bf16 per x stage
  __shared__ __align__(16) bf16_t xs[XR * XSTAGE];
  __shared__ __align__(16) f32x4_t park[4 * MT * 2 * 64];  // block bA's sums, per consumer
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int wg = blockIdx.x, mb = blockIdx.z;
  const int K = g.K;
  const int nch = g.sp.nch;
  const int U = g.sp.nblk * nch;
  const int u0 = (int)((long long)wg * U / g.sp.G);
  const int u1 = (int)((long long)(wg + 1) * U / g.sp.G);
  const int n = u1 - u0;
  const int bA = u0 / nch, cA = u0 - bA * nch;
  const int nA = min(n, nch - cA);
  const int row0 = mb * 128;
  const int xrows = g.rows - row0;  // valid rows in this row block

  // column placement of consumer wave cw's 32 columns of column block b
  auto placement = [&](int b, int cw, int& sbase, int& segn, int& nl, int& si)
      __attribute__((always_inline)) {
    const int col0 = b * NWG;
    si = 0;
    sbase = 0;
    while (si < g.nseg - 1 && col0 >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
    segn = g.seg[si].n;
    nl = col0 - sbase + cw * 32;
  };
  if (wave == 4) {
    // ---------------- producer: x tiles -> LDS ring ----------------
    constexpr int NP = MT * 2;  // 16-byte pieces per lane per chunk
    // piece j of a lane: row lane/8 + 8j (clamped to the valid rows for the
    // global read), 16-byte piece lane%8; its swizzled LDS slot depends on
    // j only through j's parity, so two bases serve all j
    const bf16_t* X = (const bf16_t*)g.x + (size_t)row0 * K + (lane & 7) * 8;
    int xo[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int row = (lane >> 3) + 8 * j;
      xo[j] = (row < xrows ? row : xrows - 1) * K;
    }
    const int lo0 = (lane >> 3) * 64 + xswz(lane >> 3, lane & 7) * 8;
    const int lo1 = ((lane >> 3) + 8) * 64 + xswz((lane >> 3) + 8, lane & 7) * 8 - 512;
    u32x4_t ring[2][NP];
    // chunk t of the run reads K chunk cA + t of block bA, or t - nA of bA + 1
    auto load = [&](int t, u32x4_t (&dst)[NP]) __attribute__((always_inline)) {
      const int kc = t < nA ? cA + t : t - nA;
#pragma unroll
      for (int j = 0; j < NP; ++j) dst[j] = *(const u32x4_t*)(X + xo[j] + kc * KC);
    };
    auto store = [&](int t, const u32x4_t (&src)[NP]) __attribute__((always_inline)) {
      bf16_t* st = xs + (t % XR) * XSTAGE;
#pragma unroll
      for (int j = 0; j < NP; ++j) *(u32x4_t*)(st + ((j & 1) ? lo1 : lo0) + 512 * j) = src[j];
    };
    // prologue: stages for chunks 0 .. XR-2, ring for the next two
    for (int t = 0; t < n && t < XR - 1; ++t) {
      load(t, ring[0]);
      store(t, ring[0]);
    }
    load(min(XR - 1, n - 1), ring[(XR - 1) & 1]);
    load(min(XR, n - 1), ring[XR & 1]);
    int t = 0;
    // steady state: store chunk t+XR-1, load chunk t+XR+1 (same ring slot)
    for (; t + XR + 3 <= n; t += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        lds_barrier();
        const int slot = (XR - 1 + u) & 1;
        store(t + u + XR - 1, ring[slot]);
        load(t + u + XR + 1, ring[slot]);
      }
    }
    for (; t < n; ++t) {
      lds_barrier();
      const int slot = (t + XR - 1) & 1;
      if (t + XR - 1 < n) {
        if (slot == 0) store(t + XR - 1, ring[0]); else store(t + XR - 1, ring[1]);
      }
      if (t + XR + 1 < n) {
        if (slot == 0) load(t + XR + 1, ring[0]); else load(t + XR + 1, ring[1]);
      }
    }
  } else {
  // ---------------- consumers: weights + MFMA ----------------
  // this wave's columns of column block b: matrix segment, its first column,
  // and the packed stripe pointers of its two 16-column tiles.  A stripe past
  // the segment reads stripe 0 (its output is discarded at the store):
  // unpredicated loads let the compiler count outstanding loads exactly
  // instead of draining them at branch joins.
  auto setup = [&](int b, const bf16_t* (&wrow)[2], int& sbase, int& segn, int& nl, int& cs)
      __attribute__((always_inline)) {
    int si;
    placement(b, wave, sbase, segn, nl, si);
    const bf16_t* W = (const bf16_t*)g.seg[si].w;
    const int bl = (nl - wave * 32) >> 7;                 // block within the segment
    const int ns = min(8, (segn + 15) / 16 - 8 * bl);      // its stripes
    cs = ns * 1024;                                        // one chunk of the block
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int sb = 2 * wave + t;
      const int ok = nl + t * 16 < segn;
      wrow[t] = W + ((size_t)bl * nch * 8 + (ok ? sb : 0)) * 1024 + lane * 8;
    }
  };
  const bf16_t* wA[2];
  const bf16_t* wB[2];
  int sbA, segnA, nlA, csA, sbB = 0, segnB = 0, nlB = 0, csB = 0;
  setup(bA, wA, sbA, segnA, nlA, csA);
  if (n > nA) setup(bA + 1, wB, sbB, segnB, nlB, csB);
  else { wB[0] = wA[0]; wB[1] = wA[1]; csB = csA; }
  // weight rows of run chunk t, offset by the chunk's K position
  auto wptr = [&](int t, int tt) __attribute__((always_inline)) {
    return t < nA ? wA[tt] + (size_t)(cA + t) * csA : wB[tt] + (size_t)(t - nA) * csB;
  };

  f32x4_t acc[MT][2];
  f32x4_t* pk = park + (size_t)wave * MT * 2 * 64 + lane;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t wr[PF][2][2];
  auto load_w = [&](int t, u32x4_t (&dst)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const bf16_t* p = wptr(t, tt);
      // streaming hint: each weight line is used once; measured 7-10% faster
      // at one row tile
      dst[tt][0] = __builtin_nontemporal_load((const u32x4_t*)p);
      dst[tt][1] = __builtin_nontemporal_load((const u32x4_t*)(p + 512));
    }
  };
  // A-fragment offsets (bf16) in a stage: row i*16 + r, k 32j + 8q .. +8
  // (16-byte piece 4j + q).  The swizzle of row i*16 + r does not depend on
  // i, so the offset is a per-j base plus i*1024.
  int abase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) abase[j] = r * 64 + xswz(r, 4 * j + q) * 8;

  auto chunk = [&](int t, u32x4_t (&w)[2][2], bool more_w) __attribute__((always_inline)) {
    if (t == nA) {
      // first chunk of block bA + 1: park block bA's sums
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          pk[(i * 2 + tt) * 64] = acc[i][tt];
          acc[i][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    lds_barrier();
    const bf16_t* st = xs + (t % XR) * XSTAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      U4B b0, b1;
      b0.u = w[0][j];
      b1.u = w[1][j];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        U4B a;
        a.u = *(const u32x4_t*)(st + abase[j] + i * 1024);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b0.v, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b1.v, acc[i][1], 0, 0, 0);
      }
    }
    if (more_w) load_w(t + PF, w);
  };

  // prologue: unconditional (a chunk past the run reloads the last one and
  // is never used), so the loop sees a fixed count of loads in flight
#pragma unroll
  for (int s = 0; s < PF; ++s) load_w(min(s, n - 1), wr[s]);
  int tb = 0;
  for (; tb + 2 * PF <= n; tb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) chunk(tb + s, wr[s], true);
  }
  for (; tb < n; tb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int t = tb + s;
      if (t < n) chunk(t, wr[s], t + PF < n);
    }
  }

  // D layout of 16x16 MFMA: lane holds rows 4q..4q+3 of column r.  Block bA's
  // piece goes to its slot among the block's pieces; block bA + 1 starts
  // with this run, so its piece is slot 0.
  auto store_block = [&](const f32x4_t (&a)[MT][2], int slot, int sbase, int segn, int nl)
      __attribute__((always_inline)) {
    if (!g.part) return;
    float* out = g.part + (size_t)slot * g.rows_pad * g.N;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int nloc = nl + tt * 16 + r;
      if (nloc >= segn) continue;
      const int col = sbase + nloc;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row0 + i * 16 + q * 4 + e;
          if (row < g.rows) out[(size_t)row * g.N + col] = a[i][tt][e];
        }
      }
    }
  };
  const int slotA = wg - plan_first_wg(g.sp, bA);
  if (n > nA) {
    store_block(acc, 0, sbB, segnB, nlB);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[i][tt] = pk[(i * 2 + tt) * 64];
    store_block(acc, slotA, sbA, segnA, nlA);
  } else {
    store_block(acc, slotA, sbA, segnA, nlA);
  }
  if (g.amax_keys) {
    // whole-block plan: this block's values to LDS as [16 * MT rows][128 columns]
    float* vs = (float*)park;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) vs[(i * 16 + q * 4 + e) * NWG + wave * 32 + tt * 16 + r] = acc[i][tt][e];
  }
  }  // consumers
  if (g.amax_keys) {
    __syncthreads();  // every wave's values in park; the x stages are free
    block_row_keys(g, (const float*)park, 32, NWG, (unsigned long long*)xs, bA, row0,
                   min(MT * 16, g.rows - row0));
  }
}

// Four symmetric waves, one per SIMD (so each may hold up to 512 registers).
// Same work split, packed weights and column ownership as k_gemm_bf16 (each
// wave: 32 columns, all MT row tiles), but no producer wave:
//  * every thread stages 1/256 of the x tile of each chunk; its x pieces ride
//    in the same in-order load pipeline as its weights, PF chunks ahead
//    (chunk t+1+PF's x right after chunk t+PF's weights), so a wave only
//    ever waits for the oldest loads it issued;
//  * two LDS stages: x(t+1) is written before the barrier of iteration t and
//    its A fragments are read right after it, while the MFMAs of chunk t run
//    on the fragments read one iteration earlier.  A stage is rewritten two
//    iterations after its last read, and every barrier waits on the wave's
//    LDS traffic, so no extra synchronisation is needed.
template <int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm4(GemmDesc g) {
  constexpr int XSTAGE = MT * 16 * 64;  // bf16 per x stage
  constexpr int NPC = MT * 128;         // 16-byte x pieces per chunk
  constexpr int XJ = (NPC + 255) / 256; // pieces per thread per chunk
  static_assert(PF % 2 == 0, "the A-fragment buffers alternate with the chunk parity");
  __shared__ __align__(16) bf16_t xs[2 * XSTAGE];
  // per wave: its 32 columns x 16*MT rows of sums, rows padded to PKS floats
  // (16-byte aligned; the 4 row groups of an MFMA tile land on distinct
  // banks).  Sums leave through it as 128-byte row segments.
  constexpr int PKS = 36;
  __shared__ __align__(16) float park[4 * MT * 16 * PKS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int wg = blockIdx.x, mb = blockIdx.z;
  const int K = g.K;
  const int nch = g.sp.nch;
  const int U = g.sp.nblk * nch;
  const int u0 = (int)((long long)wg * U / g.sp.G);
  const int u1 = (int)((long long)(wg + 1) * U / g.sp.G);
  const int n = u1 - u0;
  const int bA = u0 / nch, cA = u0 - bA * nch;
  const int nA = min(n, nch - cA);
  const int row0 = mb * 128;
  const int xrows = g.rows - row0;

  // ---- x pieces of this thread: piece tid + 256j of the chunk (row p/8,
  // 16-byte piece p%8, swizzled in LDS); a piece past the tile (odd MT)
  // reloads the last one and is not written
  const bf16_t* X = (const bf16_t*)g.x + (size_t)row0 * K;
  int xo[XJ], xl[XJ];
  bool xw[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int pid = tid + 256 * j;
    xw[j] = pid < NPC;
    const int pc = xw[j] ? pid : NPC - 1;
    const int row = pc >> 3, piece = pc & 7;
    xo[j] = (row < xrows ? row : xrows - 1) * K + piece * 8;
    xl[j] = row * 64 + xswz(row, piece) * 8;
  }
  auto load_x = [&](int t, u32x4_t (&dst)[XJ]) __attribute__((always_inline)) {
    const int tc = t < n ? t : n - 1;
    const int kc = tc < nA ? cA + tc : tc - nA;
#pragma unroll
    for (int j = 0; j < XJ; ++j) dst[j] = *(const u32x4_t*)(X + xo[j] + kc * KC);
  };
  auto store_x = [&](int t, const u32x4_t (&src)[XJ]) __attribute__((always_inline)) {
    bf16_t* st = xs + (t & 1) * XSTAGE;
#pragma unroll
    for (int j = 0; j < XJ; ++j)
      if (xw[j]) *(u32x4_t*)(st + xl[j]) = src[j];
  };

  // ---- weights: this wave's two 16-column stripes of column block b
  auto placement = [&](int b, int& sbase, int& segn, int& nl, int& si)
      __attribute__((always_inline)) {
    const int col0 = b * NWG;
    si = 0;
    sbase = 0;
    while (si < g.nseg - 1 && col0 >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
    segn = g.seg[si].n;
    nl = col0 - sbase + wave * 32;
  };
  auto setup = [&](int b, const bf16_t* (&wrow)[2], int& sbase, int& segn, int& nl, int& cs)
      __attribute__((always_inline)) {
    int si;
    placement(b, sbase, segn, nl, si);
    const bf16_t* W = (const bf16_t*)g.seg[si].w;
    const int bl = (nl - wave * 32) >> 7;                 // block within the segment
    const int ns = min(8, (segn + 15) / 16 - 8 * bl);      // its stripes
    cs = ns * 1024;                                        // one chunk of the block
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int sb = 2 * wave + t;
      const int ok = nl + t * 16 < segn;
      wrow[t] = W + ((size_t)bl * nch * 8 + (ok ? sb : 0)) * 1024 + lane * 8;
    }
  };
  const bf16_t* wA[2];
  const bf16_t* wB[2];
  int sbA, segnA, nlA, csA, sbB = 0, segnB = 0, nlB = 0, csB = 0;
  setup(bA, wA, sbA, segnA, nlA, csA);
  if (n > nA) setup(bA + 1, wB, sbB, segnB, nlB, csB);
  else { wB[0] = wA[0]; wB[1] = wA[1]; csB = csA; }
  auto load_w = [&](int t, u32x4_t (&dst)[2][2]) __attribute__((always_inline)) {
    const int tc = t < n ? t : n - 1;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const bf16_t* p = tc < nA ? wA[tt] + (size_t)(cA + tc) * csA : wB[tt] + (size_t)(tc - nA) * csB;
      // streaming hint: each weight line is used once, and the lines then
      // leave the L2 room for the x tile and for the small tensors the
      // attention and epilogue kernels read
      dst[tt][0] = __builtin_nontemporal_load((const u32x4_t*)p);
      dst[tt][1] = __builtin_nontemporal_load((const u32x4_t*)(p + 512));
    }
  };

  // ---- A fragments (row i*16 + r, k 32j + 8q .. +8) and the MFMAs
  int abase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) abase[j] = r * 64 + xswz(r, 4 * j + q) * 8;
  auto read_a = [&](int t, U4B (&dst)[MT][2]) __attribute__((always_inline)) {
    const bf16_t* st = xs + (t & 1) * XSTAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) dst[i][j].u = *(const u32x4_t*)(st + abase[j] + i * 1024);
  };
  f32x4_t acc[MT][2];
  float* pk = park + wave * MT * 16 * PKS;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // MFMA D layout: lane holds rows 4q..4q+3 of column r of each 16x16 tile
  auto park_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[(i * 16 + 4 * q + e) * PKS + tt * 16 + r] = acc[i][tt][e];
  };
  auto mfma = [&](const U4B (&a)[MT][2], const u32x4_t (&w)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      U4B b0, b1;
      b0.u = w[0][j];
      b1.u = w[1][j];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][j].v, b0.v, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][j].v, b1.v, acc[i][1], 0, 0, 0);
      }
    }
  };

  u32x4_t wr[PF][2][2];
  u32x4_t xr[PF][XJ];  // x(c) for c >= 1 lives in xr[c % PF]
  U4B A0[MT][2], A1[MT][2];
  // one chunk: x(t+1) -> LDS, barrier, A(t+1) <- LDS, MFMAs of chunk t,
  // then the loads of chunk t+PF (weights) and t+1+PF (x) into the freed slots
  auto iter = [&](int t, u32x4_t (&w)[2][2], u32x4_t (&xn)[XJ], U4B (&ac)[MT][2],
                  U4B (&an)[MT][2], bool more) __attribute__((always_inline)) {
    if (t == nA) {  // first chunk of block bA + 1: park block bA's sums
      park_acc();
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) acc[i][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (t + 1 < n) store_x(t + 1, xn);
    lds_barrier();
    if (t + 1 < n) read_a(t + 1, an);
    mfma(ac, w);
    if (more) {
      load_w(t + PF, w);
      load_x(t + 1 + PF, xn);
    }
  };

  {  // prologue: x(0) staged and its fragments read; chunks 0..PF-1 (weights)
     // and 1..PF (x) in flight, in chunk order
    u32x4_t x0[XJ];
    load_x(0, x0);
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      load_w(s, wr[s]);
      load_x(s + 1, xr[(s + 1) % PF]);
    }
    store_x(0, x0);
    lds_barrier();
    read_a(0, A0);
  }
  int tb = 0;
  for (; tb + 2 * PF <= n; tb += PF) {
#pragma unroll
    for (int s = 0; s < PF; s += 2) {
      iter(tb + s, wr[s], xr[(s + 1) % PF], A0, A1, true);
      iter(tb + s + 1, wr[s + 1], xr[(s + 2) % PF], A1, A0, true);
    }
  }
  for (; tb < n; tb += PF) {
#pragma unroll
    for (int s = 0; s < PF; s += 2) {
      if (tb + s < n) iter(tb + s, wr[s], xr[(s + 1) % PF], A0, A1, tb + s + PF < n);
      if (tb + s + 1 < n) iter(tb + s + 1, wr[s + 1], xr[(s + 2) % PF], A1, A0, tb + s + 1 + PF < n);
    }
  }

  // this wave's parked rows -> piece `slot`: lane l writes columns 4(l%8)..+4
  // of rows l/8, l/8 + 8, ...  The 16-byte stores carry the streaming hint:
  // the pieces are read once, by the next kernel, on other XCDs
  const bool vec_ok = (g.N & 3) == 0;
  auto store_rows = [&](int slot, int sbase, int segn, int nl) __attribute__((always_inline)) {
    if (!g.part) return;
    float* out = g.part + (size_t)slot * g.rows_pad * g.N;
    const int c4 = (lane & 7) * 4;
    const int nloc = nl + c4;
    if (nloc >= segn) return;
    const int nr = min(MT * 16, g.rows - row0);
    for (int rr = lane >> 3; rr < nr; rr += 8) {
      const f32x4_t v = *(const f32x4_t*)(pk + rr * PKS + c4);
      float* dst = out + (size_t)(row0 + rr) * g.N + sbase + nloc;
      if (vec_ok && nloc + 3 < segn) {
        __builtin_nontemporal_store(v, (f32x4_t*)dst);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (nloc + k < segn) dst[k] = v[k];
      }
    }
  };
  auto wave_lds_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // block bA's piece goes to its slot among the block's pieces; block bA + 1
  // starts with this run, so its piece is slot 0
  const int slotA = wg - plan_first_wg(g.sp, bA);
  if (n > nA) {
    wave_lds_sync();
    store_rows(slotA, sbA, segnA, nlA);
    wave_lds_sync();
    park_acc();
    wave_lds_sync();
    store_rows(0, sbB, segnB, nlB);
  } else {
    park_acc();
    wave_lds_sync();
    store_rows(slotA, sbA, segnA, nlA);
  }
  if (g.amax_keys) {
    // whole-block plan: the four waves' parked columns (wave w's region holds
    // columns 32w .. 32w + 31 at row stride PKS); the x stages are free
    __syncthreads();
    block_row_keys(g, park, MT * 16 * PKS, PKS, (unsigned long long*)xs, bA, row0,
                   min(MT * 16, g.rows - row0));
  }
}

// Loader / consumer form of the multi-row kernel, for MT row tiles and
// short runs (no argmax keys).  Eight waves:
//  * waves 4-5 copy each chunk's weights (one contiguous 16 KB unit of the
//    packed layout) into a ring of SW LDS stages, SW-1 chunks ahead;
//  * waves 6-7 copy the chunk's x tile into a ring of SX stages;
//  * waves 0-3 only read the rings and run the MFMAs, in the same order as
//    k_gemm4 and k_gemm_bf16 (so the sums are the same bits).
// The copies go global -> LDS directly (LDS DMA, 16 bytes a lane, lane l's
// bytes at the stage base + 16 l), so a loader's issue is never held up by
// MFMA or LDS work.  One barrier per chunk for all eight waves: a loader
// waits for its copies of chunk t (its load counter runs in order) before
// barrier t, and after it refills the stages the consumers left at it.
// Both pieces (blocks bA and bA + 1) stay in registers until the stream
// ends: stores between the weight loads slow the stream down.
// Measured against k_gemm4 inside the 7B and 13B steps, this form ends a
// run of up to ~22 chunks sooner (its loaders are SW-1 chunks ahead from
// the first instruction) but streams the long runs more slowly; at 2-4 row
// tiles it is the slower one throughout.
typedef __attribute__((address_space(3))) void lds_void;
// s_waitcnt immediate for vmcnt(v) alone (gfx9 bit layout)
__device__ constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | 0x70 | 0xF00; }
template <int MT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_dma(GemmDesc g) {
  constexpr int SW = 7, SX = 3;  // weight and x stages
  constexpr int WST = 8 * 1024;           // bf16 of one weight unit (8 stripes x 2 KB)
  constexpr int XST = MT * 16 * 64;       // bf16 of one x tile
  static_assert(MT >= 2 && MT <= 8, "two x loader waves copy MT KB each");
  static_assert((SW * WST + SX * XST) * 2 <= 160 * 1024, "LDS");
  static_assert(SW * WST * 2 >= 4 * MT * 16 * 36 * 4, "the park reuses the weight ring");
  __shared__ __align__(16) bf16_t wring[SW * WST];
  __shared__ __align__(16) bf16_t xring[SX * XST];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, mb = blockIdx.z;
  const int K = g.K;
  const int nch = g.sp.nch;
  const int U = g.sp.nblk * nch;
  const int u0 = (int)((long long)wg * U / g.sp.G);
  const int u1 = (int)((long long)(wg + 1) * U / g.sp.G);
  const int n = u1 - u0;
  const int bA = u0 / nch, cA = u0 - bA * nch;
  const int nA = min(n, nch - cA);
  const int row0 = mb * 128;
  const int xrows = g.rows - row0;
  auto placement = [&](int b, int& sbase, int& segn, int& si) __attribute__((always_inline)) {
    const int col0 = b * NWG;
    si = 0;
    sbase = 0;
    while (si < g.nseg - 1 && col0 >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
    segn = g.seg[si].n;
  };
  // loader loop (a loader wave issues C copies a chunk): wait for chunk t
  // (younger chunks t+1 .. t+S-2 may fly), barrier t, then chunk t+S-1
  // into the stage chunk t-1 left
  auto loader = [&](auto issue, auto s_tag, auto c_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(s_tag)::value;
    constexpr int C = decltype(c_tag)::value;
    for (int t = 0; t < S - 1 && t < n; ++t) issue(t);
    for (int t = 0; t < n; ++t) {
      if (t + S - 2 <= n - 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * C));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (t + S - 1 < n) issue(t + S - 1);
    }
    lds_barrier();  // barrier n: the consumers' park reuses the weight ring
  };

  if (wave == 4 || wave == 5) {
    // weights: wave 4 + lw copies stripes 4 lw .. 4 lw + 3 (both MFMA steps)
    const int lw = wave - 4;
    const bf16_t* ubase[2];
    int uns[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int b = bA + k;
      int sbase = 0, segn = 0, si = 0;
      placement(b < g.sp.nblk ? b : bA, sbase, segn, si);
      const int bl = ((b < g.sp.nblk ? b : bA) * NWG - sbase) >> 7;
      uns[k] = min(8, (segn + 15) / 16 - 8 * bl);
      ubase[k] = (const bf16_t*)g.seg[si].w + (size_t)bl * nch * 8 * 1024;
    }
    auto issue = [&](int t) __attribute__((always_inline)) {
      const int k = t < nA ? 0 : 1;
      const int c = t < nA ? cA + t : t - nA;
      const int ns = uns[k];
      const bf16_t* unit = ubase[k] + (size_t)c * ns * 1024;
      bf16_t* st = wring + (t % SW) * WST;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int sb = 4 * lw + tt;
        const int src = sb < ns ? sb : 0;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          __builtin_amdgcn_global_load_lds((const void*)(unit + src * 1024 + j * 512 + lane * 8),
                                           (lds_void*)(st + (sb * 2 + j) * 512), 16, 0, 0);
      }
    };
    loader(issue, std::integral_constant<int, SW>(), std::integral_constant<int, 8>());
    return;
  }
  if (wave >= 6) {
    // x: wave 6 + lw copies rows 8 MT lw .. 8 MT lw + 8 MT - 1, 8 rows a
    // copy; lane l loads row 8 i + l / 8, piece (l % 8) ^ swizzle(row), so
    // the LDS holds the same XOR-swizzled rows as k_gemm4's
    const int lw = wave - 6;
    const bf16_t* X = (const bf16_t*)g.x + (size_t)row0 * K;
    int xoff[MT];
#pragma unroll
    for (int ii = 0; ii < MT; ++ii) {
      const int i = lw * MT + ii;
      const int row = 8 * i + (lane >> 3);
      const int piece = (lane & 7) ^ ((row >> 1) & 7);
      xoff[ii] = (row < xrows ? row : xrows - 1) * K + piece * 8;
    }
    auto issue = [&](int t) __attribute__((always_inline)) {
      const int c = t < nA ? cA + t : t - nA;
      bf16_t* st = xring + (t % SX) * XST;
#pragma unroll
      for (int ii = 0; ii < MT; ++ii)
        __builtin_amdgcn_global_load_lds((const void*)(X + xoff[ii] + c * KC),
                                         (lds_void*)(st + (lw * MT + ii) * 512), 16, 0, 0);
    };
    loader(issue, std::integral_constant<int, SX>(), std::integral_constant<int, MT>());
    return;
  }

  // ---------------- consumers ----------------
  const int r = lane & 15, q = lane >> 4;
  int abase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) abase[j] = r * 64 + xswz(r, 4 * j + q) * 8;
  // sums of block bA and of block bA + 1: both pieces leave after the
  // stream (stores between the weight loads slow the stream down)
  f32x4_t accA[MT][2], accB[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) accA[i][t] = accB[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int sbA, segnA, siA, sbB = 0, segnB = 0, siB = 0;
  placement(bA, sbA, segnA, siA);
  const int nlA = bA * NWG - sbA + wave * 32;
  int nlB = 0;
  if (n > nA) {
    placement(bA + 1, sbB, segnB, siB);
    nlB = (bA + 1) * NWG - sbB + wave * 32;
  }
  // fragments of one chunk: A for the MT row tiles, B for the two stripes,
  // both MFMA steps j
  U4B fa[MT][2], fb[2][2];
  auto read_f = [&](int t) __attribute__((always_inline)) {
    const bf16_t* sw = wring + (t % SW) * WST;
    const bf16_t* sx = xring + (t % SX) * XST;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        fb[tt][j].u = *(const u32x4_t*)(sw + ((2 * wave + tt) * 2 + j) * 512 + lane * 8);
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i][j].u = *(const u32x4_t*)(sx + abase[j] + i * 1024);
    }
  };
  // chunk t: barrier t (chunk t is in the rings; every consumer's reads of
  // chunk t-1 completed before it, so those stages are the loaders' again),
  // all of chunk t's fragment reads, then its MFMAs: the scheduling
  // barrier keeps the reads ahead, so a chunk pays one LDS latency
  auto chunk = [&](int t, f32x4_t (&acc)[MT][2]) __attribute__((always_inline)) {
    lds_barrier();
    read_f(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i][j].v, fb[0][j].v, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i][j].v, fb[1][j].v, acc[i][1], 0, 0, 0);
      }
  };
  for (int t = 0; t < nA; ++t) chunk(t, accA);
  for (int t = nA; t < n; ++t) chunk(t, accB);
  lds_barrier();  // barrier n: every consumer done with the rings (the loaders' copies ended before barrier n-1)
  // a wave's sums -> its park region in the weight ring (rows padded to 36
  // floats) -> the piece as 128-byte row segments, as in k_gemm4
  constexpr int PKS = 36;
  float* pk = (float*)wring + wave * MT * 16 * PKS;
  auto wave_lds_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto park = [&](const f32x4_t (&acc)[MT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[(i * 16 + 4 * q + e) * PKS + tt * 16 + r] = acc[i][tt][e];
  };
  const bool vec_ok = (g.N & 3) == 0;
  auto store_rows = [&](int slot, int sbase, int segn, int nl) __attribute__((always_inline)) {
    if (!g.part) return;
    float* out = g.part + (size_t)slot * g.rows_pad * g.N;
    const int c4 = (lane & 7) * 4;
    const int nloc = nl + c4;
    if (nloc >= segn) return;
    const int nr = min(MT * 16, g.rows - row0);
    for (int rr = lane >> 3; rr < nr; rr += 8) {
      const f32x4_t v = *(const f32x4_t*)(pk + rr * PKS + c4);
      float* dst = out + (size_t)(row0 + rr) * g.N + sbase + nloc;
      if (vec_ok && nloc + 3 < segn) {
        __builtin_nontemporal_store(v, (f32x4_t*)dst);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (nloc + k < segn) dst[k] = v[k];
      }
    }
  };
  // block bA's piece goes to its slot among the block's pieces; block
  // bA + 1 starts with this run, so its piece is slot 0
  const int slotA = wg - plan_first_wg(g.sp, bA);
  park(accA);
  wave_lds_sync();
  store_rows(slotA, sbA, segnA, nlA);
  if (n > nA) {
    wave_lds_sync();
    park(accB);
    wave_lds_sync();
    store_rows(0, sbB, segnB, nlB);
  }
}

// fp32 models: one wave per output element.  Lane l sums k = l, l + 64, ...
// in order, then the 64 lane sums are added by a fixed xor-shuffle tree, so
// an element's sum does not depend on the row count; the lanes read the
// weight row and the x row contiguously.
__global__ __launch_bounds__(256) void k_gemm_f32(GemmDesc g) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int m = blockIdx.y;
  if (n >= g.N || m >= g.rows) return;  // whole waves
  int si = 0, sbase = 0;
  while (si < g.nseg - 1 && n >= sbase + g.seg[si].n) { sbase += g.seg[si].n; ++si; }
  const float* w = (const float*)g.seg[si].w + (size_t)(n - sbase) * g.K;
  const float* x = (const float*)g.x + (size_t)m * g.K;
  float acc = 0.f;
  for (int k = lane; k < g.K; k += 64) acc = fmaf(x[k], w[k], acc);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) g.part[(size_t)m * g.N + n] = acc;
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
  const int b = s >> 3, sb = s & 7;
  const int ns = min(8, (N + 15) / 16 - 8 * b);  // stripes of column block b
  *(u32x4_t*)(dst + ((size_t)b * nch * 8 + (size_t)c * ns + sb) * 1024 + j * 512 + lane * 8) = v;
}

}  // namespace

size_t packed_bytes(int N, int K) { return (size_t)((N + 15) / 16) * 16 * K * 2; }

hipError_t launch_pack(const void* src, int N, int K, void* dst, hipStream_t st) {
  la_launch(k_pack_bf16, dim3(K / KC, (N + 15) / 16), dim3(128), 0, st,
            (const bf16_t*)src, N, K, (bf16_t*)dst);
  return hipGetLastError();
}

SplitPlan gemm_plan_whole(int N, int K) {
  SplitPlan p{};
  p.nch = K / KC;
  p.nblk = (N + NWG - 1) / NWG;
  p.G = p.nblk;
  p.np = 1;
  return p;
}

SplitPlan gemm_plan(int N, int K, int dtype) {
  SplitPlan p = gemm_plan_whole(N, K);
  if (dtype != LA_BF16 || p.nch < 1) return p;
  // Workgroups: whole column blocks when they already fill >= 90% of the
  // rounds of LA_GEMM_TARGET_WG workgroups (one per CU); otherwise deal the
  // units out to full rounds, keeping >= 4 chunks per workgroup, <= 15
  // pieces per block on average, and >= nblk workgroups (so a run spans at
  // most two column blocks).  (Measured: a uniform K split with fewer
  // pieces, e.g. 2 x 96 workgroups for the 7B QKV product, is slower
  // overall, epilogue included, than the even deal over 256.)
  const int T = LA_GEMM_TARGET_WG;
  const int rounds = (p.nblk + T - 1) / T;
  const long long U = (long long)p.nblk * p.nch;
  if (p.nblk * 10 < rounds * T * 9) {
    long long G = (long long)rounds * T;
    if (G > U / 4) G = U / 4;
    if (G > 15LL * p.nblk) G = 15LL * p.nblk;
    if (G < p.nblk) G = p.nblk;
    // plan_wg_of works in 32-bit unsigned arithmetic
    if (U * G < (1LL << 31)) p.G = (int)G;
  }
  for (int b = 0; b < p.nblk; ++b) {
    const int k = plan_pieces(p, b);
    if (k > p.np) p.np = k;
  }
  return p;
}

hipError_t launch_gemm(const GemmDesc& g, int dtype, hipStream_t st) {
  if (dtype == LA_F32) {
    dim3 grid((g.N + 3) / 4, g.rows);
    la_launch(k_gemm_f32, grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  if (g.sp.nblk != (g.N + NWG - 1) / NWG || g.sp.nch != g.K / KC) return hipErrorInvalidValue;
  // row maxima need whole column blocks (one piece each, one block a workgroup)
  if (g.amax_keys && (g.sp.np != 1 || g.sp.G != g.sp.nblk || g.nseg != 1)) return hipErrorInvalidValue;
  if (!g.part && !g.amax_keys) return hipErrorInvalidValue;
  const int mblk = (g.rows + 127) / 128;
  const int rows_last = g.rows - (mblk - 1) * 128;
  // the row-tile count only changes how many rows one workgroup carries, not
  // the arithmetic of any row
  const int mt = mblk > 1 ? 8 : (rows_last + 15) / 16;
  dim3 grid(g.sp.G, 1, mblk);
  // one row tile (the autoregressive step): the producer-wave kernel, which
  // streams fastest when the MFMA work is small; more rows: the four-wave
  // kernel, or for 6-8 row tiles and runs of at most 22 chunks a workgroup
  // on average, the loader / consumer kernel (measured faster there, slower
  // on longer runs and at 2-4 row tiles).  All accumulate every output
  // element over the same chunks in the same MFMA order, so a row's sums do
  // not depend on which one ran.
  const dim3 b4(256);
  if (mt >= 6 && !g.amax_keys && (long long)g.sp.nblk * g.sp.nch <= 22LL * g.sp.G) {
    switch (mt) {
      case 6: la_launch(k_gemm_dma<6>, grid, dim3(512), 0, st, g); break;
      case 7: la_launch(k_gemm_dma<7>, grid, dim3(512), 0, st, g); break;
      default: la_launch(k_gemm_dma<8>, grid, dim3(512), 0, st, g); break;
    }
    return hipGetLastError();
  }
  switch (mt) {
    case 1: la_launch(k_gemm_bf16<1>, grid, dim3(320), 0, st, g); break;
    case 2: la_launch(k_gemm4<2>, grid, b4, 0, st, g); break;
    case 3: la_launch(k_gemm4<3>, grid, b4, 0, st, g); break;
    case 4: la_launch(k_gemm4<4>, grid, b4, 0, st, g); break;
    case 5: la_launch(k_gemm4<5>, grid, b4, 0, st, g); break;
    case 6: la_launch(k_gemm4<6>, grid, b4, 0, st, g); break;
    case 7: la_launch(k_gemm4<7>, grid, b4, 0, st, g); break;
    default: la_launch(k_gemm4<8>, grid, b4, 0, st, g); break;
  }
  return hipGetLastError();
}
