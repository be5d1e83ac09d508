// grouped_ffn.hip -- every expert's FFN as one ragged grouped GEMM pair.
//
// mkbk-pku.cn, "MOE的优化" / Grouped GEMM: instead of two GEMMs per expert,
// one grouped launch over the bucketed, contiguously packed tokens. Rows
// offsets[e] .. offsets[e+1] go through expert e. GEMM 1 computes W1 x (and
// W3 x for SwiGLU) with the activation fused into its epilogue; GEMM 2
// computes W2 h. Both operands are K-contiguous (x rows, weight rows), so
// C = A . B^T with 16-byte loads along K on both sides.
//
// Paths:
//  - bf16 x bf16 -> fp32 on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), LDS
//    tiles with an XOR swizzle, M tiles from a device-built tile table so no
//    host sync is needed;
//  - fp32 (small layers) on plain fp32 FMA;
//  - fp8 e4m3 weights with bf16 activations for few rows per expert
//    (decode): weights streamed once from HBM, converted to bf16 in
//    registers, v_mfma_f32_16x16x32_bf16, per-output-channel scale after
//    the K sum.
#include <math.h>

#include "gemm_bf16.h"
#include "moe_device.h"

namespace {

enum { MODE_ACT = 0, MODE_GLU = 1, MODE_OUT = 2 };

__device__ __forceinline__ float act_fn(int act, float v) {
  if (act == MOE_RELU) return fmaxf(v, 0.f);
  // GELU, exact erf form
  return 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
}

// silu(g) = g * sigmoid(g) with the hardware reciprocal (about 1 ulp): the
// result is rounded to bf16 (or a bf16 hi/lo pair), so the correctly rounded
// division this library is built with for its softmax is not needed here
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

// M tile tables. Expert e's rows [offsets[e], offsets[e+1]) are cut into
// bm-row tiles: tile_start[e] = number of tiles of experts before e,
// tile_start[E] = total. With split, the rows past an expert's last full
// bm-row tile (split == 1), or only such a tail of at most bm/2 rows
// (split == 2), go to a second table of bm/2-row tiles, so that an expert
// just over a multiple of bm does not pay for a nearly empty bm-row tile.
// Optional outputs (null to skip): seg_* = row range of each expert per
// table, te* = expert of each tile (saves the per-block search).
__global__ __launch_bounds__(256) void tile_table_kernel(
    const int32_t* __restrict__ offsets, int E, int bm, int split, int32_t* __restrict__ ts,
    int32_t* __restrict__ ts_r, int32_t* __restrict__ sb, int32_t* __restrict__ se,
    int32_t* __restrict__ sb_r, int32_t* __restrict__ se_r, int32_t* __restrict__ te,
    int32_t* __restrict__ te_r) {
  __shared__ int sc[2][256];
  const int e = threadIdx.x;
  int n = 0, nr = 0, beg = 0, mid = 0, end = 0;
  if (e < E) {
    beg = offsets[e];
    end = offsets[e + 1];
    const int cnt = end - beg;
    if (split) {
      n = cnt / bm;
      // split == 2: only a tail of at most bm/2 rows leaves the main table
      if (split == 2 && cnt - n * bm > bm / 2) ++n;
      mid = min(beg + n * bm, end);
      nr = (end - mid + bm / 2 - 1) / (bm / 2);
    } else {
      n = (cnt + bm - 1) / bm;
      mid = end;
    }
  }
  sc[0][e] = n;
  sc[1][e] = nr;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v0 = e >= o ? sc[0][e - o] : 0, v1 = e >= o ? sc[1][e - o] : 0;
    __syncthreads();
    sc[0][e] += v0;
    sc[1][e] += v1;
    __syncthreads();
  }
  if (e < E) {
    const int t0 = sc[0][e] - n, t1 = sc[1][e] - nr;
    ts[e] = t0;
    if (e == E - 1) ts[E] = sc[0][e];
    if (ts_r) {
      ts_r[e] = t1;
      if (e == E - 1) ts_r[E] = sc[1][e];
    }
    if (sb) { sb[e] = beg; se[e] = mid; }
    if (sb_r) { sb_r[e] = mid; se_r[e] = end; }
    if (te)
      for (int t = 0; t < n; ++t) te[t0 + t] = e;
    if (te_r)
      for (int t = 0; t < nr; ++t) te_r[t1 + t] = e;
  }
}

struct GemmArgs {
  const void* A;          // [rows][K]
  const void* B0;         // [E][Nout][K]
  const void* B1;         // [E][Nout][K] (GLU) or null
  const float* bias;      // [E][Nout] or null
  void* C;                // [rows][Nout]
  int K, Nout, E, max_mt, act;
  const int32_t* offsets;
  const int32_t* tile_start;
  const int32_t* a_rows;  // product row r reads A row a_rows[r], or r if null
  // MODE_OUT, or null: write fmaf(c_gate[r], value, 0) to row c_rows[r]
  // of C (top-1 combine in the epilogue; c_gate in packed row order)
  const int32_t* c_rows;
  const float* c_gate;
};

// Expert of M tile `mt`: tile_start[e] <= mt < tile_start[e+1].
__device__ __forceinline__ int tile_expert(const int32_t* ts, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (ts[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------- fp32 SIMT
// BM x BM output tiles on a 16 x 16 thread grid (BM / 16 square register
// blocks), 64-wide K steps. BM = 32 or 16 when 64-row tiles would leave the
// chip short of blocks: the fp32 path serves small layers (the tiny Switch
// layer's GEMM 2 ran 9 blocks of 64 x 64 with one wave per SIMD, 20 us of
// dependent FMAs per thread).
template <int MODE, int BM>
__global__ __launch_bounds__(256) void ggemm_f32_kernel(GemmArgs g) {
  constexpr int BN = BM, BK = 64, TM = BM / 16, TN = BN / 16;
  constexpr int NB = MODE == MODE_GLU ? 2 : 1;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[NB][BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % (BN / TN), ty = tid / (BN / TN);
  const int mt = blockIdx.x % g.max_mt, nt = blockIdx.x / g.max_mt;
  if (mt >= g.tile_start[g.E]) return;
  const int e = tile_expert(g.tile_start, g.E, mt);
  const int row0 = g.offsets[e] + (mt - g.tile_start[e]) * BM;
  const int row_end = g.offsets[e + 1];
  const int n0 = nt * BN;
  const int K = g.K, Nout = g.Nout;
  const float* A = (const float*)g.A;
  const float* Bp[2] = {(const float*)g.B0 + (size_t)e * Nout * K,
                        NB == 2 ? (const float*)g.B1 + (size_t)e * Nout * K : nullptr};
  float acc[NB][TM][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[b][i][j] = 0.f;
  // Staging: BM rows x 16 groups of 4 consecutive K values per operand
  // (plane), G groups a thread (row (tid + 256 u) / 16, group tid % 16),
  // loaded one K step ahead into registers; rows past the tile and K past
  // the end load zeros. 64-wide K steps: on the small shapes of this path
  // each step's global-load round trip counts. The products of an output
  // add in k order whatever the tiling.
  constexpr int G = BM * BK / 4 / 256;
  static_assert(G >= 1 && G * 256 * 4 == BM * BK, "whole 4-vectors per thread");
  const int lk = (tid % (BK / 4)) * 4;
  int lm[G];
  const float* arow_p[G];
  const float* brow_p[NB][G];
  const bool vec = (K & 3) == 0;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    lm[u] = (tid + 256 * u) / (BK / 4);
    const int ar = row0 + lm[u];
    arow_p[u] = ar < row_end ? A + (size_t)(g.a_rows ? g.a_rows[ar] : ar) * K : nullptr;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      brow_p[b][u] = n0 + lm[u] < Nout ? Bp[b] + (size_t)(n0 + lm[u]) * K : nullptr;
  }
  auto load4 = [&](const float* row, int k) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (!row) return v;
    if (vec && k + 3 < K) return *(const f32x4_t*)(row + k);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (k + q < K) v[q] = row[k + q];
    return v;
  };
  f32x4_t ar[G], br[NB][G];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      ar[u] = load4(arow_p[u], k0 + lk);
#pragma unroll
      for (int b = 0; b < NB; ++b) br[b][u] = load4(brow_p[b][u], k0 + lk);
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) As[lk + q][lm[u]] = ar[u][q];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int u = 0; u < G; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[b][lk + q][lm[u]] = br[b][u][q];
    __syncthreads();
    if (k0 + BK < K) fetch(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = As[kk][ty * TM + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float bv = Bs[b][kk][tx * TN + j];
#pragma unroll
          for (int i = 0; i < TM; ++i) acc[b][i][j] = __builtin_fmaf(a[i], bv, acc[b][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = row0 + ty * TM + i;
    if (row >= row_end) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + tx * TN + j;
      if (col >= Nout) continue;
      float v;
      if (MODE == MODE_GLU) {
        v = silu(acc[0][i][j]) * acc[NB - 1][i][j];
      } else {
        const float bv = g.bias ? g.bias[(size_t)e * Nout + col] : 0.f;
        v = acc[0][i][j] + bv;
        if (MODE == MODE_ACT) v = act_fn(g.act, v);
      }
      size_t orow = row;
      if (MODE == MODE_OUT && g.c_rows) {
        orow = g.c_rows[row];
        v = __builtin_fmaf(g.c_gate[row], v, 0.f);
      }
      ((float*)g.C)[orow * Nout + col] = v;
    }
  }
}

// ---------------------------------------------------------------- fp8 decode
struct Fp8Args {
  const uint16_t* A;   // [rows][K] bf16
  const uint8_t* B0;   // [E][Nout][K] e4m3
  const uint8_t* B1;   // GLU partner or null
  const float* s0;     // [E][Nout]
  const float* s1;     // [E][Nout] or null
  void* C;             // [rows][Nout]
  int K, Nout, E, act;
  const int32_t* offsets;
  const int32_t* a_rows;  // product row r reads A row a_rows[r], or r if null
};

// 8 e4m3 codes (two dwords) -> 8 bf16, exactly (e4m3 values are bf16 values).
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Block: 4 waves, 64 output columns (16 per wave) of one expert
// (blockIdx.y). Rows are processed in groups of 64 (four 16-row MFMA
// tiles); a lane loads 16 consecutive K bytes of one weight row and feeds
// them to two 16x16x32 MFMAs together with the matching 8+8 activations.
// The K loop is unrolled by kU steps of 64 and all weight loads of a group
// are issued before any is used, so each lane keeps kU*NB 16-byte loads in
// flight (the kernel is bound by streaming the weights once).
constexpr int kU = 4;

template <int MODE, bool OUT_BF16>
__global__ __launch_bounds__(256) void ffn_fp8_kernel(Fp8Args g) {
  constexpr int NB = MODE == MODE_GLU ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.y;
  const int r_begin = g.offsets[e], r_end = g.offsets[e + 1];
  if (r_begin >= r_end) return;
  const int n = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const int grp = lane >> 4;
  const int K = g.K;
  const uint8_t* Bp[2];
  Bp[0] = g.B0 + ((size_t)e * g.Nout + n) * K + grp * 16;
  Bp[1] = NB == 2 ? g.B1 + ((size_t)e * g.Nout + n) * K + grp * 16 : nullptr;

  for (int rb = r_begin; rb < r_end; rb += 64) {
    const int nchunk = min(4, (r_end - rb + 15) >> 4);
    f32x4_t acc[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[b][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto step = [&](int k0, const u32x4_t (&w)[NB]) {
      bf16x8_t wlo[NB], whi[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        wlo[b] = e4m3x8_to_bf16(w[b][0], w[b][1]);
        whi[b] = e4m3x8_to_bf16(w[b][2], w[b][3]);
      }
      const int kl = k0 + grp * 16;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m >= nchunk) break;
        const int row = rb + m * 16 + (lane & 15);
        u32x4_t alo = {0u, 0u, 0u, 0u}, ahi = {0u, 0u, 0u, 0u};
        if (row < r_end) {
          const int arow = g.a_rows ? g.a_rows[row] : row;
          const u32x4_t* ap = (const u32x4_t*)(g.A + (size_t)arow * K + kl);
          alo = ap[0];
          ahi = ap[1];
        }
        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, alo);
        const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, ahi);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          acc[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, wlo[b], acc[b][m], 0, 0, 0);
          acc[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, whi[b], acc[b][m], 0, 0, 0);
        }
      }
    };

    int k0 = 0;
    for (; k0 + kU * 64 <= K; k0 += kU * 64) {
      u32x4_t w[kU][NB];
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int b = 0; b < NB; ++b) w[u][b] = *(const u32x4_t*)(Bp[b] + k0 + u * 64);
#pragma unroll
      for (int u = 0; u < kU; ++u) step(k0 + u * 64, w[u]);
    }
    for (; k0 < K; k0 += 64) {
      u32x4_t w[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) w[b] = *(const u32x4_t*)(Bp[b] + k0);
      step(k0, w);
    }
    // 16x16 accumulator layout: register r of lane l holds row 4*(l>>4)+r,
    // column l & 15.
    const float sc0 = g.s0[(size_t)e * g.Nout + n];
    const float sc1 = NB == 2 ? g.s1[(size_t)e * g.Nout + n] : 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= nchunk) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb + m * 16 + 4 * grp + r;
        if (row >= r_end) continue;
        float v;
        if (MODE == MODE_GLU)
          v = silu(acc[0][m][r] * sc0) * (acc[NB - 1][m][r] * sc1);
        else if (MODE == MODE_ACT)
          v = act_fn(g.act, acc[0][m][r] * sc0);
        else
          v = acc[0][m][r] * sc0;
        const size_t o = (size_t)row * g.Nout + n;
        if (OUT_BF16)
          ((uint16_t*)g.C)[o] = moe::f32_to_bf16_bits(v);
        else
          ((float*)g.C)[o] = v;
      }
    }
  }
}

// ------------------------------------------------------- fp8 decode, streamed
// With a few rows per expert the FFN is a pure weight stream, so this path
// is built around keeping HBM reads in flight without interruption.
// Persistent blocks of NW waves walk work units: one 16-row tile of one
// expert (tile table with 16-row tiles) x 16*NW output columns, column tiles
// of a row tile being consecutive units. Every unit streams its K dimension
// through one LDS ring of NS stages of SK K values, filled by direct-to-LDS
// loads (global_load_lds): each wave brings its own 16 weight rows (SK
// contiguous e4m3 bytes per row and matrix), the first waves bring the
// unit's 16 activation rows (SK bf16 each), and every wave re-fetches its
// 16 (GLU: 2 x 16) per-channel scales so the epilogue reads them from the
// stage it finishes on. The ring runs across unit boundaries: the loads of
// the next unit start while the current one is still being multiplied, and
// all unit metadata (tile table, offsets, gather rows) sits in LDS so that
// setting up a unit never waits on the vector-memory counter. A wave waits
// only for its own loads of the stage it is about to use (s_waitcnt vmcnt
// with the count of loads issued after it), then one barrier makes every
// wave's part of the stage visible and frees the slot consumed one step
// earlier.
//
// LDS row layouts use an XOR swizzle of the 16-byte chunk index so that the
// 16 lanes reading 16 consecutive rows at one logical chunk hit 16 distinct
// bank groups: 64-byte rows ^((r>>2)&3), 128-byte rows ^((r>>1)&7),
// 256-byte rows ^(r&15).
template <int RB>
__device__ __forceinline__ int stream_swz(int r) {
  return RB == 64 ? ((r >> 2) & 3) : RB == 128 ? ((r >> 1) & 7) : (r & 15);
}

template <int SK, int NW, int NB>
struct StreamLayout {
  static constexpr int A_ROW = SK * 2;              // bytes of one bf16 activation row
  static constexpr int A_BYTES = 16 * A_ROW;
  static constexpr int A_LOADS = A_BYTES / 1024;    // one per wave, waves 0..A_LOADS-1
  static constexpr int W_ROW = SK;                  // bytes of one e4m3 weight row
  static constexpr int W_BYTES = 16 * W_ROW;        // one wave, one matrix
  static constexpr int W_LOADS = W_BYTES / 1024;
  static constexpr int S_BYTES = 256;               // scales: 64 lanes x 4 bytes per wave
  static constexpr int STAGE = A_BYTES + NW * NB * W_BYTES + NW * S_BYTES;
  static_assert(A_LOADS >= 1 && A_LOADS <= NW && W_LOADS >= 1, "stream stage shape");
};

template <int MODE, int SK, int NW, int NS>
constexpr int stream_lds_bytes(int E, int rows_cap) {
  return NS * StreamLayout<SK, NW, MODE == MODE_GLU ? 2 : 1>::STAGE +
         ((2 * (E + 1) + rows_cap) * 4 + 15) / 16 * 16;
}

template <int MODE, bool OUT_BF16, int SK, int NW, int NS>
__global__ __launch_bounds__(NW * 64) void ffn_fp8_stream_kernel(Fp8Args g,
                                                                  const int32_t* __restrict__ tile_start,
                                                                  int rows_cap) {
  constexpr int NB = MODE == MODE_GLU ? 2 : 1;
  using L = StreamLayout<SK, NW, NB>;
  constexpr int BN = 16 * NW;
  constexpr int LPW = NB * L::W_LOADS + 1;  // loads per stage of a wave without A
  static_assert((NS - 2) * (LPW + 1) <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_ts = (int32_t*)(smem + NS * L::STAGE);
  int32_t* s_off = s_ts + (g.E + 1);
  int32_t* s_arow = s_off + (g.E + 1);

  const int lane = threadIdx.x & 63, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int E = g.E, K = g.K, Nout = g.Nout;
  for (int i = threadIdx.x; i <= E; i += NW * 64) {
    s_ts[i] = tile_start[i];
    s_off[i] = g.offsets[i];
  }
  if (g.a_rows) {
    const int R = min(g.offsets[E], rows_cap);
    for (int i = threadIdx.x; i < R; i += NW * 64) s_arow[i] = g.a_rows[i];
  }
  __syncthreads();
  const int NT = Nout / BN, KT = K / SK;
  const int n_units = s_ts[E] * NT;
  const int G = gridDim.x, bid = blockIdx.x;
  const int my_units = n_units > bid ? (n_units - 1 - bid) / G + 1 : 0;
  const int Q = my_units * KT;  // stages streamed by this block
  if (Q == 0) return;

  // unit j of this block -> expert, row range [rb, re) (at most 16 rows), n0
  struct Unit {
    int e, rb, re, n0;
  };
  auto unit_of = [&](int j) {
    const int u = bid + j * G;
    const int mt = u / NT;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_ts[mid] <= mt) lo = mid; else hi = mid;
    }
    Unit t;
    t.e = __builtin_amdgcn_readfirstlane(lo);
    const int rb = s_off[t.e] + (mt - s_ts[t.e]) * 16;
    t.rb = __builtin_amdgcn_readfirstlane(rb);
    t.re = __builtin_amdgcn_readfirstlane(min(s_off[t.e + 1], rb + 16));
    t.n0 = __builtin_amdgcn_readfirstlane((u - mt * NT) * BN);
    return t;
  };

  // ---- loader: per-lane global sources of the unit being fetched
  const uint8_t* wsrc[NB][L::W_LOADS];
  const uint8_t* asrc = nullptr;
  const float* ssrc = nullptr;
  int lj = 0, lkt = 0;
  auto set_sources = [&](int j) {
    const Unit t = unit_of(j);
    constexpr int CPR = L::W_ROW / 16;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < L::W_LOADS; ++i) {
        const int r = i * (64 / CPR) + lane / CPR;
        const int c = (lane % CPR) ^ stream_swz<L::W_ROW>(r);
        const uint8_t* B = b == 0 ? g.B0 : g.B1;
        wsrc[b][i] = B + ((size_t)t.e * Nout + t.n0 + wave * 16 + r) * K + c * 16;
      }
    if (wave < L::A_LOADS) {
      constexpr int ACPR = L::A_ROW / 16;
      const int r = wave * (64 / ACPR) + lane / ACPR;
      const int c = (lane % ACPR) ^ stream_swz<L::A_ROW>(r);
      const int row = min(t.rb + r, t.re - 1);  // pad rows repeat the last row
      const int arow = g.a_rows ? s_arow[min(row, rows_cap - 1)] : row;
      asrc = (const uint8_t*)g.A + (size_t)arow * K * 2 + c * 16;
    }
    const int sb = NB == 2 ? (lane >> 4) & 1 : 0;
    ssrc = (sb ? g.s1 : g.s0) + (size_t)t.e * Nout + t.n0 + wave * 16 + (lane & 15);
  };
  auto issue = [&](int slot) {
    uint8_t* base = smem + slot * L::STAGE;
    if (wave < L::A_LOADS)
      __builtin_amdgcn_global_load_lds(
          (const void*)(asrc + (size_t)lkt * SK * 2),
          (__attribute__((address_space(3))) void*)(base + wave * 1024), 16, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < L::W_LOADS; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(wsrc[b][i] + (size_t)lkt * SK),
            (__attribute__((address_space(3))) void*)(base + L::A_BYTES +
                                                       ((wave * NB + b) * L::W_LOADS + i) * 1024),
            16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (const void*)ssrc,
        (__attribute__((address_space(3))) void*)(base + L::A_BYTES + NW * NB * L::W_BYTES +
                                                   wave * L::S_BYTES),
        4, 0, 0);
    if (++lkt == KT) {
      lkt = 0;
      if (++lj < my_units) set_sources(lj);
    }
  };

  set_sources(0);
  for (int s = 0; s < NS - 1 && s < Q; ++s) issue(s);

  f32x4_t acc[NB];
  int ckt = 0, cj = 0;
  for (int q = 0; q < Q; ++q) {
    const int slot = q % NS;
    // this wave's loads of stage q are done when at most the loads of the
    // NS-2 later stages are outstanding
    if (q + NS - 2 < Q) {
      if (wave < L::A_LOADS) moe_gemm::wait_vmcnt<(NS - 2) * (LPW + 1)>();
      else moe_gemm::wait_vmcnt<(NS - 2) * LPW>();
    } else {
      moe_gemm::wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (q + NS - 1 < Q) issue((q + NS - 1) % NS);

    if (ckt == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const uint8_t* base = smem + slot * L::STAGE;
    const int rl = lane & 15;
#pragma unroll
    for (int s = 0; s < SK / 64; ++s) {
      const int ca = s * 8 + grp * 2;
      const uint8_t* arow = base + rl * L::A_ROW;
      const u32x4_t alo = *(const u32x4_t*)(arow + ((ca ^ stream_swz<L::A_ROW>(rl)) << 4));
      const u32x4_t ahi = *(const u32x4_t*)(arow + (((ca + 1) ^ stream_swz<L::A_ROW>(rl)) << 4));
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, alo);
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, ahi);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint8_t* wrow = base + L::A_BYTES + (wave * NB + b) * L::W_BYTES + rl * L::W_ROW;
        const int cw = s * 4 + grp;
        const u32x4_t w = *(const u32x4_t*)(wrow + ((cw ^ stream_swz<L::W_ROW>(rl)) << 4));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, e4m3x8_to_bf16(w[0], w[1]), acc[b],
                                                         0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, e4m3x8_to_bf16(w[2], w[3]), acc[b],
                                                         0, 0, 0);
      }
    }

    if (ckt == KT - 1) {
      const Unit t = unit_of(cj);
      const float* sc = (const float*)(base + L::A_BYTES + NW * NB * L::W_BYTES +
                                       wave * L::S_BYTES);
      const float sc0 = sc[rl];
      const float sc1 = NB == 2 ? sc[16 + rl] : 0.f;
      const int n = t.n0 + wave * 16 + rl;
      // 16x16 accumulator layout: register r of lane l holds row 4*(l>>4)+r,
      // column l & 15
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t.rb + 4 * grp + r;
        if (row >= t.re) continue;
        float v;
        if (MODE == MODE_GLU)
          v = silu(acc[0][r] * sc0) * (acc[NB - 1][r] * sc1);
        else if (MODE == MODE_ACT)
          v = act_fn(g.act, acc[0][r] * sc0);
        else
          v = acc[0][r] * sc0;
        const size_t o = (size_t)row * Nout + n;
        if (OUT_BF16)
          ((uint16_t*)g.C)[o] = moe::f32_to_bf16_bits(v);
        else
          ((float*)g.C)[o] = v;
      }
    }
    if (++ckt == KT) {
      ckt = 0;
      ++cj;
    }
  }
}

// N tiles per group of the XCD-aware tile order (measured on the Mixtral
// shape: 2 and 4 tie for GEMM 1, 2 is best for GEMM 2)
#ifndef MOE_GROUP_N
#define MOE_GROUP_N 2
#endif
// average rows per expert from which 256-row M tiles are used
#ifndef MOE_BM256_ROWS
#define MOE_BM256_ROWS 512
#endif
// 256-row tiling of experts averaging at least MOE_BM256_ROWS rows: 1 = every
// expert's rows past its last full tile run as 128-row tiles of a second
// launch, 2 = only tails of at most 128 rows do (Mixtral shape: 2 fastest,
// 1 slower than no split). Layers with fewer rows per expert keep the tail
// in the last 256-row tile, whose unused 32-row blocks skip their MFMAs
// (DeepSeek shape: 6% faster than a tail launch, which re-reads the weights).
#ifndef MOE_SPLIT_TAIL
#define MOE_SPLIT_TAIL 2
#endif
// From this many rows per expert on average (six or more 256-row tiles),
// each expert's rows are split evenly over its 256-row tiles and there is
// no tail launch
#ifndef MOE_EVEN_ROWS
#define MOE_EVEN_ROWS 1536
#endif
// GEMM 1 (SwiGLU, 256-row tiles) runs 8 waves (2 per SIMD); GEMM 2 with
// 256-row tiles uses 256x256 tiles on 8 waves (128x64 per wave): fewer LDS
// fragment reads per MFMA than 256x128, faster than 4 waves of 128x128
// GEMM 2 with a bf16 hi/lo pair h (two A planes) and GEMM 1 with an
// activation epilogue (the Switch/GELU shape: ~86 rows per expert, d_model
// 1024): GEMM 2 runs 128x256 tiles on 2x4 waves with two 64-wide K stages.
// Its A operand is two planes of h, so a narrow tile re-streams them for
// every N tile: against 64-column tiles on 4x2 waves (twice the tiles,
// fewer idle CUs) the wide tile is 10% faster for the launch pair, with
// four 32-wide stages 6%; 128-column tiles on 4x2 or 2x2 waves are slower
// than either. GEMM 1 uses 8-wave tiles (9% faster than 2x2 waves).
#ifndef MOE_G2_PAIR_BN
#define MOE_G2_PAIR_BN 256
#endif
// N-group size of each expert GEMM launch (the pair GEMM 2 of fp32 h has
// its own); with the quota split, groups of 8 in GEMM 1 measured 1-1.5%
// faster on the Mixtral shapes and 3% slower on one GPU's EP-8 DeepSeek
// share, groups of 4 or 8 everywhere no better overall, and GEMM 2 of the
// Switch shape with all 16 N tiles per group (each XCD reading only its own
// rows of h) 4% slower
#ifndef MOE_G1_GN
#define MOE_G1_GN MOE_GROUP_N
#endif
#ifndef MOE_G2_GN
#define MOE_G2_GN MOE_GROUP_N
#endif
#ifndef MOE_G2_PAIR_GN
#define MOE_G2_PAIR_GN MOE_GROUP_N
#endif
#ifndef MOE_G2_PAIR_LDS
#define MOE_G2_PAIR_LDS MOE_LDS_BUDGET
#endif
// LDS for GEMM 1 with an activation epilogue and 128-row tiles: three
// 32-wide stages (48 KB, 74 VGPRs) let three blocks share a CU, so one
// block's fill and epilogue overlap the others' K loops (K = d_model is
// short on the Switch shape: 1024). Switch-shaped layer: GEMM 1 246 ->
// ~190 us, grouped FFN -12% against one block per CU with four 64-wide
// stages; two blocks (two 64-wide stages) -8%. The pair GEMM 2 needs 136
// VGPRs, so a smaller budget cannot add a block there.
#ifndef MOE_G1_ACT_LDS
#define MOE_G1_ACT_LDS 49152
#endif
#ifndef MOE_G2_PAIR256_BK
#define MOE_G2_PAIR256_BK 64
#endif
#ifndef MOE_G2_PAIR_WGN
#define MOE_G2_PAIR_WGN 2
#endif
#ifndef MOE_G1_ACT_WGN
#define MOE_G1_ACT_WGN 4
#endif
#ifndef MOE_G2_PAIR_WGM
#define MOE_G2_PAIR_WGM 4
#endif
#ifndef MOE_G1_WGN
#define MOE_G1_WGN 4
#endif
#ifndef MOE_G2_WIDE
#define MOE_G2_WIDE 1
#endif
#ifndef MOE_G2_WGN
#define MOE_G2_WGN 4
#endif
#ifndef MOE_G2_WIDE_WGN
#define MOE_G2_WIDE_WGN 4
#endif
#ifndef MOE_G2_WIDE_WGM
#define MOE_G2_WIDE_WGM 2
#endif
#ifndef MOE_G1_WGM
#define MOE_G1_WGM 2
#endif

moe_status gemm_status(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    moe_host::set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return MOE_EHIP;
  }
  return MOE_OK;
}

// fp8 streaming path: 128 K values per stage, 8 waves (128 output columns)
// per block, one block per CU; 3 two-matrix stages (38 KB each) or 6
// one-matrix stages (22 KB each). Measured on the 256-expert decode layer:
// 4 waves per CU (in one or two blocks) or 64-value stages stream slower,
// deeper rings change nothing.
#ifndef MOE_FP8_STREAM
#define MOE_FP8_STREAM 1
#endif
#ifndef MOE_STREAM_SK
#define MOE_STREAM_SK 128
#endif
#ifndef MOE_STREAM_NW
#define MOE_STREAM_NW 8
#endif
#ifndef MOE_STREAM_NS_GLU
#define MOE_STREAM_NS_GLU 3
#endif
#ifndef MOE_STREAM_NS1
#define MOE_STREAM_NS1 6
#endif
#ifndef MOE_STREAM_BPC
#define MOE_STREAM_BPC 1  // resident blocks per CU
#endif
constexpr int kStreamSK = MOE_STREAM_SK, kStreamNW = MOE_STREAM_NW;
constexpr int kStreamNsGlu = MOE_STREAM_NS_GLU;
constexpr int kStreamNs1 = MOE_STREAM_NS1;
constexpr int kStreamMaxRows = 2048;

// The streaming kernel re-reads an expert's weights once per 16-row tile,
// so it serves layers averaging at most 8 rows per expert (decode), and any
// call of at most 64 rows (a decode batch through the shared expert: four
// passes over a small weight set, spread over the whole chip instead of one
// workgroup per 64 columns); its shapes need K and the output width to be
// multiples of 128.
bool use_fp8_stream(int E, int d, int F, int max_rows) {
  return MOE_FP8_STREAM && (max_rows <= 8 * E || max_rows <= 64) &&
         max_rows <= kStreamMaxRows &&
         d % kStreamSK == 0 && F % kStreamSK == 0 && d % (16 * kStreamNW) == 0 &&
         F % (16 * kStreamNW) == 0;
}

int device_cu_count() {
  static int cached_dev = -1, cached_n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached_dev = dev;
    cached_n = n;
  }
  return cached_n;
}

template <int MODE, bool OUT_BF16, int NS>
hipError_t launch_stream(const Fp8Args& a, const int32_t* tile_start, int rows_cap,
                         hipStream_t st) {
  auto kern = ffn_fp8_stream_kernel<MODE, OUT_BF16, kStreamSK, kStreamNW, NS>;
  const int lds = stream_lds_bytes<MODE, kStreamSK, kStreamNW, NS>(a.E, rows_cap);
  static int configured = 0;
  if (lds > configured) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    configured = lds;
  }
  kern<<<MOE_STREAM_BPC * device_cu_count(), kStreamNW * 64, lds, st>>>(a, tile_start,
                                                                        max(rows_cap, 1));
  return hipGetLastError();
}

// GEMM 1 and GEMM 2 of the bf16 path for M tiles of BM rows. 128-column N
// tiles (GEMM 1: 128 columns of both W1 and W3), 64 when the width is not
// a multiple of 128; GEMM 2 with 256-row tiles takes 256-column tiles.
template <int BM>
hipError_t launch_g1(bool glu, bool pair, const moe_gemm::Args& g1, hipStream_t st) {
  using namespace moe_gemm;
  const bool n1 = g1.Nrows % 128 == 0;
  if (glu) {
    if (n1)
      return pair ? run_gemm<BM, 128, 1, 2, EPI_GLU, OUT_BF16_PAIR>(g1, 1, st)
                  : run_gemm<BM, 128, 1, 2, EPI_GLU, OUT_BF16, MOE_G1_WGN, MOE_GEMM_BK,
                             MOE_G1_WGM>(g1, 1, st);
    return pair ? run_gemm<BM, 64, 1, 2, EPI_GLU, OUT_BF16_PAIR>(g1, 1, st)
                : run_gemm<BM, 64, 1, 2, EPI_GLU, OUT_BF16>(g1, 1, st);
  }
  if (n1)
    return pair ? run_gemm<BM, 128, 1, 1, EPI_ACT, OUT_BF16_PAIR, MOE_G1_ACT_WGN, MOE_GEMM_BK, 2,
                           BM == 128 ? MOE_G1_ACT_LDS : MOE_LDS_BUDGET>(g1, 1, st)
                : run_gemm<BM, 128, 1, 1, EPI_ACT, OUT_BF16, MOE_G1_ACT_WGN, MOE_GEMM_BK, 2,
                           BM == 128 ? MOE_G1_ACT_LDS : MOE_LDS_BUDGET>(g1, 1, st);
  return pair ? run_gemm<BM, 64, 1, 1, EPI_ACT, OUT_BF16_PAIR>(g1, 1, st)
              : run_gemm<BM, 64, 1, 1, EPI_ACT, OUT_BF16>(g1, 1, st);
}

// narrow: 64-column tiles (the tail launch of a few experts' last rows: twice
// the blocks to stream their W2 columns, Mixtral shape 128 -> 108 us)
template <int BM, int OF32>
hipError_t launch_g2_k(bool pair, bool ybf, const moe_gemm::Args& g2, hipStream_t st,
                       bool narrow) {
  using namespace moe_gemm;
  const bool n2 = g2.Nrows % 128 == 0 && !narrow;
  if (pair) {
    moe_gemm::Args gp = g2;
    gp.group_n = MOE_G2_PAIR_GN;
    if constexpr (BM == 128 && MOE_G2_PAIR_BN == 256) {
      if (g2.Nrows % 256 == 0)
        return ybf ? run_gemm<BM, 256, 2, 1, EPI_OUT, OUT_BF16, 4, MOE_G2_PAIR256_BK, 2,
                              MOE_G2_PAIR_LDS>(gp, 1, st)
                   : run_gemm<BM, 256, 2, 1, EPI_OUT, OF32, 4, MOE_G2_PAIR256_BK, 2,
                              MOE_G2_PAIR_LDS>(gp, 1, st);
    }
    if constexpr (MOE_G2_PAIR_BN == 128) {
      if (n2)
        return ybf ? run_gemm<BM, 128, 2, 1, EPI_OUT, OUT_BF16, MOE_G2_PAIR_WGN>(gp, 1, st)
                   : run_gemm<BM, 128, 2, 1, EPI_OUT, OF32, MOE_G2_PAIR_WGN>(gp, 1, st);
    }
    return ybf ? run_gemm<BM, 64, 2, 1, EPI_OUT, OUT_BF16, 2, MOE_GEMM_BK, MOE_G2_PAIR_WGM>(gp, 1, st)
               : run_gemm<BM, 64, 2, 1, EPI_OUT, OF32, 2, MOE_GEMM_BK, MOE_G2_PAIR_WGM>(gp, 1, st);
  }
  if constexpr (MOE_G2_WIDE && BM == 256) {  // (no 128-row instances of the wide tiles)
    if (g2.Nrows % 256 == 0)
      return ybf ? run_gemm<BM, 256, 1, 1, EPI_OUT, OUT_BF16, MOE_G2_WIDE_WGN, MOE_GEMM_BK,
                            MOE_G2_WIDE_WGM>(g2, 1, st)
                 : run_gemm<BM, 256, 1, 1, EPI_OUT, OF32, MOE_G2_WIDE_WGN, MOE_GEMM_BK,
                            MOE_G2_WIDE_WGM>(g2, 1, st);
  }
  if (n2)
    return ybf ? run_gemm<BM, 128, 1, 1, EPI_OUT, OUT_BF16, MOE_G2_WGN>(g2, 1, st)
               : run_gemm<BM, 128, 1, 1, EPI_OUT, OF32, MOE_G2_WGN>(g2, 1, st);
  return ybf ? run_gemm<BM, 64, 1, 1, EPI_OUT, OUT_BF16>(g2, 1, st)
             : run_gemm<BM, 64, 1, 1, EPI_OUT, OF32>(g2, 1, st);
}

// GEMM 2 with fp32 output into packed rows, or (c_rows set) scattered to
// token rows with the gate applied
template <int BM>
hipError_t launch_g2(bool pair, bool ybf, const moe_gemm::Args& g2, hipStream_t st,
                     bool narrow = false) {
  using namespace moe_gemm;
  if (g2.c_rows) return launch_g2_k<BM, OUT_F32_SCATTER>(pair, false, g2, st, narrow);
  return launch_g2_k<BM, OUT_F32>(pair, ybf, g2, st, narrow);
}

moe_gemm::Args base_args(const void* A, const void* B0, const void* B1, const float* bias,
                         void* C, int K, int Nrows, int E, int max_mt, int act,
                         const int32_t* offsets, const int32_t* tile_start) {
  moe_gemm::Args g{};
  g.A = A;
  g.B[0] = (const uint16_t*)B0;
  g.B[1] = (const uint16_t*)B1;
  g.B[2] = nullptr;
  g.bias = bias;
  g.C = C;
  g.K = K;
  g.Nrows = Nrows;
  g.n_valid = Nrows;
  g.ldc = Nrows;
  g.c_split = 0;
  g.k_chunk = K;
  g.E = E;
  g.max_mt = max_mt;
  g.act = act;
  g.group_n = MOE_GROUP_N;
  g.offsets = offsets;
  g.tile_start = tile_start;
  return g;
}

}  // namespace

namespace moe_host {

static size_t h_bytes(const moe_ffn_weights* w, moe_dtype act_dt, int max_rows) {
  const size_t es = (act_dt == MOE_F32 || w->h_fp32) ? 4 : 2;
  return align256((size_t)max_rows * w->d_ff * es);
}

// Tile tables after h (int32): tile_start and split-remainder tile_start
// [E+1] each, segment bounds of both [E] x 4, the tile -> expert maps (main:
// at most max_rows/128 + E tiles, remainder: at most 2E).
struct TileTables {
  int32_t *ts, *ts_r, *sb, *se, *sb_r, *se_r, *te, *te_r;
};
static size_t table_ints(int E, int max_rows) {
  return (size_t)6 * E + 2 + (size_t)(max_rows / 128 + E + 1) + 2 * (size_t)E;
}
static TileTables tile_tables(char* base, int E, int max_rows) {
  int32_t* p = (int32_t*)base;
  TileTables t;
  t.ts = p;
  t.ts_r = p + (E + 1);
  t.sb = p + 2 * (E + 1);
  t.se = t.sb + E;
  t.sb_r = t.se + E;
  t.se_r = t.sb_r + E;
  t.te = t.se_r + E;
  t.te_r = t.te + (max_rows / 128 + E + 1);
  return t;
}

// After the tile tables: the gates in packed row order [max_rows] fp32 (top-1
// combine in GEMM 2's epilogue).
size_t grouped_ffn_workspace_bytes(const moe_ffn_weights* w, moe_dtype act_dt, int max_rows) {
  return h_bytes(w, act_dt, max_rows) +
         align256(table_ints(w->n_experts, max_rows) * sizeof(int32_t)) +
         align256((size_t)max_rows * sizeof(float));
}

float* row_gates_ws(const moe_ffn_weights* w, moe_dtype act_dt, int max_rows, void* ws) {
  return (float*)((char*)ws + h_bytes(w, act_dt, max_rows) +
                  align256(table_ints(w->n_experts, max_rows) * sizeof(int32_t)));
}

moe_status grouped_ffn_launch(const moe_ffn_weights* w, const void* x_rows, moe_dtype act_dt,
                              const int32_t* row_index, const int32_t* offsets, int max_rows,
                              void* y_rows, moe_dtype y_dt, void* workspace, hipStream_t st,
                              uint16_t* preact, uint16_t* h_out, const int32_t* out_token,
                              const float* out_gate) {
  const int E = w->n_experts, d = w->d_model, F = w->d_ff;
  char* ws = (char*)workspace;
  // training: h goes to the caller's buffer (it is an operand of the weight
  // gradient of W2) and GEMM 1 also stores the pre-activations
  void* h = h_out ? (void*)h_out : (void*)ws;
  const TileTables tt = tile_tables(ws + h_bytes(w, act_dt, max_rows), E, max_rows);
  int32_t* tile_start = tt.ts;
  const bool glu = w->act == MOE_SWIGLU;
  moe_status s;

  if (w->w_dt == MOE_FP8_E4M3) {
    Fp8Args a1{(const uint16_t*)x_rows, (const uint8_t*)w->w1, (const uint8_t*)w->w3,
               w->s1, w->s3, h, d, F, E, (int)w->act, offsets, row_index};
    Fp8Args a2{(const uint16_t*)h, (const uint8_t*)w->w2, nullptr, w->s2, nullptr, y_rows,
               F, d, E, (int)w->act, offsets, nullptr};
    if (use_fp8_stream(E, d, F, max_rows)) {
      tile_table_kernel<<<1, 256, 0, st>>>(offsets, E, 16, 0, tile_start, nullptr, nullptr,
                                           nullptr, nullptr, nullptr, nullptr, nullptr);
      s = launch_status("tile table");
      if (s != MOE_OK) return s;
      const int cap1 = row_index ? max_rows : 0;
      hipError_t e = glu ? launch_stream<MODE_GLU, true, kStreamNsGlu>(a1, tile_start, cap1, st)
                         : launch_stream<MODE_ACT, true, kStreamNs1>(a1, tile_start, cap1, st);
      if (e != hipSuccess) return gemm_status(e, "grouped FFN fp8 stream GEMM 1");
      e = y_dt == MOE_BF16 ? launch_stream<MODE_OUT, true, kStreamNs1>(a2, tile_start, 0, st)
                           : launch_stream<MODE_OUT, false, kStreamNs1>(a2, tile_start, 0, st);
      return gemm_status(e, "grouped FFN fp8 stream GEMM 2");
    }
    dim3 g1(F / 64, E);
    if (glu)
      ffn_fp8_kernel<MODE_GLU, true><<<g1, 256, 0, st>>>(a1);
    else
      ffn_fp8_kernel<MODE_ACT, true><<<g1, 256, 0, st>>>(a1);
    s = launch_status("grouped FFN fp8 GEMM 1");
    if (s != MOE_OK) return s;
    dim3 g2(d / 64, E);
    if (y_dt == MOE_BF16)
      ffn_fp8_kernel<MODE_OUT, true><<<g2, 256, 0, st>>>(a2);
    else
      ffn_fp8_kernel<MODE_OUT, false><<<g2, 256, 0, st>>>(a2);
    return launch_status("grouped FFN fp8 GEMM 2");
  }

  // 256-row M tiles when experts average at least 512 rows, or at least 256
  // with a long K (d_model >= 4096: each M tile streams the expert's weights,
  // so fewer tiles per expert pay off), else 128 rows (less padding in
  // partly filled tiles; measured faster with d_model = 1024). With 256-row
  // tiles, short tails of the experts run as a second launch of 128-row tiles.
  const int avg_rows = max_rows / E;
  // fp32: 64-row tiles, 32-row ones while those would give fewer blocks than
  // two per CU, 16-row ones below half a block per CU (the tiny Switch
  // layer: grouped FFN 39 -> 31 -> 26 us from 64 to 32 to 16 rows)
  const size_t f32_blocks64 =
      (size_t)(max_rows / 64 + E) * (size_t)(((F > d ? F : d) + 63) / 64);
  const int f32_bm = f32_blocks64 < (size_t)device_cu_count() / 2   ? 16
                     : f32_blocks64 < (size_t)2 * device_cu_count() ? 32
                                                                    : 64;
  const int bm = act_dt == MOE_F32 ? f32_bm
                 : (avg_rows >= MOE_BM256_ROWS || (avg_rows >= 256 && d >= 4096)) ? 256
                                                                                  : 128;
  // With many tiles per expert there is no tail launch: each expert's rows
  // are split evenly over its ceil(rows / 256) tiles (heights a multiple of
  // 32), so its tiles run at one pace and the waves' unused 32-row blocks
  // skip their MFMAs. One GPU's EP-8 DeepSeek share (2048 rows per expert):
  // grouped FFN 5.53 -> 5.44 ms against a GEMM 1 over whole experts (tail in
  // a partly filled last tile) plus a GEMM 2 tail launch. On the Mixtral
  // shape (4 tiles and a tail per expert) the even split is 6% slower: GEMM
  // 2's 512 main tiles are exactly two rounds of the 256 CUs, 640 even ones
  // start a third; an XCD runs 4 M x 8 N tiles at once, so the fifth M tile
  // of an expert also re-streams its weights. DeepSeek shape: 1% slower.
  const bool even = bm == 256 && avg_rows >= MOE_EVEN_ROWS;
  const bool split = bm == 256 && avg_rows >= MOE_BM256_ROWS && MOE_SPLIT_TAIL && !even;
  if (act_dt == MOE_F32)
    tile_table_kernel<<<1, 256, 0, st>>>(offsets, E, bm, 0, tt.ts, nullptr, nullptr, nullptr,
                                         nullptr, nullptr, nullptr, nullptr);
  else
    tile_table_kernel<<<1, 256, 0, st>>>(offsets, E, bm, split ? MOE_SPLIT_TAIL : 0, tt.ts, tt.ts_r, tt.sb,
                                         tt.se, tt.sb_r, tt.se_r, tt.te, tt.te_r);
  s = launch_status("tile table");
  if (s != MOE_OK) return s;
  const int max_mt = (max_rows + bm - 1) / bm + E;

  if (act_dt == MOE_F32) {
    GemmArgs a1{x_rows, w->w1, w->w3, w->b1, h, d, F, E, max_mt, (int)w->act, offsets,
                tile_start, row_index, nullptr, nullptr};
    GemmArgs a2{h, w->w2, nullptr, w->b2, y_rows, F, d, E, max_mt, (int)w->act, offsets,
                tile_start, nullptr, out_token, out_gate};
    const int g1 = max_mt * ((F + bm - 1) / bm), g2 = max_mt * ((d + bm - 1) / bm);
    if (bm == 16) {
      if (glu)
        ggemm_f32_kernel<MODE_GLU, 16><<<g1, 256, 0, st>>>(a1);
      else
        ggemm_f32_kernel<MODE_ACT, 16><<<g1, 256, 0, st>>>(a1);
      ggemm_f32_kernel<MODE_OUT, 16><<<g2, 256, 0, st>>>(a2);
    } else if (bm == 32) {
      if (glu)
        ggemm_f32_kernel<MODE_GLU, 32><<<g1, 256, 0, st>>>(a1);
      else
        ggemm_f32_kernel<MODE_ACT, 32><<<g1, 256, 0, st>>>(a1);
      ggemm_f32_kernel<MODE_OUT, 32><<<g2, 256, 0, st>>>(a2);
    } else {
      if (glu)
        ggemm_f32_kernel<MODE_GLU, 64><<<g1, 256, 0, st>>>(a1);
      else
        ggemm_f32_kernel<MODE_ACT, 64><<<g1, 256, 0, st>>>(a1);
      ggemm_f32_kernel<MODE_OUT, 64><<<g2, 256, 0, st>>>(a2);
    }
    return launch_status("grouped FFN fp32");
  }

  using namespace moe_gemm;
  const bool pair = w->h_fp32 != 0;
  const bool ybf = y_dt == MOE_BF16;
  Args g1 = base_args(x_rows, w->w1, w->w3, w->b1, h, d, F, E, max_mt, (int)w->act, offsets,
                      tt.ts);
  // N tiles per group of the XCD-aware order. 256-row tiles (the prefill
  // shapes): 8 for a few large experts, 4 for many (GEMM pair on the
  // Mixtral shape 2.91 -> 2.86 ms and 2.77 -> 2.68 ms with expert choice,
  // groups of 2; one GPU's EP-8 DeepSeek share 6.09 ms with 2 or 4, 6.26
  // with 8; the DeepSeek-shaped layer 7.98 -> 7.86 ms with 4)
  const int gn256 = E <= 16 ? 8 : 4;
  g1.group_n = bm == 256 ? gn256 : MOE_G1_GN;
  g1.a_rows = row_index;
  g1.pre = preact;
  g1.seg_begin = tt.sb;
  g1.seg_end = tt.se;
  g1.tile_e = tt.te;
  Args g2 = base_args(h, w->w2, nullptr, w->b2, y_rows, F, d, E, max_mt, (int)w->act, offsets,
                      tt.ts);
  g2.group_n = bm == 256 ? gn256 : MOE_G2_GN;
  g2.c_rows = out_token;
  g2.c_gate = out_gate;
  g2.seg_begin = tt.sb;
  g2.seg_end = tt.se;
  g2.tile_e = tt.te;
  g1.even = g2.even = even ? 1 : 0;
  g1.c_plane = (long long)max_rows * F;  // lo plane of the bf16 pair h
  g2.a_plane = (long long)max_rows * F;
  // remainder launches: same operands, the second table, 128-row tiles
  Args g1r = g1, g2r = g2;
  g1r.tile_start = g2r.tile_start = tt.ts_r;
  g1r.seg_begin = g2r.seg_begin = tt.sb_r;
  g1r.seg_end = g2r.seg_end = tt.se_r;
  g1r.tile_e = g2r.tile_e = tt.te_r;
  g1r.max_mt = g2r.max_mt = 2 * E;
  hipError_t err;
  if (bm == 256) {
    err = launch_g1<256>(glu, pair, g1, st);
    if (err == hipSuccess && split) err = launch_g1<128>(glu, pair, g1r, st);
    if (err == hipSuccess) err = launch_g2<256>(pair, ybf, g2, st);
    if (err == hipSuccess && split) err = launch_g2<128>(pair, ybf, g2r, st, true);
  } else {
    err = launch_g1<128>(glu, pair, g1, st);
    if (err == hipSuccess) err = launch_g2<128>(pair, ybf, g2, st);
  }
  return gemm_status(err, "grouped FFN GEMM");
}

}  // namespace moe_host
