// gemm_bwd.h -- bf16 MFMA grouped GEMMs of the expert FFN's backward pass on
// gfx950: products whose operands have the contraction index as their slow
// (row) dimension in memory.
//
// The forward GEMMs multiply token rows by weights stored with K contiguous
// (both operands K-major). Backward needs the other layouts:
//   data gradient   dH[r][n]  = sum_k dO[r][k] * W[k][n]       (W is K-slow)
//   weight gradient dW_e[m][n] = sum_{rows r of e} A[r][m] B[r][n]  (both K-slow)
// A K-slow tile is staged into LDS exactly as it lies in memory, [BK][cols]
// with cols contiguous (16-byte chunks straight from global memory with
// global_load_lds), and the MFMA fragment, which wants 8 consecutive K
// values per lane, is read with gfx950's transposing LDS read
// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4p+c supplies the
// address of 4 consecutive columns (8 bytes) of LDS row p, and lane j
// receives column j's 4 values of the 4 rows. Two such reads (rows k..k+3
// and k+4..k+7) give a lane its 8 K values of one column.
//
// K-slow LDS rows are swizzled in 16-byte chunks: physical chunk = logical
// chunk ^ ((row & 3) << 2), so the four rows one transposing read touches
// fall on four different 64-byte bank groups. K-contiguous tiles use the
// forward GEMM's layout ([rows][BK], chunk ^ ((row >> 1) & 7)).
//
// Two tile spaces:
//   ROWS  (data gradient): M = packed rows grouped by expert (ragged, tile
//         table as in the forward), A = rows [R][K] K-contiguous, B = the
//         expert's weight [K][N] K-slow, optionally as two K segments
//         (k < kseg from B0, else B1: W1 then W3 for SwiGLU's gate and up).
//   DENSE (weight gradient): per expert a full M x N output; K = the
//         expert's row count (ragged, masked in the last K tile); A = rows
//         [R][M] and B = rows [R][N], both K-slow; the output rows m < mseg
//         go to C0, the rest to C1 (dW1 and dW3 from one launch).
#pragma once

#include "gemm_bf16.h"
#include "moe_device.h"

namespace moe_bwd {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

enum { MODE_ROWS = 0, MODE_DENSE = 1 };
enum { BEPI_F32 = 0, BEPI_DSWIGLU = 1, BEPI_DACT = 2 };

struct BwdArgs {
  const uint16_t* A;   // ROWS: [R][lda] rows, K-contiguous. DENSE: [R][lda] rows (K = row)
  const uint16_t* B0;  // ROWS: weights [E][K][ldb]. DENSE: [R][ldb] rows
  const uint16_t* B1;  // ROWS: second K segment (k >= kseg), or null
  void* C0;            // output: ROWS [R][ldc] fp32; DENSE [E][mseg][ldc] (m < mseg)
  void* C1;            // DENSE: [E][M - mseg][ldc] (m >= mseg), or null
  int c_bf16;          // DENSE: outputs rounded to bf16 instead of fp32
  const uint16_t* pre; // DSWIGLU: saved pre-activations [R][2 N] (gate | up); DACT: [R][N]
  uint16_t* dpre;      // DSWIGLU: out [R][2 N] (d gate | d up); DACT: out [R][N]
  int act;             // DACT: MOE_RELU or MOE_GELU
  int M, N, K;         // DENSE: M, N; ROWS: N (columns), K (contraction)
  int lda, ldb, ldc;
  int kseg, mseg;
  long long b_expert;  // ROWS: elements between experts' weights
  int E, max_mt, n_tiles_n, group_n;
  const int32_t* offsets;     // [E+1] rows of each expert
  const int32_t* tile_start;  // ROWS: [E+1] first M tile of each expert
};

__device__ __forceinline__ int ks_phys(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

// Element offset in a K-slow LDS tile [BK][BC] of the first of the two
// transposing reads that give this lane its MFMA fragment (32 columns x 16 K)
// at column block cb and K step kk; the second read is 4 rows further.
template <int BC>
__device__ __forceinline__ int kslow_off(int cb, int kk, int lane) {
  const int G = lane >> 4, s = lane & 15, p = s >> 2, c4 = s & 3;
  const int row = kk * 16 + 8 * (G >> 1) + p;
  const int col = cb + 16 * (G & 1) + 4 * c4;
  return row * BC + (ks_phys(row, col >> 3) << 3) + (col & 7);  // row + 4: same swizzle
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// N K-slow fragments of 256-column tiles (second read 4 rows = 2048 bytes
// further), read with ds_read_b64_tr_b16 from one asm block that ends with
// s_waitcnt lgkmcnt(0), so every output is in its register when the block
// ends. (Written through the compiler's builtin instead, each transposing
// read is preceded by a vmcnt(0) wait: the compiler cannot tell it from a
// read of LDS that the in-flight global_load_lds transfers are still
// writing, and so waits for the next stages' operand loads at every K step.)
template <int N>
__device__ __forceinline__ void kslow_read(s16x4_t (&lo)[N], s16x4_t (&hi)[N],
                                           const uint32_t (&a)[N]);

template <>
__device__ __forceinline__ void kslow_read<4>(s16x4_t (&lo)[4], s16x4_t (&hi)[4],
                                              const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
        "=&v"(lo[3]), "=&v"(hi[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

template <>
__device__ __forceinline__ void kslow_read<6>(s16x4_t (&lo)[6], s16x4_t (&hi)[6],
                                              const uint32_t (&a)[6]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %13\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %14\n\t"
      "ds_read_b64_tr_b16 %5, %14 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %15\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %16\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %17\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
        "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}

__device__ __forceinline__ bf16x8_t kslow_join(s16x4_t lo, s16x4_t hi) {
  union {
    s16x4_t h[2];
    bf16x8_t v;
  } u;
  u.h[0] = lo;
  u.h[1] = hi;
  return u.v;
}

// BM x BN tile, BK = 64, NS LDS stages, WGM x WGN waves.
template <int MODE, int BEPI, int BM, int BN, int NS, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_bwd_kernel(BwdArgs g) {
  constexpr int BK = 64;
  constexpr int KK = BK / 16;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  constexpr int STAGE = A_ELEMS + B_ELEMS;
  // 1 KB segments: K-contiguous [rows][64] = 8 rows; K-slow [64][cols] = 512/cols rows
  constexpr int A_SEG_ROWS = MODE == MODE_ROWS ? 8 : 512 / BM;
  constexpr int B_SEG_ROWS = 512 / BN;
  constexpr int A_SEGS = (MODE == MODE_ROWS ? BM : BK) / A_SEG_ROWS;
  constexpr int B_SEGS = BK / B_SEG_ROWS;
  constexpr int A_IT = A_SEGS / NW, B_IT = B_SEGS / NW;
  constexpr int LPT = A_IT + B_IT;
  static_assert(A_IT * NW == A_SEGS && B_IT * NW == B_SEGS, "segments per wave");
  static_assert(BN >= 128 && (MODE == MODE_ROWS || BM >= 128), "K-slow tiles need >= 16 chunks");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- tile -> (expert, M tile, N tile); XCD-aware as in the forward GEMM
  [[maybe_unused]] const int per_xcd = gridDim.x >> 3;
  int e, mt, nt, row0 = 0, row_end = 0, kbeg = 0, kcount = 0;
  if constexpr (MODE == MODE_ROWS) {
    // an equal share of the M tiles that exist per XCD (the grid is sized
    // for max_mt); spare blocks exit
    const int n_real = g.tile_start[g.E];
    const int total = ((g.n_tiles_n + g.group_n - 1) / g.group_n) * n_real * g.group_n;
    const int quota = (total + 7) >> 3;
    if ((int)(blockIdx.x >> 3) >= quota) return;
    const int logical = (blockIdx.x & 7) * quota + (blockIdx.x >> 3);
    if (logical >= total) return;
    const int span = n_real * g.group_n;
    const int ng = logical / span, rem = logical - ng * span;
    mt = rem / g.group_n;
    nt = ng * g.group_n + (rem - mt * g.group_n);
    if (nt >= g.n_tiles_n || mt >= g.tile_start[g.E]) return;
    e = moe_gemm::tile_expert(g.tile_start, g.E, mt);
    row0 = g.offsets[e] + (mt - g.tile_start[e]) * BM;
    row_end = g.offsets[e + 1];
    kcount = g.K;
  } else {
    const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    const int mtiles = g.M / BM;
    const int span = mtiles * g.group_n;
    const int per_e = span * ((g.n_tiles_n + g.group_n - 1) / g.group_n);
    e = logical / per_e;
    const int rest = logical - e * per_e;
    const int ng = rest / span, rem = rest - ng * span;
    mt = rem / g.group_n;
    nt = ng * g.group_n + (rem - mt * g.group_n);
    if (e >= g.E || nt >= g.n_tiles_n) return;
    kbeg = g.offsets[e];
    kcount = g.offsets[e + 1] - kbeg;
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT = (kcount + BK - 1) / BK;

  // ---- per-lane source pointers at k = 0 for each 1 KB segment (16 bytes a
  // lane); a K tile then adds a uniform offset. K-slow rows past an
  // expert's count (DENSE tail tile) are clamped to its last row.
  const uint16_t* asrc[A_IT];
  int arow[A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int seg = wave + i * NW;
    if constexpr (MODE == MODE_ROWS) {
      const int r = seg * 8 + (lane >> 3);
      int row = row0 + r;
      row = row < row_end ? row : row_end - 1;
      const int c = (lane & 7) ^ moe_gemm::chunk_swz<64>(r);
      asrc[i] = g.A + (size_t)row * g.lda + c * 8;
      arow[i] = r;
    } else {
      constexpr int CPR = BM / 8;
      const int r = seg * A_SEG_ROWS + lane / CPR;
      const int c = ks_phys(r, lane % CPR);
      asrc[i] = g.A + (size_t)kbeg * g.lda + m0 + c * 8;
      arow[i] = r;
    }
  }
  const uint16_t* bsrc0[B_IT];
  const uint16_t* bsrc1[B_IT];
  int brow[B_IT];
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int seg = wave + i * NW;
    constexpr int CPR = BN / 8;
    const int r = seg * B_SEG_ROWS + lane / CPR;
    const int c = ks_phys(r, lane % CPR);
    brow[i] = r;
    if constexpr (MODE == MODE_ROWS) {
      const size_t col = (size_t)e * g.b_expert + n0 + c * 8;
      bsrc0[i] = g.B0 + col + (size_t)r * g.ldb;
      bsrc1[i] = g.B1 ? g.B1 + col + (size_t)r * g.ldb : nullptr;
    } else {
      bsrc0[i] = g.B0 + (size_t)kbeg * g.ldb + n0 + c * 8;
      bsrc1[i] = nullptr;
    }
  }

  auto issue = [&](int kt, int stage) {
    uint16_t* base = smem + stage * STAGE;
    const int k0 = kt * BK;
    const bool tail = MODE == MODE_DENSE && k0 + BK > kcount;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int seg = wave + i * NW;
      const uint16_t* src;
      if constexpr (MODE == MODE_ROWS) {
        src = asrc[i] + k0;
      } else {
        const int kr = tail ? min(k0 + arow[i], kcount - 1) : k0 + arow[i];
        src = asrc[i] + (size_t)kr * g.lda;
      }
      __builtin_amdgcn_global_load_lds(
          (const void*)src, (__attribute__((address_space(3))) void*)(base + seg * 512), 16, 0, 0);
    }
    const bool second = MODE == MODE_ROWS && g.B1 && k0 >= g.kseg;
    const size_t kofs = (size_t)(second ? k0 - g.kseg : k0) * g.ldb;
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int seg = wave + i * NW;
      const uint16_t* src;
      if constexpr (MODE == MODE_ROWS) {
        src = (second ? bsrc1[i] : bsrc0[i]) + kofs;
      } else {
        const int kr = tail ? min(k0 + brow[i], kcount - 1) : k0 + brow[i];
        src = bsrc0[i] + (size_t)kr * g.ldb;
      }
      __builtin_amdgcn_global_load_lds(
          (const void*)src,
          (__attribute__((address_space(3))) void*)(base + A_ELEMS + seg * 512), 16, 0, 0);
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frags {
    bf16x8_t a[FM];
    bf16x8_t b[FN];
  };
  static_assert(BN == 256 && (MODE == MODE_ROWS || BM == 256),
                "the transposing-read block assumes 256-column K-slow tiles");
  constexpr int NKS = (MODE == MODE_DENSE ? FM : 0) + FN;  // K-slow fragments per K step
  auto read_frags = [&](Frags& f, int stage, int kk, int kvalid) {
    const uint16_t* cur = smem + stage * STAGE;
    uint32_t addr[NKS];
    if constexpr (MODE == MODE_ROWS) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        f.a[i] = *(const bf16x8_t*)(cur + moe_gemm::dlds_off<64>(wm * WM + i * 32 + (lane & 31),
                                                                  kk * 2 + (lane >> 5)));
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        addr[i] = lds_addr(cur + kslow_off<BM>(wm * WM + i * 32, kk, lane));
    }
    constexpr int B0 = MODE == MODE_DENSE ? FM : 0;
#pragma unroll
    for (int j = 0; j < FN; ++j)
      addr[B0 + j] = lds_addr(cur + A_ELEMS + kslow_off<BN>(wn * WN + j * 32, kk, lane));
    s16x4_t lo[NKS], hi[NKS];
    kslow_read<NKS>(lo, hi, addr);
    if constexpr (MODE == MODE_DENSE) {
      if (kvalid < BK) {
        // this lane holds K = kk*16 + 8*(lane>>5) + 0..7 of its column
        const int k0 = kk * 16 + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (k0 + t >= kvalid) lo[i][t] = 0;
            if (k0 + 4 + t >= kvalid) hi[i][t] = 0;
          }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) f.a[i] = kslow_join(lo[i], hi[i]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[j] = kslow_join(lo[B0 + j], hi[B0 + j]);
  };
  auto mfma = [&](const Frags& f) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // ---- main loop: NS-stage ring. Per K tile kt (stage kt % NS): the MFMAs
  // of each 16-wide K step run while the next step's fragments are read;
  // after the last step's reads, wait for this wave's reads and for tile
  // kt+1's loads, barrier (no wave reads stage kt % NS any more), issue the
  // loads of tile kt+NS into it, read the first fragments of tile kt+1, and
  // only then run the last MFMAs of tile kt, so the barrier and the first
  // LDS reads of the next tile hide under MFMAs and NS tiles stay in flight.
  // Only the A operand of a DENSE tile is masked: rows past the expert's
  // count repeat its last row (finite), so a zero A gives a zero product.
  auto kvalid_of = [&](int kt) { return MODE == MODE_DENSE ? min(BK, kcount - kt * BK) : BK; };
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (j < KT) issue(j, j);
  Frags fr[2];
  if (KT > 0) {
    if (KT > NS - 1) moe_gemm::wait_vmcnt<(NS - 1) * LPT>();
    else moe_gemm::wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(fr[0], 0, 0, kvalid_of(0));
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % NS;
    const int kv = kvalid_of(kt);
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      read_frags(fr[(kk + 1) & 1], st, kk + 1, kv);
      mfma(fr[kk & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    if (kt + NS - 1 < KT) moe_gemm::wait_vmcnt<(NS - 2) * LPT>();
    else moe_gemm::wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + NS < KT) issue(kt + NS, st);
    if (kt + 1 < KT) read_frags(fr[KK & 1], (kt + 1) % NS, 0, kvalid_of(kt + 1));
    mfma(fr[(KK - 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue, staged through LDS: each 32 x 32 accumulator block goes
  // to a wave-private LDS patch (rows padded to 36 floats: 16-byte aligned,
  // and the two row halves a store instruction touches fall on different
  // banks), and comes back as 4 consecutive columns per lane, so every
  // global access is 16 bytes of fp32 (8 of bf16) and a store instruction
  // covers 8 full 128-byte row segments instead of 2.
  __syncthreads();  // every wave is done with the operand stages
  constexpr int SP = 36;
  float* stage = (float*)smem + wave * 32 * SP;
  const int rq = lane >> 3, c4 = (lane & 7) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stage[((r & 3) + 4 * (lane >> 5) + 8 * (r >> 2)) * SP + (lane & 31)] = acc[i][j][r];
      const int col = n0 + wn * WN + j * 32 + c4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int br = rq + 8 * q;
        const f32x4_t v = *(const f32x4_t*)(stage + br * SP + c4);
        const int lr = wm * WM + i * 32 + br;
        if constexpr (MODE == MODE_ROWS) {
          const int row = row0 + lr;
          if (row >= row_end) continue;
          if constexpr (BEPI == BEPI_DACT) {
            // h = act(a): da = v act'(a); ReLU' = [a > 0], GELU' = Phi(a) + a phi(a)
            const size_t o = (size_t)row * g.N + col;
            const u32x2_t ab = *(const u32x2_t*)(g.pre + o);
            float da[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float a = moe::bf16_bits_to_f32((uint16_t)(ab[t >> 1] >> (16 * (t & 1))));
              float dact;
              if (g.act == MOE_RELU) {
                dact = a > 0.f ? 1.f : 0.f;
              } else {
                const float Phi = 0.5f * (1.f + erff(a * 0.70710678118654752f));
                dact = Phi + a * 0.39894228040143268f * __expf(-0.5f * a * a);
              }
              da[t] = v[t] * dact;
            }
            *(u32x2_t*)(g.dpre + o) = u32x2_t{moe::pack_bf16x2(da[0], da[1]),
                                              moe::pack_bf16x2(da[2], da[3])};
          } else if constexpr (BEPI == BEPI_DSWIGLU) {
            // h = silu(a) * u; dh = v: da = v u silu'(a), du = v silu(a),
            // silu'(a) = sig (1 + a (1 - sig))
            const size_t o = (size_t)row * 2 * g.N + col;
            const u32x2_t ab = *(const u32x2_t*)(g.pre + o);
            const u32x2_t ub = *(const u32x2_t*)(g.pre + o + g.N);
            float da[4], du[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float a = moe::bf16_bits_to_f32((uint16_t)(ab[t >> 1] >> (16 * (t & 1))));
              const float u = moe::bf16_bits_to_f32((uint16_t)(ub[t >> 1] >> (16 * (t & 1))));
              const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-a));
              da[t] = v[t] * u * sig * (1.f + a * (1.f - sig));
              du[t] = v[t] * a * sig;
            }
            *(u32x2_t*)(g.dpre + o) = u32x2_t{moe::pack_bf16x2(da[0], da[1]),
                                              moe::pack_bf16x2(da[2], da[3])};
            *(u32x2_t*)(g.dpre + o + g.N) = u32x2_t{moe::pack_bf16x2(du[0], du[1]),
                                                    moe::pack_bf16x2(du[2], du[3])};
          } else {
            __builtin_nontemporal_store(v, (f32x4_t*)((float*)g.C0 + (size_t)row * g.ldc + col));
          }
        } else {
          const int m = m0 + lr;
          const size_t o = m < g.mseg ? ((size_t)e * g.mseg + m) * g.ldc + col
                                      : ((size_t)e * (g.M - g.mseg) + (m - g.mseg)) * g.ldc + col;
          void* C = m < g.mseg ? g.C0 : g.C1;
          if (g.c_bf16)
            *(u32x2_t*)((uint16_t*)C + o) = u32x2_t{moe::pack_bf16x2(v[0], v[1]),
                                                    moe::pack_bf16x2(v[2], v[3])};
          else  // written once, read by a later call: a streaming store
            __builtin_nontemporal_store(v, (f32x4_t*)((float*)C + o));
        }
      }
    }
  }
}

template <int MODE, int BEPI, int BM, int BN, int NS, int WGM, int WGN>
inline hipError_t launch_bwd(BwdArgs g, long long tiles, hipStream_t st) {
  constexpr size_t lds = (size_t)NS * (BM + BN) * 64 * sizeof(uint16_t);
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = gemm_bwd_kernel<MODE, BEPI, BM, BN, NS, WGM, WGN>;
  static bool configured = false;
  if (!configured) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    configured = true;
  }
  const int grid = (int)((tiles + 7) / 8 * 8);
  kern<<<grid, WGM * WGN * 64, lds, st>>>(g);
  return hipGetLastError();
}

}  // namespace moe_bwd
