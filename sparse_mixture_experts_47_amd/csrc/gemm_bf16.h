// gemm_bf16.h -- ragged grouped GEMM C = A . B^T on gfx950 bf16 MFMA.
//
// A [rows][K] and every B [E][Nrows][K] are K-contiguous, so both operands
// load as 16-byte row chunks. Rows offsets[e] .. offsets[e+1] of the product
// belong to group (expert) e and multiply that group's B; product row r
// reads A row r, or A row a_rows[r] when a row map is given (the token
// gather of dispatch fused into the operand load, as a fused MoE kernel
// does). M tiles come from a device-built tile table (no host sync on the
// group sizes).
//
// Operand planes: an operand may be given as several bf16 planes whose sum
// is the value (NA planes of A, NB planes of B): NA = 2 is an fp32 operand
// held as hi = bf16(a), lo = bf16(a - hi); NB = 3 holds an fp32 matrix as
// three bf16 planes (hi, mid, lo). All plane
// products go into one accumulator, except for the gated (GLU) epilogue
// where B plane 0 (gate) and plane 1 (up) keep separate accumulators.
//
// Pipeline: operands go from global memory straight into a ring of LDS
// stages (see the direct-to-LDS kernel below), several K tiles ahead of the
// MFMAs.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so block b is
// remapped to a logical tile such that each XCD walks one contiguous range
// of logical tiles; logical tiles run GN N-tiles fastest, then M tiles, then
// the next group of GN N-tiles, so the blocks resident on one XCD at a time
// share a few A row panels and B weight panels in that XCD's L2. The grid
// is sized for the most M tiles the row counts could need; the ranges are
// cut from the tiles that exist (read from the tile table), an equal share
// per XCD, and the spare blocks exit at once.
#pragma once

#include <type_traits>

#include "moe_device.h"

namespace moe_gemm {

enum { EPI_ACT = 0, EPI_GLU = 1, EPI_OUT = 2, EPI_SUM = 3 };

struct Args {
  const void* A;         // [rows][K]: bf16, or fp32 when NA == 2
  const uint16_t* B[3];  // planes, each [E][Nrows][K] bf16
  const float* bias;     // [E][Nrows] or null (ACT/OUT)
  void* C;               // output, row stride ldc, split stride c_split
  int K;                 // full K
  int Nrows;             // rows of each B plane per group (multiple of BN)
  int n_valid;           // columns to store (<= Nrows)
  int ldc;
  long long c_split;     // element offset between K-split outputs
  long long a_plane;     // element offset between A planes (direct-LDS kernel)
  long long c_plane;     // element offset of the lo plane of a bf16 pair output
  int k_chunk;           // K per split (multiple of BK)
  int E, max_mt, act;
  int n_tiles_n;         // Nrows / BN
  int group_n;           // GN
  const int32_t* offsets;     // [E+1]
  const int32_t* tile_start;  // [E+1], or null: one group of rows1 rows (no table)
  int rows1;
  const int32_t* a_rows;      // row r of the product reads A row a_rows[r] (or r if null)
  // rows of group e covered by this launch: [seg_begin[e], seg_end[e]), or
  // [offsets[e], offsets[e+1]) when null; tile_e[mt] = group of M tile mt
  // (binary search over tile_start when null)
  const int32_t* seg_begin;
  const int32_t* seg_end;
  const int32_t* tile_e;
  // GLU / ACT, or null: the pre-activations are also stored, bf16, as rows
  // of 2 * Nrows (gate | up) or Nrows -- the state the backward pass
  // differentiates
  uint16_t* pre;
  // OUT with fp32 output, or null: product row r is the only kept
  // assignment of token c_rows[r] (top-1 routing), and the epilogue writes
  // fmaf(c_gate[r], value, 0) to row c_rows[r] of C -- the gate-weighted
  // combine, done where the expert output is made (c_gate: the gates in
  // packed row order)
  const int32_t* c_rows;
  const float* c_gate;
  // nonzero: the rows of group e are split evenly over its M tiles
  // (tile_start[e+1] - tile_start[e] of them) instead of BM rows a tile
  int even;
};

__device__ __forceinline__ float act_fn(int act, float v) {
  if (act == MOE_RELU) return fmaxf(v, 0.f);
  return 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
}

// silu(g) = g * sigmoid(g) with the hardware reciprocal (about 1 ulp): the
// result is rounded to bf16 (or a bf16 hi/lo pair), so the correctly rounded
// division this library is built with for its softmax is not needed here
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

__device__ __forceinline__ int tile_expert(const int32_t* ts, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant (bf16 A only): every 16-byte chunk goes from global
// memory straight into LDS with global_load_lds_dwordx4, so no staging
// registers are needed and NS LDS stages let the loads run NS-1 K steps ahead
// of the MFMAs. One such instruction writes 1 KB of LDS: lane l's 16 bytes
// land at l*16. With BK = 32 (64-byte LDS rows, 4 chunks) a 1 KB segment is
// 16 rows; lane l of segment j covers row 16j + l/4, physical chunk l%4, and
// fetches the logical chunk that the swizzle places there:
// c = (l%4) ^ ((row >> 2) & 3). The same swizzle serves the MFMA reads: a
// 16-byte LDS read serves 16 lanes (16 consecutive rows, one logical chunk)
// per cycle over 64 four-byte banks; rows r, r+4, r+8, r+12 share bank
// group r%4, and the swizzle gives them four different chunks.
// LDS bytes the stages of one tile may take
#ifndef MOE_LDS_BUDGET
#define MOE_LDS_BUDGET 147456
#endif

// LDS element offset of logical 16-byte chunk c of row r. BK = 32: 64-byte
// rows, chunk ^ ((r >> 2) & 3); BK = 64: 128-byte rows, chunk ^ ((r >> 1) & 7).
// Either way the 16 consecutive rows read in one LDS cycle at one logical
// chunk land on 16 distinct 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int chunk_swz(int r) {
  return BK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}
template <int BK>
__device__ __forceinline__ int dlds_off(int r, int c) {
  return r * BK + ((c ^ chunk_swz<BK>(r)) << 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with only the vector-memory counter limited to N
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Issue order for the scheduler. ilv_reads: MF groups of one MFMA, the
// first RD of them followed by one LDS read. ilv_tail: the first H = MF/2
// MFMAs each followed by up to VPM global loads (LPT in all), the other H by
// up to RPM LDS reads (RD in all) -- the reads come after the loads, which
// write LDS. Group masks: 0x008 MFMA, 0x100 LDS read, 0x230 vector-memory
// read or write and LDS write (a direct-to-LDS load matches as either).
template <int I, int MF, int RD>
__device__ __forceinline__ void ilv_reads() {
  if constexpr (I < MF) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    ilv_reads<I + 1, MF, RD>();
  }
}
template <int I, int MF, int RD, int LPT>
__device__ __forceinline__ void ilv_tail() {
  // a single MFMA (H = 1, nothing after it) takes the loads and the reads
  constexpr int H = MF >= 2 ? MF / 2 : 1, NR = MF - H;
  constexpr int VPM = (LPT + H - 1) / H, RPM = NR > 0 ? (RD + NR - 1) / NR : RD;
  constexpr int RB = NR > 0 ? H : 0;  // first MFMA followed by reads
  if constexpr (I < MF) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I < H && I * VPM < LPT)
      __builtin_amdgcn_sched_group_barrier(0x230, (VPM < LPT - I * VPM ? VPM : LPT - I * VPM), 0);
    if constexpr (I >= RB && (I - RB) * RPM < RD)
      __builtin_amdgcn_sched_group_barrier(0x100, (RPM < RD - (I - RB) * RPM ? RPM : RD - (I - RB) * RPM), 0);
    ilv_tail<I + 1, MF, RD, LPT>();
  }
}

// Output kinds of the direct-LDS kernel.
// OUT_F32_SCATTER: fp32, each product row to the token row c_rows[r], times
// its gate (the top-1 combine; its own instance so that the plain fp32 GEMM
// keeps no registers for the tokens and gates)
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_BF16_PAIR = 2, OUT_F32_SCATTER = 3 };

// NA A planes (bf16, plane p at A + p * a_plane elements): NA = 2 is an fp32
// operand kept as hi + lo bf16 parts. OUT_BF16_PAIR writes the result the
// same way: hi = bf16(v) at C, lo = bf16(v - hi) at C + c_plane.
template <int BM, int BN, int BK, int NS, int WGM, int WGN, int NA, int NB, int EPI, int OUTK>
__global__ __launch_bounds__(WGM * WGN * 64) void grouped_gemm_dlds_kernel(Args g) {
  constexpr int KK = BK / 16;                     // MFMA K steps per stage (even)
  constexpr int CPR = BK / 8;                     // 16-byte chunks per LDS row
  constexpr int SEG_ROWS = 1024 / (BK * 2);       // rows per 1 KB segment
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int NACC = EPI == EPI_GLU ? 2 : 1;
  constexpr int A_SEG = BM / SEG_ROWS, B_SEG = BN / SEG_ROWS;  // 1 KB segments per plane
  constexpr int A_IT = A_SEG / NW, B_IT = B_SEG / NW;
  constexpr int LPT = NA * A_IT + NB * B_IT;      // load instructions per stage
  constexpr int A_PLANE = BM * BK, B_PLANE = BN * BK;
  constexpr int STAGE = NA * A_PLANE + NB * B_PLANE;  // bf16 elements
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(KK % 2 == 0, "fragment sets alternate over an even number of K steps");
  static_assert(A_IT * NW == A_SEG && B_IT * NW == B_SEG, "segments per wave");
  static_assert(LPT * (NS - 1) < 64, "vmcnt range");
  static_assert(EPI != EPI_GLU || (NB == 2 && NA == 1), "GLU takes gate and up planes");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  // the grid is sized for max_mt M tiles; the XCDs split the tiles that
  // exist (tile_start[E] of them) evenly instead, each walking a contiguous
  // range, and the surplus blocks of every XCD exit
  const bool one_group = g.tile_start == nullptr;
  const int n_real = one_group ? (g.rows1 + BM - 1) / BM : g.tile_start[g.E];
  const int total = ((g.n_tiles_n + g.group_n - 1) / g.group_n) * n_real * g.group_n;
  const int quota = (total + 7) >> 3;
  if ((int)(blockIdx.x >> 3) >= quota) return;
  const int logical = (blockIdx.x & 7) * quota + (blockIdx.x >> 3);
  if (logical >= total) return;
  const int span = n_real * g.group_n;
  const int ng = logical / span, rem = logical - ng * span;
  const int mt = rem / g.group_n;
  const int nt = ng * g.group_n + (rem - mt * g.group_n);
  if (nt >= g.n_tiles_n || mt >= n_real) return;
  const int e = one_group ? 0 : g.tile_e ? g.tile_e[mt] : tile_expert(g.tile_start, g.E, mt);
  int row0, row_end;
  if (one_group) {
    row0 = mt * BM;
    row_end = g.rows1;
  } else {
    const int beg = g.seg_begin ? g.seg_begin[e] : g.offsets[e];
    const int end = g.seg_end ? g.seg_end[e] : g.offsets[e + 1];
    if (g.even) {
      // the group's rows split evenly over its M tiles, heights a multiple
      // of 32 (at most BM, as the tile count is ceil(rows / BM))
      const int nte = g.tile_start[e + 1] - g.tile_start[e];
      const int h = (((end - beg) + nte - 1) / nte + 31) & ~31;
      row0 = beg + (mt - g.tile_start[e]) * h;
      row_end = min(row0 + h, end);
    } else {
      row0 = beg + (mt - g.tile_start[e]) * BM;
      row_end = end;
    }
  }
  const int n0 = nt * BN;
  const int K = g.K;
  // top-1 combine: the token and gate of every row this lane will store,
  // loaded now so that their latency hides behind the K loop
  constexpr bool SCATTER = EPI == EPI_OUT && OUTK == OUT_F32_SCATTER;
  static_assert(OUTK != OUT_F32_SCATTER || EPI == EPI_OUT, "scatter is the output GEMM's");
  int tokv[SCATTER ? FM : 1][4];
  float gatev[SCATTER ? FM : 1][4];
  if constexpr (SCATTER) {
    {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = min(row0 + wm * WM + i * 32 + (lane >> 3) + 8 * q, row_end - 1);
          tokv[i][q] = g.c_rows[row];
          gatev[i][q] = g.c_gate[row];
        }
    }
  }
  // 32-row blocks of this wave's rows that hold at least one row of the
  // group: the rest of a partly filled M tile needs no fragment reads and
  // no MFMAs (uniform per wave)
  // (256-row tiles only: with 128-row tiles the checked loop measured slower
  // than computing the padding)
  int nfm = FM;
  if constexpr (BM == 256)
    nfm = __builtin_amdgcn_readfirstlane(
        max(0, min(FM, (row_end - row0 - wm * WM + 31) / 32)));
  const int k_begin = blockIdx.y * g.k_chunk;
  const int k_end = min(K, k_begin + g.k_chunk);
  const int KT = (k_end - k_begin) / BK;

  // per-lane global source pointers (at k = k_begin) for each segment: lane
  // l of a segment lands at byte l*16, i.e. row l / CPR, physical chunk
  // l % CPR, and fetches the logical chunk the swizzle puts there
  const int lr = lane / CPR;
  const uint16_t* asrc[NA][A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int r = (wave + i * NW) * SEG_ROWS + lr;
    int row = row0 + r;
    row = row < row_end ? row : row_end - 1;
    if (g.a_rows) row = g.a_rows[row];  // gather fused into the operand load
    const int c = (lane % CPR) ^ chunk_swz<BK>(r);
#pragma unroll
    for (int p = 0; p < NA; ++p)
      asrc[p][i] = (const uint16_t*)g.A + (size_t)p * g.a_plane + (size_t)row * K + k_begin + c * 8;
  }
  const uint16_t* bsrc[NB][B_IT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int r = (wave + i * NW) * SEG_ROWS + lr;
      const int c = (lane % CPR) ^ chunk_swz<BK>(r);
      bsrc[b][i] = g.B[b] + ((size_t)e * g.Nrows + n0 + r) * K + k_begin + c * 8;
    }

  auto issue = [&](int kt, int stage) {
    uint16_t* base = smem + stage * STAGE;
    const int koff = kt * BK;
#pragma unroll
    for (int p = 0; p < NA; ++p)
#pragma unroll
      for (int i = 0; i < A_IT; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(asrc[p][i] + koff),
            (__attribute__((address_space(3))) void*)(base + p * A_PLANE + (wave + i * NW) * 512),
            16, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < B_IT; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(bsrc[b][i] + koff),
            (__attribute__((address_space(3))) void*)(base + NA * A_PLANE + b * B_PLANE +
                                                       (wave + i * NW) * 512),
            16, 0, 0);
  };

  f32x16_t acc[NACC][FM][FN];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][i][j][r] = 0.f;

  // MFMA operand fragments of one 16-wide K half of a stage
  struct Frags {
    bf16x8_t a[NA][FM];
    bf16x8_t b[NB][FN];
  };
  // `cnt`: std::integral_constant<int, M>; M >= 0: the wave's first M
  // 32-row blocks are in use, known when the loop is compiled (no per-block
  // checks in it); M < 0: the first nfm, checked at run time
  auto read_frags = [&](Frags& f, int stage, int kk, auto cnt) {
    constexpr int M = decltype(cnt)::value;
    const uint16_t* cur = smem + stage * STAGE;
    const int c = kk * 2 + (lane >> 5);  // chunk of this lane's 8 K values
#pragma unroll
    for (int p = 0; p < NA; ++p)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        if (M >= 0 ? i < M : i < nfm)
          f.a[p][i] = *(const bf16x8_t*)(cur + p * A_PLANE +
                                         dlds_off<BK>(wm * WM + i * 32 + (lane & 31), c));
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        f.b[b][j] = *(const bf16x8_t*)(cur + NA * A_PLANE + b * B_PLANE +
                                       dlds_off<BK>(wn * WN + j * 32 + (lane & 31), c));
  };
  auto mfma = [&](const Frags& f, auto cnt) {
    constexpr int M = decltype(cnt)::value;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int p = 0; p < NA; ++p)
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            if (M >= 0 ? i >= M : i >= nfm) continue;
            f32x16_t& d = acc[EPI == EPI_GLU ? b : 0][i][j];
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[p][i], f.b[b][j], d, 0, 0, 0);
          }
  };

  {
    // Schedule per K tile kt (stage kt % NS), in two 16-wide halves:
    //   read half 1 of tile kt; MFMAs on half 0;
    //   wait for this wave's LDS reads and for tile kt+1's loads; barrier
    //   (now no wave reads stage kt % NS any more, and tile kt+1 is visible);
    //   issue the loads of tile kt+NS into stage kt % NS;
    //   read half 0 of tile kt+1; MFMAs on half 1 of tile kt.
    // LDS reads always run under the previous half's MFMAs, and the global
    // loads run NS-1 to NS tiles ahead. sched_barrier keeps the compiler from
    // moving MFMAs across the waits.
    // Interleaved schedule (full tiles, at least NS K tiles): the same
    // stages and waits, but the region after the barrier has no branches --
    // past the last tile the loads re-read tile KT-1 into the stage just
    // released (no tile reads it again) and the fragment reads of tile KT
    // go unused -- so the loads of tile kt+NS and the first fragment reads
    // of tile kt+1 can be issued between the MFMAs of the last half of tile
    // kt instead of ahead of them, and the matrix pipe does not drain while
    // they issue. Every iteration issues LPT loads, so the wait for tile
    // kt+1 is always vmcnt((NS-2) LPT).
    // Measured against the plain loop (grouped FFN): Mixtral-shaped 2.81 ->
    // 2.65 ms, DeepSeek-shaped 7.93 -> 7.35, one GPU's EP-8 DeepSeek share
    // 6.47 -> 5.41; the Switch-shaped kernels (activation epilogue with three
    // blocks per CU, and the two-plane h of GEMM 2) were 3% slower with it,
    // so they keep the plain loop.
    constexpr bool kInterleave = EPI != EPI_ACT && NA == 1;
    auto k_loop_ilv = [&](Frags(&fr)[2], auto full) {
      // MFMAs and fragment reads of one 16-wide step for the blocks in use
      constexpr int M = decltype(full)::value;
      constexpr int RD = NA * M + NB * FN, MF = NA * M * NB * FN;
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
          read_frags(fr[(kk + 1) & 1], kt % NS, kk + 1, full);
          mfma(fr[kk & 1], full);
          ilv_reads<0, MF, RD>();
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        wait_vmcnt<(NS - 2) * LPT>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(min(kt + NS, KT - 1), kt % NS);
        read_frags(fr[KK & 1], (kt + 1) % NS, 0, full);
        mfma(fr[(KK - 1) & 1], full);
        ilv_tail<0, MF, RD, LPT>();
        __builtin_amdgcn_sched_barrier(0);
      }
      // the loads past the last tile land in LDS the epilogue reuses
      wait_vmcnt<0>();
    };
    // one instance for waves whose 32-row blocks are all in use, one with
    // per-block checks (only the last M tile of a group can need it); both
    // run the same barriers
    auto k_loop = [&](auto full) {
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (j < KT) issue(j, j);
      Frags fr[2];
      if (KT > 0) {
        if (KT > NS - 1) wait_vmcnt<(NS - 1) * LPT>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        read_frags(fr[0], 0, 0, full);
      }
      if constexpr (kInterleave && decltype(full)::value > 0) {
        if (KT >= NS) {
          k_loop_ilv(fr, full);
          return;
        }
      }
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
          read_frags(fr[(kk + 1) & 1], kt % NS, kk + 1, full);
          mfma(fr[kk & 1], full);
          __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's LDS reads of tile kt are done; tile kt+1 may still be
        // followed by up to NS-2 younger tiles in flight
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        if (kt + NS - 1 < KT) wait_vmcnt<(NS - 2) * LPT>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kt + NS < KT) issue(kt + NS, kt % NS);
        if (kt + 1 < KT) read_frags(fr[KK & 1], (kt + 1) % NS, 0, full);
        mfma(fr[(KK - 1) & 1], full);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // a partly filled last M tile: the waves with some blocks in use run the
    // interleaved loop compiled for their block count (256-row tiles have 4
    // blocks a wave); waves with none, and other shapes, check at run time
    if (nfm == FM) {
      k_loop(std::integral_constant<int, FM>{});
    } else if constexpr (kInterleave && FM == 4) {
      if (nfm == 3) k_loop(std::integral_constant<int, 3>{});
      else if (nfm == 2) k_loop(std::integral_constant<int, 2>{});
      else if (nfm == 1) k_loop(std::integral_constant<int, 1>{});
      else k_loop(std::integral_constant<int, -1>{});
    } else {
      k_loop(std::integral_constant<int, -1>{});
    }
  }

  constexpr bool F32OUT = OUTK == OUT_F32 || OUTK == OUT_F32_SCATTER;
  constexpr int OB = F32OUT ? 4 : 2;
  char* Cb = (char*)g.C + (size_t)blockIdx.y * g.c_split * OB;
  // Epilogue, staged through LDS: each 32 x 32 block of results goes to a
  // wave-private patch (rows padded to 36 floats: 16-byte aligned, and the
  // row halves of one write fall on different banks) and comes back as 4
  // consecutive columns per lane, so the global stores are 16 bytes (fp32)
  // or 8 (bf16) a lane and one instruction covers 8 whole row segments.
  static_assert(NS * STAGE * 2 >= NW * 32 * 36 * 4, "LDS for the staged epilogue");
  const int rq = lane >> 3, c4 = (lane & 7) * 4;
  __syncthreads();  // every wave is done with the operand stages
  constexpr int SP = 36;
  float* stage = (float*)smem + wave * 32 * SP;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int colv = n0 + wn * WN + j * 32 + (lane & 31);
      const float bv = ((EPI == EPI_ACT || EPI == EPI_OUT) && g.bias && colv < g.n_valid)
                           ? g.bias[(size_t)e * g.Nrows + colv] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int br = (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        float v;
        if (EPI == EPI_GLU) {
          v = silu(acc[0][i][j][r]) * acc[NACC - 1][i][j][r];
          const int row = row0 + wm * WM + i * 32 + br;
          if (g.pre && row < row_end && colv < g.n_valid) {
            const size_t po = (size_t)row * 2 * g.Nrows + colv;
            g.pre[po] = moe::f32_to_bf16_bits(acc[0][i][j][r]);
            g.pre[po + g.Nrows] = moe::f32_to_bf16_bits(acc[NACC - 1][i][j][r]);
          }
        } else if (EPI == EPI_ACT) {
          v = act_fn(g.act, acc[0][i][j][r] + bv);
          const int row = row0 + wm * WM + i * 32 + br;
          if (g.pre && row < row_end && colv < g.n_valid)
            g.pre[(size_t)row * g.Nrows + colv] = moe::f32_to_bf16_bits(acc[0][i][j][r] + bv);
        } else {
          v = acc[0][i][j][r] + bv;
        }
        stage[br * SP + (lane & 31)] = v;
      }
      const int col = n0 + wn * WN + j * 32 + c4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int br = rq + 8 * q;
        const int row = row0 + wm * WM + i * 32 + br;
        if (row >= row_end || col >= g.n_valid) continue;
        f32x4_t v = *(const f32x4_t*)(stage + br * SP + c4);
        size_t o = (size_t)row * g.ldc + col;
        if constexpr (SCATTER) {
          const float gt = gatev[i][q];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(gt, v[t], 0.f);
          o = (size_t)tokv[i][q] * g.ldc + col;
        }
        if (col + 4 <= g.n_valid) {
          if (F32OUT) {
            // fp32 rows are read back only by a later call (combine or the
            // caller): streaming stores (DeepSeek-shaped grouped FFN -0.8%,
            // one GPU's EP-8 share -1.1%, Mixtral shape unchanged; with the
            // backward's fp32 gradient stores, its expert backward -2.5%)
            __builtin_nontemporal_store(v, (f32x4_t*)((float*)Cb + o));
          } else {
            uint16_t hb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) hb[t] = moe::f32_to_bf16_bits(v[t]);
            *(u32x2_t*)((uint16_t*)Cb + o) =
                u32x2_t{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16),
                        (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
            if (OUTK == OUT_BF16_PAIR) {
              float lo[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) lo[t] = v[t] - moe::bf16_bits_to_f32(hb[t]);
              *(u32x2_t*)((uint16_t*)Cb + g.c_plane + o) =
                  u32x2_t{moe::pack_bf16x2(lo[0], lo[1]), moe::pack_bf16x2(lo[2], lo[3])};
            }
          }
        } else {
          for (int t = 0; t < 4 && col + t < g.n_valid; ++t) {
            if (F32OUT) {
              ((float*)Cb)[o + t] = v[t];
            } else {
              const uint16_t hi = moe::f32_to_bf16_bits(v[t]);
              ((uint16_t*)Cb)[o + t] = hi;
              if (OUTK == OUT_BF16_PAIR)
                ((uint16_t*)Cb)[g.c_plane + o + t] =
                    moe::f32_to_bf16_bits(v[t] - moe::bf16_bits_to_f32(hi));
            }
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, int NA, int NB, int EPI, int OUTK>
inline hipError_t launch_dlds(Args g, int k_splits, hipStream_t st) {
  constexpr size_t lds = (size_t)NS * (NA * BM + NB * BN) * BK * sizeof(uint16_t);
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = grouped_gemm_dlds_kernel<BM, BN, BK, NS, WGM, WGN, NA, NB, EPI, OUTK>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  g.n_tiles_n = g.Nrows / BN;
  if (g.group_n > g.n_tiles_n) g.group_n = g.n_tiles_n;
  const int n_groups = (g.n_tiles_n + g.group_n - 1) / g.group_n;
  const long long tiles = (long long)g.max_mt * n_groups * g.group_n;
  const int grid_x = (int)((tiles + 7) / 8 * 8);
  dim3 grid(grid_x, k_splits);
  kern<<<grid, WGM * WGN * 64, lds, st>>>(g);
  return hipGetLastError();
}

#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif

// LDS stages for a tile: as many as fit in the budget (144 KB unless a
// launch asks for less, at most 8), bounded so that (stages - 1) x
// loads-per-stage fits the 6-bit vmcnt (4 waves).
template <int BM, int BN, int BK, int NA, int NB, int BUDGET = MOE_LDS_BUDGET>
constexpr int pick_stages() {
  constexpr int stage_bytes = (NA * BM + NB * BN) * BK * 2;
  constexpr int lpt = (NA * BM + NB * BN) * BK * 2 / 1024 / 4;  // with 4 waves
  int ns = BUDGET / stage_bytes;
  if (ns > 8) ns = 8;
  while (ns > 2 && (ns - 1) * lpt >= 64) --ns;
  return ns;
}

// K width of a stage: the preferred one if two stages of it fit, else 32.
template <int BM, int BN, int NA, int NB, int BKP, int BUDGET = MOE_LDS_BUDGET>
constexpr int pick_bk() {
  return pick_stages<BM, BN, BKP, NA, NB, BUDGET>() >= 2 ? BKP : 32;
}

template <int BM, int BN, int NA, int NB, int EPI, int OUTK, int WGN = 2, int BKP = MOE_GEMM_BK,
          int WGM = 2, int BUDGET = MOE_LDS_BUDGET>
inline hipError_t run_gemm(const Args& g, int k_splits, hipStream_t st) {
  constexpr int bk = pick_bk<BM, BN, NA, NB, BKP, BUDGET>();
  constexpr int ns = pick_stages<BM, BN, bk, NA, NB, BUDGET>();
  static_assert(ns >= 2, "tile too large for two LDS stages");
  return launch_dlds<BM, BN, bk, ns, WGM, WGN, NA, NB, EPI, OUTK>(g, k_splits, st);
}

}  // namespace moe_gemm
