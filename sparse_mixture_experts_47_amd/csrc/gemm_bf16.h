// gemm_bf16.h -- ragged grouped GEMM C = A . B^T on gfx950 bf16 MFMA.
//
// A [rows][K] and every B [E][Nrows][K] are K-contiguous, so both operands
// load as 16-byte row chunks. Rows offsets[e] .. offsets[e+1] of A belong to
// group (expert) e and multiply that group's B. M tiles come from a
// device-built tile table (no host sync on the group sizes).
//
// Operand planes: an operand may be given as several bf16 planes whose sum
// is the value (NA planes of A, NB planes of B). NA = 2 takes fp32 A and
// splits every element into hi = bf16(a), lo = bf16(a - hi) while staging;
// NB = 3 takes three bf16 planes of an fp32 matrix (hi, mid, lo). All plane
// products go into one accumulator, except for the gated (GLU) epilogue
// where B plane 0 (gate) and plane 1 (up) keep separate accumulators.
//
// Pipeline: double-buffered LDS. While the MFMAs consume K tile t from one
// buffer, the global loads of tile t+1 are in flight into registers; they are
// written to the other buffer after the compute, then one barrier.
// LDS rows are BK bf16 = BK/8 16-byte chunks; chunk c of row r sits at chunk
// position c ^ (r & 7), so the 8 rows that one 128-byte LDS cycle serves
// (for the MFMA operand reads: 8 lanes, 8 consecutive rows, one chunk each)
// fall on distinct banks.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so block b is
// remapped to a logical tile such that each XCD walks one contiguous range
// of logical tiles; logical tiles run GN N-tiles fastest, then M tiles, then
// the next group of GN N-tiles, so the blocks resident on one XCD at a time
// share a few A row panels and B weight panels in that XCD's L2.
#pragma once

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
  int k_chunk;           // K per split (multiple of BK)
  int E, max_mt, act;
  int n_tiles_n;         // Nrows / BN
  int group_n;           // GN
  const int32_t* offsets;     // [E+1]
  const int32_t* tile_start;  // [E+1]
};

__device__ __forceinline__ float act_fn(int act, float v) {
  if (act == MOE_RELU) return fmaxf(v, 0.f);
  return 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

__device__ __forceinline__ int tile_expert(const int32_t* ts, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

template <int BK>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BK + ((c ^ (r & 7)) << 3);
}

__device__ __forceinline__ u32x4_t split_hi_lo(const f32x4_t& a, const f32x4_t& b, u32x4_t& lo) {
  u32x4_t hi;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float x0 = a[2 * i], x1 = a[2 * i + 1];
    const uint16_t h0 = moe::f32_to_bf16_bits(x0), h1 = moe::f32_to_bf16_bits(x1);
    hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[i] = moe::pack_bf16x2(x0 - moe::bf16_bits_to_f32(h0), x1 - moe::bf16_bits_to_f32(h1));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float x0 = b[2 * i], x1 = b[2 * i + 1];
    const uint16_t h0 = moe::f32_to_bf16_bits(x0), h1 = moe::f32_to_bf16_bits(x1);
    hi[2 + i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[2 + i] = moe::pack_bf16x2(x0 - moe::bf16_bits_to_f32(h0), x1 - moe::bf16_bits_to_f32(h1));
  }
  return hi;
}

template <int BM, int BN, int BK, int WGM, int WGN, int NA, int NB, int EPI, bool OUT_BF16>
__global__ __launch_bounds__(WGM * WGN * 64) void grouped_gemm_kernel(Args g) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int NACC = EPI == EPI_GLU ? 2 : 1;
  constexpr int CPR = BK / 8;                    // 16-byte chunks per LDS row
  constexpr int A_IT = BM * CPR / NT;            // staging chunks per thread (A)
  constexpr int B_IT = BN * CPR / NT;            // per B plane
  constexpr int A_PLANE = BM * BK, B_PLANE = BN * BK;
  constexpr int STAGE = NA * A_PLANE + NB * B_PLANE;  // bf16 elements per buffer
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(A_IT * NT == BM * CPR && B_IT * NT == BN * CPR, "staging split");
  static_assert(EPI != EPI_GLU || (NB == 2 && NA == 1), "GLU takes gate and up planes");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- tile of this block (XCD-aware order, GN N-tiles fastest)
  const int total_blocks = gridDim.x;
  const int per_xcd = total_blocks >> 3;  // grid is a multiple of 8
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int span = g.max_mt * g.group_n;
  const int ng = logical / span, rem = logical - ng * span;
  const int mt = rem / g.group_n;
  const int nt = ng * g.group_n + (rem - mt * g.group_n);
  if (nt >= g.n_tiles_n || mt >= g.tile_start[g.E]) return;
  const int e = tile_expert(g.tile_start, g.E, mt);
  const int row0 = g.offsets[e] + (mt - g.tile_start[e]) * BM;
  const int row_end = g.offsets[e + 1];
  const int n0 = nt * BN;
  const int K = g.K;
  const int k_begin = blockIdx.y * g.k_chunk;
  const int k_end = min(K, k_begin + g.k_chunk);
  const int KT = (k_end - k_begin) / BK;

  // ---- staging: which (row, chunk) each thread moves
  const uint16_t* Bp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) Bp[b] = g.B[b] + ((size_t)e * g.Nrows + n0) * K;

  u32x4_t ra[A_IT][NA == 2 ? 2 : 1];
  u32x4_t rb[NB][B_IT];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int q = tid + it * NT;
      const int r = q / CPR, c = q % CPR;
      int row = row0 + r;
      row = row < row_end ? row : row_end - 1;
      if (NA == 1) {
        ra[it][0] = *(const u32x4_t*)((const uint16_t*)g.A + (size_t)row * K + k0 + c * 8);
      } else {
        const float* ap = (const float*)g.A + (size_t)row * K + k0 + c * 8;
        ra[it][0] = *(const u32x4_t*)ap;
        ra[it][NA == 2 ? 1 : 0] = *(const u32x4_t*)(ap + 4);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int q = tid + it * NT;
        const int r = q / CPR, c = q % CPR;
        rb[b][it] = *(const u32x4_t*)(Bp[b] + (size_t)r * K + k0 + c * 8);
      }
  };
  auto store_tile = [&](uint16_t* buf) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int q = tid + it * NT;
      const int r = q / CPR, c = q % CPR;
      if (NA == 1) {
        *(u32x4_t*)(buf + lds_off<BK>(r, c)) = ra[it][0];
      } else {
        u32x4_t lo;
        const u32x4_t hi = split_hi_lo(__builtin_bit_cast(f32x4_t, ra[it][0]),
                                       __builtin_bit_cast(f32x4_t, ra[it][NA == 2 ? 1 : 0]), lo);
        *(u32x4_t*)(buf + lds_off<BK>(r, c)) = hi;
        *(u32x4_t*)(buf + A_PLANE + lds_off<BK>(r, c)) = lo;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int q = tid + it * NT;
        const int r = q / CPR, c = q % CPR;
        *(u32x4_t*)(buf + NA * A_PLANE + b * B_PLANE + lds_off<BK>(r, c)) = rb[b][it];
      }
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

  if (KT > 0) {
    load_tile(k_begin);
    store_tile(smem);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    uint16_t* cur = smem + (kt & 1) * STAGE;
    if (kt + 1 < KT) load_tile(k_begin + (kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8_t af[NA][FM];
#pragma unroll
      for (int p = 0; p < NA; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[p][i] = *(const bf16x8_t*)(cur + p * A_PLANE +
                                        lds_off<BK>(wm * WM + i * 32 + (lane & 31), c));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const bf16x8_t bfr = *(const bf16x8_t*)(cur + NA * A_PLANE + b * B_PLANE +
                                                  lds_off<BK>(wn * WN + j * 32 + (lane & 31), c));
#pragma unroll
          for (int p = 0; p < NA; ++p)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              f32x16_t& d = acc[EPI == EPI_GLU ? b : 0][i][j];
              d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p][i], bfr, d, 0, 0, 0);
            }
        }
      }
    }
    if (kt + 1 < KT) store_tile(smem + ((kt + 1) & 1) * STAGE);
    __syncthreads();
  }

  // ---- epilogue. 32x32 accumulator: register r of lane l is
  // row (r & 3) + 4 (l >> 5) + 8 (r >> 2), column l & 31.
  char* Cb = (char*)g.C + (size_t)blockIdx.y * g.c_split * (OUT_BF16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + (lane & 31);
      if (col >= g.n_valid) continue;
      const float bv = ((EPI == EPI_ACT || EPI == EPI_OUT) && g.bias)
                           ? g.bias[(size_t)e * g.Nrows + col] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * WM + i * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        if (row >= row_end) continue;
        float v;
        if (EPI == EPI_GLU)
          v = silu(acc[0][i][j][r]) * acc[NACC - 1][i][j][r];
        else if (EPI == EPI_ACT)
          v = act_fn(g.act, acc[0][i][j][r] + bv);
        else
          v = acc[0][i][j][r] + bv;
        const size_t o = (size_t)row * g.ldc + col;
        if (OUT_BF16)
          ((uint16_t*)Cb)[o] = moe::f32_to_bf16_bits(v);
        else
          ((float*)Cb)[o] = v;
      }
    }
  }
}

// Launch helper: grid = 8-aligned count of (max_mt x n_tiles_n) tiles, times
// the K splits in grid.y. Dynamic LDS = 2 stages.
template <int BM, int BN, int BK, int WGM, int WGN, int NA, int NB, int EPI, bool OUT_BF16>
inline hipError_t launch(Args g, int k_splits, hipStream_t st) {
  constexpr int STAGE = NA * BM * BK + NB * BN * BK;
  constexpr size_t lds = 2 * STAGE * sizeof(uint16_t);
  auto kern = grouped_gemm_kernel<BM, BN, BK, WGM, WGN, NA, NB, EPI, OUT_BF16>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  g.n_tiles_n = g.Nrows / BN;
  const int n_groups = (g.n_tiles_n + g.group_n - 1) / g.group_n;
  const long long tiles = (long long)g.max_mt * n_groups * g.group_n;
  const int grid_x = (int)((tiles + 7) / 8 * 8);
  dim3 grid(grid_x, k_splits);
  kern<<<grid, WGM * WGN * 64, lds, st>>>(g);
  return hipGetLastError();
}

}  // namespace moe_gemm
