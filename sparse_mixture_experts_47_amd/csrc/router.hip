// router.hip -- router GEMM, fp32 softmax and wave-level top-k for gfx950.
//
// The router scores every token against every expert's learned vector,
// applies a softmax, and keeps the top-k experts (heavensheep.xyz MoE notes,
// "Routing Function"; "MoE" on ld246.com, Q1: router = FFN + softmax).
// Noisy gating H = x.W_g + N(0,1) * softplus(x.W_noise) follows the
// chiang97912 MoE notes, "KeepTopK 策略". The selection key adds a
// per-expert bias to the softmax score before top-k (ld246.com Q3, item 2).
#include <math.h>

#include "gemm_bf16.h"
#include "moe_device.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;

// Tokens per wave in the select kernel: one while that leaves the GPU
// short of waves (few tokens: the kernel is latency bound), four for large
// batches (fewer per-block score partials to sum afterwards).
inline int select_tok_per_wave(int N) { return N >= 2048 ? 4 : 1; }
// K splits of the router GEMM whose partials the select kernel adds itself
// (loaded together, summed in order); up to kMaxGemmSplits (a few tokens:
// few tiles, so the weight planes need many workgroups) a reduce kernel
// adds them first
constexpr int kMaxSplits = 8;
constexpr int kMaxGemmSplits = 64;
inline int select_blocks(int N) {
  const int per_block = select_tok_per_wave(N) * kWaves;
  return (N + per_block - 1) / per_block;
}

// ---------------------------------------------------------------- GEMM
// out[t][c] = sum_k x[t][k] * W[c][k] with W = [w_gate ; w_noise] (E or 2E
// rows), fp32 accumulation in k order. Tiles: BM tokens x BN router columns,
// BK-wide K steps, each thread a TM x TN register block. x is bf16 or fp32.
template <int BM, int BN, int BK, int TM, int TN, bool XBF16>
__global__ __launch_bounds__(kThreads) void router_gemm_kernel(
    const void* __restrict__ xv, const float* __restrict__ wg, const float* __restrict__ wn,
    float* __restrict__ out, int N, int d, int E, int E2) {
  static_assert((BM / TM) * (BN / TN) == kThreads, "tile");
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % (BN / TN), ty = tid / (BN / TN);
  const int t0 = blockIdx.x * BM, c0 = blockIdx.y * BN;
  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  // staging: each thread loads groups of 4 consecutive K values (one A row
  // segment and, while there are B rows left, one B row segment per group),
  // one K step ahead into registers; past-the-end rows and K load zeros
  constexpr int AG = BM * BK / 4 / kThreads, BG = (BN * BK / 4 + kThreads - 1) / kThreads;
  static_assert(AG >= 1 && AG * kThreads * 4 == BM * BK, "A staging");
  const bool vec = (d & 3) == 0;
  auto ldx = [&](int t, int k) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (t >= N) return v;
    const size_t off = (size_t)t * d + k;
    if constexpr (XBF16) {
      for (int q = 0; q < 4; ++q)
        if (k + q < d) v[q] = moe::bf16_bits_to_f32(((const uint16_t*)xv)[off + q]);
    } else {
      if (vec && k + 3 < d) return *(const f32x4_t*)((const float*)xv + off);
      for (int q = 0; q < 4; ++q)
        if (k + q < d) v[q] = ((const float*)xv)[off + q];
    }
    return v;
  };
  auto ldw = [&](int c, int k) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (c >= E2) return v;
    const float* row = c < E ? wg + (size_t)c * d : wn + (size_t)(c - E) * d;
    if (vec && k + 3 < d) return *(const f32x4_t*)(row + k);
    for (int q = 0; q < 4; ++q)
      if (k + q < d) v[q] = row[k + q];
    return v;
  };
  f32x4_t ar[AG], br[BG];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < AG; ++u) {
      const int i = tid + u * kThreads, m = i / (BK / 4), kq = (i % (BK / 4)) * 4;
      ar[u] = ldx(t0 + m, k0 + kq);
    }
#pragma unroll
    for (int u = 0; u < BG; ++u) {
      const int i = tid + u * kThreads, n = i / (BK / 4), kq = (i % (BK / 4)) * 4;
      br[u] = i < BN * BK / 4 ? ldw(c0 + n, k0 + kq) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < d; k0 += BK) {
#pragma unroll
    for (int u = 0; u < AG; ++u) {
      const int i = tid + u * kThreads, m = i / (BK / 4), kq = (i % (BK / 4)) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) As[kq + q][m] = ar[u][q];
    }
#pragma unroll
    for (int u = 0; u < BG; ++u) {
      const int i = tid + u * kThreads, n = i / (BK / 4), kq = (i % (BK / 4)) * 4;
      if (i < BN * BK / 4)
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[kq + q][n] = br[u][q];
    }
    __syncthreads();
    if (k0 + BK < d) fetch(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = As[kk][ty * TM + i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = Bs[kk][tx * TN + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int t = t0 + ty * TM + i;
    if (t >= N) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int c = c0 + tx * TN + j;
      if (c < E2) out[(size_t)t * E2 + c] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------- select
struct SelectArgs {
  int N, E, k, C, renorm;
  const float* src;  // [nsplit][N][stride]: logits, then (if noise) E noise columns
  int stride;
  int nsplit;        // K-split partials summed in order s = 0 .. nsplit-1
  long long split_stride;
  int from_gemm;     // 1: apply logit_bias and noise to src; 0: src is logits_in
  int noise;
  const float* logit_bias;
  const float* select_bias;
  uint64_t seed;
  int32_t* cand;
  float* cand_s;
  float* gates;
  float* logits_out;
  float* scores_out;  // [N][E] softmax scores, or null
  float* noise_out;   // [N][E] noise pre-activations v, or null
  double* partials;  // [gridDim.x][E+1] or null
  int tok_per_wave;
};

__device__ __forceinline__ float pick(const float* v, int slot, int n) {
  float r = v[0];
#pragma unroll
  for (int s = 1; s < 4; ++s)
    if (s < n && slot == s) r = v[s];
  return r;
}

// The logit a token's softmax sees for expert e, from the summed GEMM
// outputs v (x . w_gate) and nv (x . w_noise): + logit bias, then noisy
// gating H = l + z * softplus(nv) (chiang97912 "KeepTopK 策略"); also
// written out when asked for.
__device__ __forceinline__ float token_logit(const SelectArgs& a, int t, int e, float v,
                                             float nv) {
  const int E = a.E;
  if (a.from_gemm) {
    if (a.logit_bias) v = v + a.logit_bias[e];
    if (a.noise) {
      if (a.noise_out) a.noise_out[(size_t)t * E + e] = nv;
      const float sp = nv > 20.f ? nv : (float)log1p(exp((double)nv));
      const float z = moe::noise_normal(a.seed, (uint32_t)t, (uint32_t)e, (uint32_t)E);
      v = __builtin_fmaf(z, sp, v);
    }
  }
  if (a.logits_out) a.logits_out[(size_t)t * E + e] = v;
  return v;
}

// Softmax, top-C and gates of token t, one wave; expert e lives in lane
// e % 64, register slot e / 64 (l = -inf where !valid). Adds the token's
// scores to acc and lse^2 to lse2 (lane 0) for the balance statistics.
// Softmax tree: the zero-padded 256-wide halving tree equals the tree padded
// to the next power of two (adding +0 changes nothing), so in-lane slot
// sums (0+2, 1+3, then the two) are the h = 128 and h = 64 levels and the
// wave butterfly does h = 32 .. 1.
template <int SLOTS>
__device__ __forceinline__ void finish_token(const SelectArgs& a, int t, int lane,
                                             const float (&l)[SLOTS],
                                             const bool (&valid)[SLOTS], double (&acc)[SLOTS],
                                             double& lse2) {
  float m = l[0];
#pragma unroll
  for (int s = 1; s < SLOTS; ++s) m = fmaxf(m, l[s]);
  m = moe::wave_max(m);

  float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    float dlt = l[s] - m;
    u[s] = (valid[s] && !(dlt < -87.0f)) ? moe::softmax_exp(dlt) : 0.f;
  }
  float part;
  {
#pragma clang fp contract(off)
    float a0 = u[0] + u[2];
    float a1 = u[1] + u[3];
    part = a0 + a1;
  }
  const float S = moe::wave_tree_sum(part);

  float sc[4] = {0.f, 0.f, 0.f, 0.f};
  uint64_t key[4] = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = lane + 64 * s;
    if (valid[s]) {
      sc[s] = u[s] / S;
      if (a.scores_out) a.scores_out[(size_t)t * a.E + e] = sc[s];
      float kv = a.select_bias ? sc[s] + a.select_bias[e] : sc[s];
      if (kv == 0.0f) kv = 0.0f;
      key[s] = ((uint64_t)moe::orderable(kv) << 32) | (uint32_t)(0xFFFFu - (uint32_t)e);
      acc[s] += (double)sc[s];
    }
  }
  if (lane == 0) {
    double lse = (double)m + log((double)S);
    lse2 += lse * lse;
  }

  // top-C: C rounds of a wave-wide max over each lane's best remaining key
  uint64_t best = key[0];
#pragma unroll
  for (int s = 1; s < SLOTS; ++s) best = key[s] > best ? key[s] : best;
  int my_c = 0;
  float my_cs = 0.f;
  for (int j = 0; j < a.C; ++j) {
    const uint64_t w = moe::wave_max_u64(best);
    const int ew = (int)(0xFFFFu - (uint32_t)(w & 0xFFFFu));
    const int owner = ew & 63, slot = ew >> 6;
    const float sw = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(pick(sc, slot, SLOTS)), owner));
    if (lane == j) {
      my_c = ew;
      my_cs = sw;
    }
    if (lane == owner) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        if (s == slot) key[s] = 0;
      best = key[0];
#pragma unroll
      for (int s = 1; s < SLOTS; ++s) best = key[s] > best ? key[s] : best;
    }
  }
  if (lane < a.C) {
    a.cand[(size_t)t * a.C + lane] = my_c;
    a.cand_s[(size_t)t * a.C + lane] = my_cs;
  }
  float Sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_cs), 0));
  for (int j = 1; j < a.k; ++j) {
#pragma clang fp contract(off)
    Sk = Sk + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_cs), j));
  }
  if (lane < a.k) a.gates[(size_t)t * a.k + lane] = a.renorm ? my_cs / Sk : my_cs;
}

// The block's sums of every expert's scores and of lse^2, waves added in
// order, as one row of the per-block partials.
template <int SLOTS>
__device__ __forceinline__ void write_partials(const SelectArgs& a, int lane, int wave,
                                               const double (&acc)[SLOTS], double lse2,
                                               double (*red)[257]) {
  const int E = a.E;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = lane + 64 * s;
    if (e < E) red[wave][e] = acc[s];
  }
  if (lane == 0) red[wave][E] = lse2;
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += kThreads) {
    double v = red[0][e];
#pragma unroll
    for (int w = 1; w < kThreads / MOE_WAVE; ++w) v += red[w][e];
    a.partials[(size_t)blockIdx.x * (E + 1) + e] = v;
  }
}

// One wave per token (tok_per_wave tokens in turn) over logits that come in
// (logits_in) or as K-split GEMM partials (summed in split order).
template <int SLOTS>
__global__ __launch_bounds__(kThreads) void router_select_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ double red[kThreads / MOE_WAVE][257];
  double acc[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) acc[s] = 0.0;
  double lse2 = 0.0;
  const int E = a.E;

  const int tpw = a.tok_per_wave;
  for (int i = 0; i < tpw; ++i) {
    const int t = (blockIdx.x * kWaves + wave) * tpw + i;
    if (t >= a.N) break;
    const float* row = a.src + (size_t)t * a.stride;
    float l[SLOTS];
    bool valid[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int e = lane + 64 * s;
      valid[s] = e < E;
      float v = -INFINITY;
      if (valid[s]) {
        // all split partials are loaded before the in-order sum (unrolled:
        // the loads of every slot go out together)
        float pv[kMaxSplits];
#pragma unroll
        for (int q = 0; q < kMaxSplits; ++q)
          pv[q] = q < a.nsplit ? row[q * a.split_stride + e] : 0.f;
        v = pv[0];
#pragma unroll
        for (int q = 1; q < kMaxSplits; ++q)
          if (q < a.nsplit) v = v + pv[q];
        float nv = 0.f;
        if (a.from_gemm && a.noise) {
#pragma unroll
          for (int q = 0; q < kMaxSplits; ++q)
            pv[q] = q < a.nsplit ? row[q * a.split_stride + E + e] : 0.f;
          nv = pv[0];
#pragma unroll
          for (int q = 1; q < kMaxSplits; ++q)
            if (q < a.nsplit) nv = nv + pv[q];
        }
        v = token_logit(a, t, e, v, nv);
      }
      l[s] = v;
    }
    finish_token<SLOTS>(a, t, lane, l, valid, acc, lse2);
  }
  if (a.partials) write_partials<SLOTS>(a, lane, wave, acc, lse2, red);
}

// ---------------------------------------------------------------- fused router
// Router GEMM, softmax, top-k and gates in one kernel for up to 32 GEMM
// columns (experts and noise columns) and bf16 x: the logits of the block's
// 16 RB tokens never leave the CU. 16 waves split the work as NCB 16-column
// blocks x KW = 16 / NCB K slices: slice s takes the 64-wide K steps s,
// s + KW, s + 2 KW, ..., loading step i+1 while multiplying step i. Each wave
// multiplies the token rows, read straight from global memory, with the
// router weights' three bf16 planes on v_mfma_f32_16x16x32_bf16 (every
// product exact in fp32); the K-slice partial sums meet in LDS and are
// added in slice order, then each wave runs softmax and top-k for RB
// tokens, expert e in lane e. Sixteen waves keep enough loads in flight to
// stream x at HBM speed with one block per CU.
//
// MFMA operands: lane l supplies row (token, or weight column) l % 16 and
// K values kl .. kl+15, kl = k + 16 (l / 16), as two 8-value halves for two
// MFMAs; A and B use the same K assignment, so the two MFMAs together sum
// 64 distinct K. Result register r of lane l: token 4 (l / 16) + r, column
// l % 16.
struct FusedArgs {
  const uint16_t* x;        // [N][d] bf16
  const uint16_t* planes;   // [3][E2pad][d] bf16: hi, mid, lo
  long long plane_stride;   // E2pad * d
  int d;
};

constexpr int kFusedWaves = 16;

__device__ __forceinline__ float add_nc(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// PACK (at most 8 GEMM columns, NCB = 1): the 16 MFMA columns carry the hi
// plane in columns 0-7 and the mid plane in 8-15, and a second operand the
// lo plane in 0-7 (zero in 8-15), so each K step takes two products and two
// thirds of the plane bytes; a K slice's logit is then (hi + mid) + lo.
template <int RB, int NCB, bool PACK>
__global__ __launch_bounds__(kFusedWaves * 64) void router_fused_kernel(FusedArgs f,
                                                                        SelectArgs a) {
  static_assert(!PACK || NCB == 1, "packed planes: one column block");
  constexpr int NP = PACK ? 2 : 3;  // B operands per K step
  constexpr int TM = 16 * RB, W = NCB * 16;
  constexpr int KW = kFusedWaves / NCB;  // K slices; wave = (column block, K slice)
  __shared__ float part[KW][TM][W + 1];
  __shared__ float tile[TM][W + 1];
  __shared__ double red[kFusedWaves][65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % KW, cb = wave / KW;
  const int t0 = blockIdx.x * TM;
  const int r16 = lane & 15, grp = lane >> 4;
  const int d = f.d, nsteps = d / 64;
  const uint16_t* xr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = min(t0 + rb * 16 + r16, a.N - 1);  // rows past N read row N-1
    xr[rb] = f.x + (size_t)t * d + grp * 16;
  }
  // B operand p of this lane: plane p, row cb * 16 + r16; packed: hi or mid
  // (r16 < 8 or not) row r16 % 8, then lo row r16 (lanes with r16 >= 8 load
  // nothing and supply zeros)
  const uint16_t* wr[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (PACK)
      wr[p] = f.planes + (p == 0 ? (r16 < 8 ? 0 : f.plane_stride) : 2 * f.plane_stride) +
              (size_t)(r16 & 7) * d + grp * 16;
    else
      wr[p] = f.planes + p * f.plane_stride + (size_t)(cb * 16 + r16) * d + grp * 16;
  }
  const bool wlive1 = !PACK || r16 < 8;
  // one 64-wide K step: x (two 8-value halves per row block) and the weight
  // operands
  struct Step {
    u32x4_t x[RB][2];
    u32x4_t w[NP][2];
  };
  auto load = [&](Step& o, int st) {
    const int k = st * 64;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      o.x[rb][0] = *(const u32x4_t*)(xr[rb] + k);
      o.x[rb][1] = *(const u32x4_t*)(xr[rb] + k + 8);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint16_t* w = wr[p] + k;
      if (p == 0 || wlive1) {
        o.w[p][0] = *(const u32x4_t*)w;
        o.w[p][1] = *(const u32x4_t*)(w + 8);
      } else {
        o.w[p][0] = u32x4_t{0u, 0u, 0u, 0u};
        o.w[p][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  // packed: acc[.][0] sums hi | mid, acc[.][1] sums lo; else one sum
  constexpr int NA = PACK ? 2 : 1;
  f32x4_t acc[RB][NA];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int q = 0; q < NA; ++q) acc[rb][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mult = [&](const Step& o) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int q = PACK ? p : 0;
          acc[rb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, o.x[rb][h]), __builtin_bit_cast(bf16x8_t, o.w[p][h]),
              acc[rb][q], 0, 0, 0);
        }
  };
  // Slice ks holds steps ks, ks + KW, ...; blocks start their walk at
  // different steps of the slice so that they do not all read the same
  // weight lines at once. The loads of the next step go out before the
  // products of this one (two buffers, unrolled by hand so that both stay in
  // registers); the last prefetch re-reads a step instead of branching, so
  // the compiler's load counters stay exact.
  const int nper = nsteps > ks ? (nsteps - ks + KW - 1) / KW : 0;
  const int rot = nper ? (int)(blockIdx.x % nper) : 0;
  auto step_of = [&](int j) {
    int q = j + rot;
    q = q >= nper ? q - nper : q;
    return ks + q * KW;
  };
  Step b0, b1;
  int j = 0;
  // a short slice: every step's loads go out at once (one wait for the
  // memory latency instead of one per step), products in the same order
  // (Mixtral-shaped router, four steps a slice: 21.1 -> 19.0 us a call);
  // only where four steps fit in 96 of the 128 VGPRs a lane has at 16 waves
  constexpr int kStepRegs = (RB * 2 + NP * 2) * 4;
  if constexpr (4 * kStepRegs <= 96) if (nper <= 4) {
    Step b2, b3;
    if (nper > 0) load(b0, step_of(0));
    if (nper > 1) load(b1, step_of(1));
    if (nper > 2) load(b2, step_of(2));
    if (nper > 3) load(b3, step_of(3));
    __builtin_amdgcn_sched_barrier(0);
    if (nper > 0) mult(b0);
    if (nper > 1) mult(b1);
    if (nper > 2) mult(b2);
    if (nper > 3) mult(b3);
    j = nper;
  }
  if (j < nper) load(b0, step_of(0));
  while (j < nper) {
    load(b1, step_of(min(j + 1, nper - 1)));
    __builtin_amdgcn_sched_barrier(0);
    mult(b0);
    __builtin_amdgcn_sched_barrier(0);
    if (++j >= nper) break;
    load(b0, step_of(min(j + 1, nper - 1)));
    __builtin_amdgcn_sched_barrier(0);
    mult(b1);
    __builtin_amdgcn_sched_barrier(0);
    ++j;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = acc[rb][0][r];
      if (PACK) {
        // column r16 < 8: its hi sum here, its mid sum 8 lanes on (row_ror:8)
        const float mid = __uint_as_float(moe::detail::dpp<0x128>(__float_as_uint(v)));
        v = add_nc(add_nc(v, mid), acc[rb][1][r]);
      }
      if (!PACK || r16 < 8) part[ks][rb * 16 + 4 * grp + r][cb * 16 + r16] = v;
    }
  __syncthreads();
  // the K slices, added in slice order
  for (int i = threadIdx.x; i < TM * W; i += kFusedWaves * 64) {
    const int row = i / W, col = i % W;
    float v = part[0][row][col];
#pragma unroll
    for (int q = 1; q < KW; ++q) v = v + part[q][row][col];
    tile[row][col] = v;
  }
  __syncthreads();
  double sacc[1] = {0.0};
  double lse2 = 0.0;
  const int E = a.E;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int ti = rb * kFusedWaves + wave, tt = t0 + ti;
    if (tt < a.N) {
      float l[1] = {-INFINITY};
      bool valid[1] = {lane < E};
      if (valid[0])
        l[0] = token_logit(a, tt, lane, tile[ti][lane], a.noise ? tile[ti][E + lane] : 0.f);
      finish_token<1>(a, tt, lane, l, valid, sacc, lse2);
    }
  }
  if (a.partials) {
    if (lane < E) red[wave][lane] = sacc[0];
    if (lane == 0) red[wave][E] = lse2;
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += kFusedWaves * 64) {
      double v = red[0][e];
#pragma unroll
      for (int w = 1; w < kFusedWaves; ++w) v += red[w][e];
      a.partials[(size_t)blockIdx.x * (E + 1) + e] = v;
    }
  }
}

// The router weights as three bf16 planes whose sum is the fp32 value:
// hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each step
// exact in fp32). Rows: w_gate 0..E-1, w_noise E..2E-1, zero padding.
// x is bf16, so x . W runs on bf16 MFMA with every product exact. Four
// consecutive k per thread (d is a multiple of 64 on this path).
__global__ __launch_bounds__(kThreads) void router_split_weights_kernel(
    const float* __restrict__ wg, const float* __restrict__ wn, int E, int E2, int E2pad, int d,
    uint16_t* __restrict__ planes) {
  const size_t n = (size_t)E2pad * d, n4 = n / 4;
  for (size_t i4 = (size_t)blockIdx.x * kThreads + threadIdx.x; i4 < n4;
       i4 += (size_t)gridDim.x * kThreads) {
    const size_t i = i4 * 4;
    const int c = (int)(i / d), k = (int)(i % d);
    f32x4_t w = {0.f, 0.f, 0.f, 0.f};
    if (c < E) w = *(const f32x4_t*)(wg + (size_t)c * d + k);
    else if (c < E2) w = *(const f32x4_t*)(wn + (size_t)(c - E) * d + k);
    uint16_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hi[j] = moe::f32_to_bf16_bits(w[j]);
      const float r1 = w[j] - moe::bf16_bits_to_f32(hi[j]);
      mid[j] = moe::f32_to_bf16_bits(r1);
      lo[j] = moe::f32_to_bf16_bits(r1 - moe::bf16_bits_to_f32(mid[j]));
    }
    auto pack = [](const uint16_t* v) {
      return make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                        (uint32_t)v[2] | ((uint32_t)v[3] << 16));
    };
    *(uint2*)(planes + i) = pack(hi);
    *(uint2*)(planes + n + i) = pack(mid);
    *(uint2*)(planes + 2 * n + i) = pack(lo);
  }
}

// More K splits than the select kernel adds itself: every logit's split
// partials added in split order (all loaded first) into split 0's slot.
__global__ __launch_bounds__(kThreads) void router_split_reduce_kernel(float* __restrict__ raw,
                                                                       int nsplit,
                                                                       long long stride) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < stride;
       i += (long long)gridDim.x * kThreads) {
    float pv[kMaxGemmSplits];
#pragma unroll
    for (int q = 0; q < kMaxGemmSplits; ++q) pv[q] = q < nsplit ? raw[q * stride + i] : 0.f;
    float v = pv[0];
#pragma unroll
    for (int q = 1; q < kMaxGemmSplits; ++q)
      if (q < nsplit) v = v + pv[q];
    raw[i] = v;
  }
}

// score_sums[e] = sum over blocks b of partials[b][e]: one workgroup per
// column; thread i adds rows i, i + 256, ... in order, then a fixed halving
// tree over the 256 threads. The order never changes, so the sum is
// reproducible bit for bit.
__global__ __launch_bounds__(kThreads) void router_sum_partials_kernel(
    const double* __restrict__ partials, int nblk, int width, double* __restrict__ out) {
  __shared__ double buf[kThreads];
  const int e = blockIdx.x;
  double v = 0.0;
  for (int b = threadIdx.x; b < nblk; b += kThreads) v += partials[(size_t)b * width + e];
  buf[threadIdx.x] = v;
  __syncthreads();
  for (int h = kThreads / 2; h >= 1; h >>= 1) {
    if ((int)threadIdx.x < h) buf[threadIdx.x] += buf[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = buf[0];
}

}  // namespace

// ---------------------------------------------------------------- host side
namespace moe_host {

namespace {
// Router GEMM: 128-row M tiles, 64 columns of each of the three weight
// planes, 4 waves, two 40 KB LDS stages so that two workgroups share a CU
// (measured: 3 stages with one workgroup per CU, or 256-row tiles on 8
// waves, are 1.2-1.6x slower for the DeepSeek-shaped router)
constexpr int kRouterBM = 128;

struct RouterPlan {
  bool mfma;
  int bm;
  int E2, E2pad, bn, nsplit, k_chunk;
  size_t planes_bytes, raw_bytes, stat_bytes;
};

RouterPlan plan_router(int N, int d, int E, int with_noise, bool x_bf16) {
  RouterPlan p{};
  p.E2 = with_noise ? 2 * E : E;
  p.mfma = x_bf16 && d > 0 && d % 64 == 0;
  p.nsplit = 1;
  p.k_chunk = d;
  p.bm = kRouterBM;
  if (p.mfma) {
    p.bn = 64;
    p.E2pad = (p.E2 + p.bn - 1) / p.bn * p.bn;
    const int tiles = ((N + p.bm - 1) / p.bm) * (p.E2pad / p.bn);
    const int KT = d / 64;
    // enough K splits for ~512 workgroups
    int want = (512 + tiles - 1) / tiles;
    want = want < 1 ? 1 : (want > kMaxGemmSplits ? kMaxGemmSplits : want);
    want = want > KT ? KT : want;
    const int steps = (KT + want - 1) / want;
    p.k_chunk = steps * 64;
    p.nsplit = (KT + steps - 1) / steps;
    p.planes_bytes = align256((size_t)3 * p.E2pad * d * sizeof(uint16_t));
  } else {
    p.bn = 0;
    p.E2pad = p.E2;
  }
  p.raw_bytes = align256((size_t)p.nsplit * N * p.E2pad * sizeof(float));
  const size_t nblk = (size_t)select_blocks(N);
  p.stat_bytes = align256(nblk * (E + 1) * sizeof(double));
  return p;
}
}  // namespace

size_t router_workspace_bytes(int N, int d, int E, int with_noise) {
  // the larger of the two plans (x dtype is not known at query time)
  RouterPlan a = plan_router(N, d, E, with_noise, true);
  RouterPlan b = plan_router(N, d, E, with_noise, false);
  size_t sa = a.planes_bytes + a.raw_bytes + a.stat_bytes;
  size_t sb = b.planes_bytes + b.raw_bytes + b.stat_bytes;
  return sa > sb ? sa : sb;
}

size_t router_planes_bytes(int E, int d, int with_noise) {
  const int E2 = with_noise ? 2 * E : E;
  const int E2pad = (E2 + 63) / 64 * 64;
  return (size_t)3 * E2pad * d * sizeof(uint16_t);
}

moe_status router_prepare_launch(const float* w_gate, const float* w_noise, int E, int d,
                                 uint16_t* planes, hipStream_t st) {
  const int E2 = w_noise ? 2 * E : E;
  const int E2pad = (E2 + 63) / 64 * 64;
  const size_t n = (size_t)E2pad * d;
  const size_t sblk = (n / 4 + kThreads - 1) / kThreads;
  const int sgrid = (int)(sblk < 2048 ? sblk : 2048);
  router_split_weights_kernel<<<sgrid, kThreads, 0, st>>>(w_gate, w_noise, E, E2, E2pad, d,
                                                          planes);
  return launch_status("router weight planes");
}

namespace {
// The fused kernel serves bf16 x (d % 64 == 0) and up to 32 GEMM columns
// (experts, plus their noise columns). Its 32-token blocks each read the
// whole weight planes, so with more columns the plane traffic outgrows x
// and the split-K GEMM with its 128-row tiles followed by the select kernel
// is faster (measured on 64 experts with noise: 155 us fused against 62).
bool fused_router(const RouterPlan& pl, int E) { return pl.mfma && E <= 32 && pl.E2 <= 32; }

// Tokens a block: 16, or 32 once that still gives a block to every CU (the
// weight planes are then read once per 32 tokens and the grid runs in one
// round: one GPU's EP-8 DeepSeek share, 8192 tokens x 32 experts, 121 ->
// 82 us; with 4096 tokens the 128 blocks of 32 leave half the CUs idle,
// 19 -> 27.5 us)
inline int fused_rb(int N) { return N >= 32 * 256 ? 2 : 1; }

template <int RB>
void launch_fused_rb(int ncb, int nblk, const FusedArgs& f, const SelectArgs& a,
                     hipStream_t st) {
  constexpr int th = kFusedWaves * 64;
  if (ncb == 0)
    router_fused_kernel<RB, 1, true><<<nblk, th, 0, st>>>(f, a);
  else if (ncb == 1)
    router_fused_kernel<RB, 1, false><<<nblk, th, 0, st>>>(f, a);
  else
    router_fused_kernel<RB, 2, false><<<nblk, th, 0, st>>>(f, a);
}

hipError_t launch_fused(int ncb, int rb, int nblk, const FusedArgs& f, const SelectArgs& a,
                        hipStream_t st) {
  if (rb == 2)
    launch_fused_rb<2>(ncb, nblk, f, a, st);
  else
    launch_fused_rb<1>(ncb, nblk, f, a, st);
  return hipGetLastError();
}
}  // namespace

moe_status router_launch(const moe_router_params* p, const void* x, moe_dtype x_dt,
                         const float* w_gate, const float* logits_in, int32_t* cand_ids,
                         float* cand_scores, float* gates, float* logits_out,
                         double* score_sums, void* workspace, hipStream_t st) {
  const int N = p->n_tokens, d = p->d_model, E = p->n_experts;
  const int noise = (!logits_in && p->w_noise) ? 1 : 0;
  // same effective d as the workspace check: no GEMM when logits come in
  const RouterPlan pl = plan_router(N, logits_in ? 0 : d, E, noise, x_dt == MOE_BF16);
  int nblk = select_blocks(N);
  char* ws = (char*)workspace;
  uint16_t* planes = (uint16_t*)ws;
  float* raw = (float*)(ws + pl.planes_bytes);
  double* partials = (double*)(ws + pl.planes_bytes + pl.raw_bytes);

  SelectArgs a;
  a.N = N;
  a.E = E;
  a.k = p->top_k;
  a.C = p->n_cand;
  a.renorm = p->renormalize;
  a.src = logits_in;
  a.stride = E;
  a.nsplit = 1;
  a.split_stride = (long long)N * E;
  a.from_gemm = logits_in ? 0 : 1;
  a.noise = noise;
  a.logit_bias = logits_in ? nullptr : p->logit_bias;
  a.select_bias = p->select_bias;
  a.seed = p->noise_seed;
  a.cand = cand_ids;
  a.cand_s = cand_scores;
  a.gates = gates;
  a.logits_out = logits_out;
  a.scores_out = p->scores_out;
  a.noise_out = p->noise_out;
  a.partials = score_sums ? partials : nullptr;
  a.tok_per_wave = select_tok_per_wave(N);

  bool selected = false;
  if (!logits_in) {
    const int E2 = pl.E2;
    if (pl.mfma) {
      const size_t n = (size_t)pl.E2pad * d;
      const bool fused = fused_router(pl, E);
      // weight planes: the caller's prepared ones, else split into the
      // workspace now
      if (!p->w_planes) {
        const size_t sblk = (n / 4 + kThreads - 1) / kThreads;
        const int sgrid = (int)(sblk < 2048 ? sblk : 2048);
        router_split_weights_kernel<<<sgrid, kThreads, 0, st>>>(w_gate, p->w_noise, E, E2,
                                                                pl.E2pad, d, planes);
        moe_status s = launch_status("router weight split");
        if (s != MOE_OK) return s;
      } else {
        planes = (uint16_t*)p->w_planes;
      }
      if (fused) {
        FusedArgs f{(const uint16_t*)x, planes, (long long)n, d};
        // 0: hi and mid planes packed into one operand (at most 8 columns)
        const int ncb = E2 <= 8 ? 0 : E2 <= 16 ? 1 : 2;
        const int rb = fused_rb(N);
        nblk = (N + 16 * rb - 1) / (16 * rb);
        const hipError_t err = launch_fused(ncb, rb, nblk, f, a, st);
        if (err != hipSuccess) {
          set_error("router (fused): launch failed: %s", hipGetErrorString(err));
          return MOE_EHIP;
        }
        selected = true;
      } else {
      using namespace moe_gemm;
      Args g{};
      g.A = x;
      g.B[0] = planes;
      g.B[1] = planes + n;
      g.B[2] = planes + 2 * n;
      g.bias = nullptr;
      g.C = raw;
      g.K = d;
      g.Nrows = pl.E2pad;
      g.n_valid = E2;
      g.ldc = pl.E2pad;
      g.c_split = (long long)N * pl.E2pad;
      g.k_chunk = pl.k_chunk;
      g.E = 1;
      g.max_mt = (N + pl.bm - 1) / pl.bm;
      g.act = 0;
      g.group_n = 8;
      g.offsets = nullptr;     // one group of N token rows, no tile table
      g.tile_start = nullptr;
      g.rows1 = N;
      const hipError_t err =
          launch_dlds<kRouterBM, 64, 64, 2, 2, 2, 1, 3, EPI_SUM, OUT_F32>(g, pl.nsplit, st);
      if (err != hipSuccess) {
        set_error("router GEMM: launch failed: %s", hipGetErrorString(err));
        return MOE_EHIP;
      }
      a.stride = pl.E2pad;
      a.nsplit = pl.nsplit;
      if (pl.nsplit > kMaxSplits) {
        const long long cnt = (long long)N * pl.E2pad;
        const long long rblk = (cnt + kThreads - 1) / kThreads;
        router_split_reduce_kernel<<<(int)(rblk < 4096 ? rblk : 4096), kThreads, 0, st>>>(
            raw, pl.nsplit, cnt);
        moe_status s = launch_status("router split reduce");
        if (s != MOE_OK) return s;
        a.nsplit = 1;
      }
      }
    } else {
      // a few columns: 64-token tiles with 64-wide K steps (the tiny Switch
      // layer, 256 tokens x d 64 x 4 experts: one 256-token block walking
      // four 16-wide steps, each a global-load round trip, took 9.1 us)
      if (E2 <= 16) {
        dim3 grid((N + 63) / 64, 1);
        if (x_dt == MOE_BF16)
          router_gemm_kernel<64, 16, 64, 2, 2, true><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
        else
          router_gemm_kernel<64, 16, 64, 2, 2, false><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
      } else {
        dim3 grid((N + 63) / 64, (E2 + 63) / 64);
        if (x_dt == MOE_BF16)
          router_gemm_kernel<64, 64, 16, 4, 4, true><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
        else
          router_gemm_kernel<64, 64, 16, 4, 4, false><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
      }
      moe_status s = launch_status("router_gemm");
      if (s != MOE_OK) return s;
      a.stride = E2;
    }
    a.src = raw;
    a.split_stride = (long long)N * a.stride;
  }
  moe_status s = MOE_OK;
  if (!selected) {
    if (E <= 64)
      router_select_kernel<1><<<nblk, kThreads, 0, st>>>(a);
    else if (E <= 128)
      router_select_kernel<2><<<nblk, kThreads, 0, st>>>(a);
    else
      router_select_kernel<4><<<nblk, kThreads, 0, st>>>(a);
    s = launch_status("router_select");
    if (s != MOE_OK) return s;
  }
  if (score_sums) {
    router_sum_partials_kernel<<<E + 1, kThreads, 0, st>>>(partials, nblk, E + 1, score_sums);
    s = launch_status("router_sum_partials");
  }
  return s;
}

}  // namespace moe_host
