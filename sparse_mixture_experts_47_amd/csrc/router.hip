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
constexpr int kMaxSplits = 8;  // K splits of the router GEMM (partials summed in order)
inline int select_blocks(int N) {
  const int per_block = select_tok_per_wave(N) * kWaves;
  return (N + per_block - 1) / per_block;
}

// ---------------------------------------------------------------- GEMM
// out[t][c] = sum_k x[t][k] * W[c][k] with W = [w_gate ; w_noise] (E or 2E
// rows), fp32 accumulation. Tiles: BM tokens x BN router columns, BK = 16,
// each thread a 4x4 register block. x is bf16 or fp32.
template <int BM, int BN, bool XBF16>
__global__ __launch_bounds__(kThreads) void router_gemm_kernel(
    const void* __restrict__ xv, const float* __restrict__ wg, const float* __restrict__ wn,
    float* __restrict__ out, int N, int d, int E, int E2) {
  constexpr int BK = 16, TM = 4, TN = 4;
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

// One wave per token (tok_per_wave tokens in turn); expert e lives in lane
// e % 64, register slot e / 64.
// Softmax tree: the zero-padded 256-wide halving tree equals the tree padded
// to the next power of two (adding +0 changes nothing), so in-lane slot
// sums (0+2, 1+3, then the two) are the h = 128 and h = 64 levels and the
// wave butterfly does h = 32 .. 1.
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
        // all split partials are loaded before the in-order sum
        float pv[kMaxSplits];
#pragma unroll
        for (int q = 0; q < kMaxSplits; ++q)
          pv[q] = q < a.nsplit ? row[q * a.split_stride + e] : 0.f;
        v = pv[0];
#pragma unroll
        for (int q = 1; q < kMaxSplits; ++q)
          if (q < a.nsplit) v = v + pv[q];
        if (a.from_gemm) {
          if (a.logit_bias) v = v + a.logit_bias[e];
          if (a.noise) {
#pragma unroll
            for (int q = 0; q < kMaxSplits; ++q)
              pv[q] = q < a.nsplit ? row[q * a.split_stride + E + e] : 0.f;
            float nv = pv[0];
#pragma unroll
            for (int q = 1; q < kMaxSplits; ++q)
              if (q < a.nsplit) nv = nv + pv[q];
            if (a.noise_out) a.noise_out[(size_t)t * E + e] = nv;
            float sp = nv > 20.f ? nv : (float)log1p(exp((double)nv));
            float z = moe::noise_normal(a.seed, (uint32_t)t, (uint32_t)e, (uint32_t)E);
            v = __builtin_fmaf(z, sp, v);
          }
        }
        if (a.logits_out) a.logits_out[(size_t)t * E + e] = v;
      }
      l[s] = v;
    }
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
        if (a.scores_out) a.scores_out[(size_t)t * E + e] = sc[s];
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
      const float sw = __shfl(pick(sc, slot, SLOTS), owner, MOE_WAVE);
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
    float Sk = __shfl(my_cs, 0, MOE_WAVE);
    for (int j = 1; j < a.k; ++j) {
#pragma clang fp contract(off)
      Sk = Sk + __shfl(my_cs, j, MOE_WAVE);
    }
    if (lane < a.k) a.gates[(size_t)t * a.k + lane] = a.renorm ? my_cs / Sk : my_cs;
  }

  if (a.partials) {
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
}

// The router weights as three bf16 planes whose sum is the fp32 value:
// hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each step
// exact in fp32). Rows: w_gate 0..E-1, w_noise E..2E-1, zero padding.
// x is bf16, so x . W runs on bf16 MFMA with every product exact. Four
// consecutive k per thread (d is a multiple of 64 on this path). The first
// thread also writes the one-group tile table of the GEMM over N token
// rows: offsets = {0, N}, tile_start = {0, ceil(N / bm)}.
__global__ __launch_bounds__(kThreads) void router_split_weights_kernel(
    const float* __restrict__ wg, const float* __restrict__ wn, int E, int E2, int E2pad, int d,
    uint16_t* __restrict__ planes, int N, int bm, int32_t* __restrict__ table) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    table[0] = 0;
    table[1] = N;
    table[2] = 0;
    table[3] = (N + bm - 1) / bm;
  }
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
  size_t planes_bytes, raw_bytes, table_bytes, stat_bytes;
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
    // enough K splits for ~512 workgroups, at most 8 (the select kernel sums
    // the split partials of every logit in order)
    int want = (512 + tiles - 1) / tiles;
    want = want < 1 ? 1 : (want > kMaxSplits ? kMaxSplits : want);
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
  p.table_bytes = 256;
  const size_t nblk = (size_t)select_blocks(N);
  p.stat_bytes = align256(nblk * (E + 1) * sizeof(double));
  return p;
}
}  // namespace

size_t router_workspace_bytes(int N, int d, int E, int with_noise) {
  // the larger of the two plans (x dtype is not known at query time)
  RouterPlan a = plan_router(N, d, E, with_noise, true);
  RouterPlan b = plan_router(N, d, E, with_noise, false);
  size_t sa = a.planes_bytes + a.raw_bytes + a.table_bytes + a.stat_bytes;
  size_t sb = b.planes_bytes + b.raw_bytes + b.table_bytes + b.stat_bytes;
  return sa > sb ? sa : sb;
}

moe_status router_launch(const moe_router_params* p, const void* x, moe_dtype x_dt,
                         const float* w_gate, const float* logits_in, int32_t* cand_ids,
                         float* cand_scores, float* gates, float* logits_out,
                         double* score_sums, void* workspace, hipStream_t st) {
  const int N = p->n_tokens, d = p->d_model, E = p->n_experts;
  const int noise = (!logits_in && p->w_noise) ? 1 : 0;
  // same effective d as the workspace check: no GEMM when logits come in
  const RouterPlan pl = plan_router(N, logits_in ? 0 : d, E, noise, x_dt == MOE_BF16);
  const int nblk = select_blocks(N);
  char* ws = (char*)workspace;
  uint16_t* planes = (uint16_t*)ws;
  float* raw = (float*)(ws + pl.planes_bytes);
  int32_t* table = (int32_t*)(ws + pl.planes_bytes + pl.raw_bytes);
  double* partials = (double*)(ws + pl.planes_bytes + pl.raw_bytes + pl.table_bytes);

  const float* src = logits_in;
  int stride = E, nsplit = 1;
  if (!logits_in) {
    const int E2 = pl.E2;
    if (pl.mfma) {
      const size_t n = (size_t)pl.E2pad * d;
      const size_t sblk = (n / 4 + kThreads - 1) / kThreads;
      const int sgrid = (int)(sblk < 2048 ? sblk : 2048);
      router_split_weights_kernel<<<sgrid, kThreads, 0, st>>>(w_gate, p->w_noise, E, E2,
                                                              pl.E2pad, d, planes, N, pl.bm,
                                                              table);
      moe_status s = launch_status("router weight split");
      if (s != MOE_OK) return s;
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
      g.offsets = table;
      g.tile_start = table + 2;
      const hipError_t err =
          launch_dlds<kRouterBM, 64, 64, 2, 2, 2, 1, 3, EPI_SUM, OUT_F32>(g, pl.nsplit, st);
      if (err != hipSuccess) {
        set_error("router GEMM: launch failed: %s", hipGetErrorString(err));
        return MOE_EHIP;
      }
      stride = pl.E2pad;
      nsplit = pl.nsplit;
    } else {
      if (E2 <= 16) {
        dim3 grid((N + 255) / 256, 1);
        if (x_dt == MOE_BF16)
          router_gemm_kernel<256, 16, true><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
        else
          router_gemm_kernel<256, 16, false><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
      } else {
        dim3 grid((N + 63) / 64, (E2 + 63) / 64);
        if (x_dt == MOE_BF16)
          router_gemm_kernel<64, 64, true><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
        else
          router_gemm_kernel<64, 64, false><<<grid, kThreads, 0, st>>>(x, w_gate, p->w_noise, raw, N, d, E, E2);
      }
      moe_status s = launch_status("router_gemm");
      if (s != MOE_OK) return s;
      stride = E2;
    }
    src = raw;
  }
  SelectArgs a;
  a.N = N;
  a.E = E;
  a.k = p->top_k;
  a.C = p->n_cand;
  a.renorm = p->renormalize;
  a.src = src;
  a.stride = stride;
  a.nsplit = nsplit;
  a.split_stride = (long long)N * stride;
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
  if (E <= 64)
    router_select_kernel<1><<<nblk, kThreads, 0, st>>>(a);
  else if (E <= 128)
    router_select_kernel<2><<<nblk, kThreads, 0, st>>>(a);
  else
    router_select_kernel<4><<<nblk, kThreads, 0, st>>>(a);
  moe_status s = launch_status("router_select");
  if (s != MOE_OK) return s;
  if (score_sums) {
    router_sum_partials_kernel<<<E + 1, kThreads, 0, st>>>(partials, nblk, E + 1, score_sums);
    s = launch_status("router_sum_partials");
  }
  return s;
}

}  // namespace moe_host
