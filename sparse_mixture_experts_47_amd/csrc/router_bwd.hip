// router_bwd.hip -- backward pass of the router on gfx950: gates -> scores
// -> logits (with the auxiliary and z-loss terms) -> W_g, the logit bias and
// the token rows, plus the sum of the experts' row gradients back to tokens.
//
// heavensheep.xyz MoE notes, "Training": the main loss reaches only the
// selected experts' scores (top-k passes no gradient to the rest), and the
// Switch auxiliary loss E * sum_i f_i P_i is what gives every expert's
// router weights a gradient; CS336 notes section 4: the z-loss
// (1/N) sum_t lse_t^2. chiang97912 MoE notes, "KeepTopK 策略": the gates
// are the softmax renormalised over the kept k (G = Softmax(KeepTopK(H,k))).
// Per token t (s = softmax(l), lse = log sum exp l):
//   renormalised: g_j = s_{c_j} / S, S = sum_j s_{c_j}:
//                 dL/ds_{c_j} = (dg_j - sum_i dg_i g_i) / S
//   Switch:       g = s_e of the expert used: dL/ds_e = dg
//   auxiliary:    dL/ds_te += alpha E f_e / N, f_e = routed_e / (N k)
//   softmax:      dl_te = s_te (ds_te - sum_e' s_te' ds_te')
//   z-loss:       dl_te += beta 2 lse_t s_te / N
//   noise (chiang97912 "KeepTopK 策略": H = x W_g + z softplus(x W_noise)):
//                 dv_te = dl_te z_te sigmoid(v_te) (1 where softplus is v, v > 20),
//                 dW_noise = dv^T x,  dx_t += dv_t W_noise
//   router GEMM:  dW_g = dl^T x,  d(logit bias) = sum_t dl_t,  dx_t += dl_t W_g
// dx_t also sums the token's kept expert-row gradients in slot order and the
// shared expert's token-row gradient.
#include "moe_device.h"

namespace {

constexpr int kThreads = 256;

// one wave per token
__global__ __launch_bounds__(kThreads) void router_bwd_token_kernel(
    int N, int E, int k, int C, int renormalize, const float* __restrict__ logits,
    const int32_t* __restrict__ cand_ids, const int32_t* __restrict__ expert_of,
    const int32_t* __restrict__ row_of, const float* __restrict__ dgates,
    const int32_t* __restrict__ counts_routed, float alpha, float beta,
    float* __restrict__ dlogits, const float* __restrict__ noise_v, uint64_t seed,
    float* __restrict__ dv) {
  __shared__ float s_sh[kThreads / 64][256];
  __shared__ float ds_sh[kThreads / 64][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + wave;
  if (t >= N) return;  // whole waves leave together; no block barrier below
  float* S_ = s_sh[wave];
  float* D_ = ds_sh[wave];
  const float* l = logits + (size_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
  m = moe::wave_max(m);
  float part = 0.f;
  for (int e = lane; e < E; e += 64) {
    const float u = __expf(l[e] - m);
    S_[e] = u;
    part += u;
  }
  const float S = moe::wave_tree_sum(part);
  const float lse = m + __logf(S);
  const float invNk = 1.f / ((float)N * (float)k);
  for (int e = lane; e < E; e += 64) {
    S_[e] = S_[e] / S;
    D_[e] = alpha * (float)E * ((float)counts_routed[e] * invNk) / (float)N;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane == 0) {
    const float* dg = dgates + (size_t)t * k;
    if (renormalize) {
      const int32_t* c = cand_ids + (size_t)t * C;
      float Ssel = 0.f;
      for (int j = 0; j < k; ++j) Ssel += S_[c[j]];
      float dot = 0.f;
      for (int j = 0; j < k; ++j) dot += dg[j] * (S_[c[j]] / Ssel);
      for (int j = 0; j < k; ++j) D_[c[j]] += (dg[j] - dot) / Ssel;
    } else {
      for (int j = 0; j < k; ++j) {
        const int e = expert_of[(size_t)t * k + j];
        if (row_of[(size_t)t * k + j] >= 0 && e >= 0) D_[e] += dg[j];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float sd = 0.f;
  for (int e = lane; e < E; e += 64) sd += S_[e] * D_[e];
  sd = moe::wave_tree_sum(sd);
  const float zc = beta * 2.f * lse / (float)N;
  for (int e = lane; e < E; e += 64) {
    const float s = S_[e];
    const float g = s * (D_[e] - sd) + zc * s;
    dlogits[(size_t)t * E + e] = g;
    if (noise_v) {
      const float v = noise_v[(size_t)t * E + e];
      const float z = moe::noise_normal(seed, (uint32_t)t, (uint32_t)e, (uint32_t)E);
      const float sig = v > 20.f ? 1.f : 1.f / (1.f + __expf(-v));
      dv[(size_t)t * E + e] = g * z * sig;
    }
  }
}

// Four consecutive fp32 values of a row at column col (masked past d; as
// one 16-byte access when rows are 16-byte aligned, i.e. d % 4 == 0).
__device__ __forceinline__ f32x4_t load4(const float* __restrict__ row, int col, int d,
                                         bool vec) {
  if (vec && col + 3 < d) return *(const f32x4_t*)(row + col);
  f32x4_t v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = col + q < d ? row[col + q] : 0.f;
  return v;
}

// dx_t = sum_j dx_rows[row_of[t][j]] (kept slots in order) + dx_shared[t]
//        + sum_e dl_te W_g[e] (e ascending) + sum_e dv_te W_noise[e] (with
//        noise). A block takes kDxT tokens x kDxC columns; each thread holds
//        4 tokens x 16 columns (4 groups of 4 consecutive columns, 64 apart),
//        and the product runs over LDS chunks of kDxE experts: the chunk's
//        gradient columns (transposed, [e][token]) and weight rows
//        ([e][column]), 64 FMAs per 5 LDS reads. (Loading the next chunk into
//        registers during the products needs 200 VGPRs, and the halved
//        occupancy slows the row gather more than the overlap gains.)
constexpr int kDxT = 64, kDxC = 256, kDxE = 32;
__global__ __launch_bounds__(kThreads) void router_bwd_dx_kernel(
    int N, int d, int E, int k, const float* __restrict__ dl, const float* __restrict__ w_gate,
    const int32_t* __restrict__ row_of, const float* __restrict__ dx_rows,
    const float* __restrict__ dx_shared, const float* __restrict__ dv,
    const float* __restrict__ w_noise, float* __restrict__ dx) {
  __shared__ __align__(16) float gs[kDxE][kDxT];
  __shared__ __align__(16) float ws[kDxE][kDxC];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int t0 = blockIdx.x * kDxT, c0 = blockIdx.y * kDxC;
  const bool vec = (d & 3) == 0;
  f32x4_t acc[4][4];  // [token i][column group j]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = c0 + 64 * j + tx * 4;
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
      if (t < N && col < d) {
        if (dx_rows)
          for (int s = 0; s < k; ++s) {
            const int r = row_of[(size_t)t * k + s];
            if (r >= 0) a += load4(dx_rows + (size_t)r * d, col, d, vec);
          }
        if (dx_shared) a += load4(dx_shared + (size_t)t * d, col, d, vec);
      }
      acc[i][j] = a;
    }
  }
  for (int pass = 0; pass < (dv ? 2 : 1); ++pass) {
    const float* G = pass == 0 ? dl : dv;
    const float* Wm = pass == 0 ? w_gate : w_noise;
    for (int e0 = 0; e0 < E; e0 += kDxE) {
      __syncthreads();  // the previous chunk is consumed
      for (int i = tid; i < kDxE * kDxT; i += kThreads) {
        const int tt = i / kDxE, ee = i - tt * kDxE;
        const int t = t0 + tt, e = e0 + ee;
        gs[ee][tt] = (t < N && e < E) ? G[(size_t)t * E + e] : 0.f;
      }
      for (int i = tid; i < kDxE * (kDxC / 4); i += kThreads) {
        const int ee = i / (kDxC / 4), c4 = i - ee * (kDxC / 4);
        const int e = e0 + ee;
        *(f32x4_t*)&ws[ee][c4 * 4] =
            e < E ? load4(Wm + (size_t)e * d, c0 + c4 * 4, d, vec) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      __syncthreads();
      const int ne = min(kDxE, E - e0);
#pragma unroll 4
      for (int ee = 0; ee < ne; ++ee) {
        const f32x4_t g = *(const f32x4_t*)&gs[ee][ty * 4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t w = *(const f32x4_t*)&ws[ee][64 * j + tx * 4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(g[i], w[q], acc[i][j][q]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = c0 + 64 * j + tx * 4;
      float* out = dx + (size_t)t * d;
      if (vec && col + 3 < d) {
        *(f32x4_t*)(out + col) = acc[i][j];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (col + q < d) out[col + q] = acc[i][j][q];
      }
    }
  }
}

// Tokens per partial sum of a weight gradient: 256, halved (down to 128)
// while the grid would have fewer than 2048 blocks.
int wg_chunk_tokens(int N, int d, int E) {
  const long long base = (long long)((d + 255) / 256) * ((E + 31) / 32);
  int ch = 256;
  while (ch > 128 && base * ((N + ch - 1) / ch) < 2048) ch >>= 1;
  return ch;
}

// partial[chunk][e][c] = sum over the chunk's tokens (ascending) of
// g[t][e] x[t][c]. A block takes 32 experts x 256 columns of one chunk; each
// thread holds 4 experts x 8 columns (2 groups of 4, 128 apart). Tokens go
// through LDS 32 at a time (g as [t][e], x converted to fp32 as [t][c]),
// each group loaded into registers while the previous one is multiplied.
constexpr int kWgE = 32, kWgC = 256, kWgT = 32;
template <typename XT>
__global__ __launch_bounds__(kThreads) void router_bwd_wg_partial_kernel(
    int N, int d, int E, int chunk_tokens, const float* __restrict__ gsrc,
    const XT* __restrict__ x, float* __restrict__ partial) {
  __shared__ __align__(16) float gs[kWgT][kWgE];
  __shared__ __align__(16) float xs[kWgT][kWgC];
  const int tid = threadIdx.x, eg = tid >> 5, cg = tid & 31;
  const int c0 = blockIdx.x * kWgC, e0 = blockIdx.y * kWgE, chunk = blockIdx.z;
  const int t0 = chunk * chunk_tokens, t1 = min(N, t0 + chunk_tokens);
  // staging: 4 gradient values and 8 groups of 4 consecutive x values a thread
  constexpr int GPT = kWgT * kWgE / kThreads, XPT = kWgT * (kWgC / 4) / kThreads;
  const bool vec = (d & 3) == 0;
  float gr[GPT];
  f32x4_t xr[XPT];
  auto fetch = [&](int ts) {
    const int nt = min(kWgT, t1 - ts);
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int i = tid + u * kThreads, tt = i / kWgE, ee = i - tt * kWgE;
      const int e = e0 + ee;
      gr[u] = (tt < nt && e < E) ? gsrc[(size_t)(ts + tt) * E + e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int i = tid + u * kThreads, tt = i / (kWgC / 4), c4 = i - tt * (kWgC / 4);
      const int c = c0 + c4 * 4;
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (tt < nt) {
        const XT* row = x + (size_t)(ts + tt) * d;
        if constexpr (sizeof(XT) == 2) {
          if (vec && c + 3 < d) {
            const u32x2_t b = *(const u32x2_t*)(row + c);
            v = f32x4_t{moe::bf16_bits_to_f32((uint16_t)b[0]),
                        moe::bf16_bits_to_f32((uint16_t)(b[0] >> 16)),
                        moe::bf16_bits_to_f32((uint16_t)b[1]),
                        moe::bf16_bits_to_f32((uint16_t)(b[1] >> 16))};
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (c + q < d) v[q] = moe::bf16_bits_to_f32(row[c + q]);
          }
        } else {
          v = load4(row, c, d, vec);
        }
      }
      xr[u] = v;
    }
  };
  f32x4_t acc[4][2];  // [expert i][column group h]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[i][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (t0 < t1) fetch(t0);
  for (int ts = t0; ts < t1; ts += kWgT) {
    const int nt = min(kWgT, t1 - ts);
    __syncthreads();  // the previous tokens are consumed
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int i = tid + u * kThreads, tt = i / kWgE, ee = i - tt * kWgE;
      gs[tt][ee] = gr[u];
    }
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int i = tid + u * kThreads, tt = i / (kWgC / 4), c4 = i - tt * (kWgC / 4);
      *(f32x4_t*)&xs[tt][c4 * 4] = xr[u];
    }
    __syncthreads();
    if (ts + kWgT < t1) fetch(ts + kWgT);
    for (int tt = 0; tt < nt; ++tt) {
      const f32x4_t g = *(const f32x4_t*)&gs[tt][eg * 4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t xv = *(const f32x4_t*)&xs[tt][128 * h + cg * 4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][h][q] = __builtin_fmaf(g[i], xv[q], acc[i][h][q]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + eg * 4 + i;
    if (e >= E) continue;
    float* out = partial + ((size_t)chunk * E + e) * d;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + 128 * h + cg * 4;
      if (vec && c + 3 < d) {
        *(f32x4_t*)(out + c) = acc[i][h];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c + q < d) out[c + q] = acc[i][h][q];
      }
    }
  }
}

// dW_g[e][c] = sum of the partials in chunk order
__global__ __launch_bounds__(kThreads) void router_bwd_wg_reduce_kernel(
    int d, int E, int chunks, const float* __restrict__ partial, float* __restrict__ dw) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)E * d) return;
  float acc = 0.f;
#pragma unroll 8
  for (int ch = 0; ch < chunks; ++ch) acc += partial[(size_t)ch * E * d + i];
  dw[i] = acc;
}

// d(logit bias)[e] = sum_t dl[t][e]: one block per expert, fixed tree
__global__ __launch_bounds__(kThreads) void router_bwd_bias_kernel(int N, int E,
                                                                   const float* __restrict__ dl,
                                                                   float* __restrict__ db) {
  __shared__ float red[kThreads / 64];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int t = threadIdx.x; t < N; t += kThreads) acc += dl[(size_t)t * E + e];
  acc = moe::wave_tree_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) s += red[w];
    db[e] = s;
  }
}

}  // namespace

namespace moe_host {

// workspace: dW partials [chunks][E][d] | dv [N][E]
size_t router_backward_workspace_bytes(int N, int d, int E) {
  const int ch = wg_chunk_tokens(N, d, E);
  const int chunks = (N + ch - 1) / ch;
  return align256((size_t)chunks * E * d * 4) + align256((size_t)N * E * 4);
}

moe_status router_backward_launch(int N, int d, int E, int k, int C, int renormalize,
                                  const void* x, moe_dtype x_dt, const float* w_gate,
                                  const float* logits, const int32_t* cand_ids,
                                  const int32_t* expert_of, const int32_t* row_of,
                                  const float* dgates, const int32_t* counts_routed, float alpha,
                                  float beta, const float* dx_rows, const float* dx_shared,
                                  const float* w_noise, const float* noise_v, uint64_t seed,
                                  float* dlogits, float* dw_gate, float* dlogit_bias,
                                  float* dw_noise, float* dx, void* workspace, hipStream_t st) {
  const int ch = wg_chunk_tokens(N, d, E);
  const int chunks = (N + ch - 1) / ch;
  float* partial = (float*)workspace;
  float* dv = w_noise ? (float*)((char*)workspace + align256((size_t)chunks * E * d * 4)) : nullptr;
  const int per_block = kThreads / 64;
  router_bwd_token_kernel<<<(N + per_block - 1) / per_block, kThreads, 0, st>>>(
      N, E, k, C, renormalize, logits, cand_ids, expert_of, row_of, dgates, counts_routed, alpha,
      beta, dlogits, w_noise ? noise_v : nullptr, seed, dv);
  moe_status s = launch_status("router backward (scores)");
  if (s != MOE_OK) return s;
  dim3 gdx((N + kDxT - 1) / kDxT, (d + kDxC - 1) / kDxC);
  router_bwd_dx_kernel<<<gdx, kThreads, 0, st>>>(N, d, E, k, dlogits, w_gate, row_of, dx_rows,
                                                 dx_shared, dv, w_noise, dx);
  s = launch_status("router backward (dx)");
  if (s != MOE_OK) return s;
  // dW = g^T x for g = dl (-> dW_g) and, with noise, g = dv (-> dW_noise)
  for (int pass = 0; pass < (w_noise ? 2 : 1); ++pass) {
    const float* gsrc = pass == 0 ? dlogits : dv;
    float* out = pass == 0 ? dw_gate : dw_noise;
    dim3 grid((d + kWgC - 1) / kWgC, (E + kWgE - 1) / kWgE, chunks);
    if (x_dt == MOE_BF16)
      router_bwd_wg_partial_kernel<uint16_t><<<grid, kThreads, 0, st>>>(
          N, d, E, ch, gsrc, (const uint16_t*)x, partial);
    else
      router_bwd_wg_partial_kernel<float><<<grid, kThreads, 0, st>>>(
          N, d, E, ch, gsrc, (const float*)x, partial);
    s = launch_status("router backward (weight gradient partials)");
    if (s != MOE_OK) return s;
    router_bwd_wg_reduce_kernel<<<(int)(((size_t)E * d + kThreads - 1) / kThreads), kThreads, 0,
                                  st>>>(d, E, chunks, partial, out);
    s = launch_status("router backward (weight gradient)");
    if (s != MOE_OK) return s;
  }
  if (dlogit_bias) {
    router_bwd_bias_kernel<<<E, kThreads, 0, st>>>(N, E, dlogits, dlogit_bias);
    s = launch_status("router backward (logit bias)");
  }
  return s;
}

}  // namespace moe_host
