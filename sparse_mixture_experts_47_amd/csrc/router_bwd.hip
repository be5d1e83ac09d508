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
constexpr int kChunkTokens = 256;  // tokens per partial sum of dW_g

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

// dx_t = sum_j dx_rows[row_of[t][j]] (kept slots in order) + dx_shared[t]
//        + sum_e dl_te W_g[e] (e ascending) + sum_e dv_te W_noise[e] (with
//        noise). A block takes kDxTokens tokens x
// 256 columns: their dl rows sit in LDS and every W_g element read serves
// all of the block's tokens.
constexpr int kDxTokens = 16;
__global__ __launch_bounds__(kThreads) void router_bwd_dx_kernel(
    int N, int d, int E, int k, const float* __restrict__ dl, const float* __restrict__ w_gate,
    const int32_t* __restrict__ row_of, const float* __restrict__ dx_rows,
    const float* __restrict__ dx_shared, const float* __restrict__ dv,
    const float* __restrict__ w_noise, float* __restrict__ dx) {
  __shared__ __align__(16) float dls[kDxTokens][256];
  __shared__ __align__(16) float dvs[kDxTokens][256];
  const int t0 = blockIdx.x * kDxTokens, c = blockIdx.y * kThreads + threadIdx.x;
  const int nt = min(kDxTokens, N - t0);
  const int E4 = (E + 3) & ~3;  // dl columns past E are zero
  for (int i = threadIdx.x; i < kDxTokens * E4; i += kThreads) {
    const int tt = i / E4, e = i - tt * E4;
    dls[tt][e] = (tt < nt && e < E) ? dl[(size_t)(t0 + tt) * E + e] : 0.f;
    if (dv) dvs[tt][e] = (tt < nt && e < E) ? dv[(size_t)(t0 + tt) * E + e] : 0.f;
  }
  __syncthreads();
  if (c >= d) return;
  float acc[kDxTokens];
#pragma unroll
  for (int tt = 0; tt < kDxTokens; ++tt) {
    float a = 0.f;
    if (tt < nt) {
      const int t = t0 + tt;
      if (dx_rows)
        for (int j = 0; j < k; ++j) {
          const int r = row_of[(size_t)t * k + j];
          if (r >= 0) a += dx_rows[(size_t)r * d + c];
        }
      if (dx_shared) a += dx_shared[(size_t)t * d + c];
    }
    acc[tt] = a;
  }
  for (int e = 0; e < E4; e += 4) {
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = e + i < E ? w_gate[(size_t)(e + i) * d + c] : 0.f;
#pragma unroll
    for (int tt = 0; tt < kDxTokens; ++tt) {
      const f32x4_t v = *(const f32x4_t*)&dls[tt][e];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[tt] = __builtin_fmaf(v[i], w[i], acc[tt]);
    }
  }
  if (dv)
    for (int e = 0; e < E4; e += 4) {
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = e + i < E ? w_noise[(size_t)(e + i) * d + c] : 0.f;
#pragma unroll
      for (int tt = 0; tt < kDxTokens; ++tt) {
        const f32x4_t v = *(const f32x4_t*)&dvs[tt][e];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tt] = __builtin_fmaf(v[i], w[i], acc[tt]);
      }
    }
#pragma unroll
  for (int tt = 0; tt < kDxTokens; ++tt)
    if (tt < nt) dx[(size_t)(t0 + tt) * d + c] = acc[tt];
}

// partial[chunk][e][c] = sum over the chunk's tokens (ascending) of
// dl[t][e] x[t][c]; a block takes 256 columns x kWgExperts experts, with the
// chunk's dl columns in LDS, so x is read once per expert group
constexpr int kWgExperts = 32;
template <typename XT>
__global__ __launch_bounds__(kThreads) void router_bwd_wg_partial_kernel(
    int N, int d, int E, const float* __restrict__ dl, const XT* __restrict__ x,
    float* __restrict__ partial) {
  __shared__ __align__(16) float dls[kChunkTokens][kWgExperts];
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const int e0 = blockIdx.y * kWgExperts, chunk = blockIdx.z;
  const int t0 = chunk * kChunkTokens, t1 = min(N, t0 + kChunkTokens);
  const int ne = min(kWgExperts, E - e0);
  for (int i = threadIdx.x; i < kChunkTokens * kWgExperts; i += kThreads) {
    const int tt = i / kWgExperts, ei = i - tt * kWgExperts;
    dls[tt][ei] = (t0 + tt < t1 && ei < ne) ? dl[(size_t)(t0 + tt) * E + e0 + ei] : 0.f;
  }
  __syncthreads();
  if (c >= d) return;
  float acc[kWgExperts];
#pragma unroll
  for (int i = 0; i < kWgExperts; ++i) acc[i] = 0.f;
  for (int t = t0; t < t1; ++t) {
    float xv;
    if constexpr (sizeof(XT) == 2) xv = moe::bf16_bits_to_f32(x[(size_t)t * d + c]);
    else xv = x[(size_t)t * d + c];
#pragma unroll
    for (int i = 0; i < kWgExperts; i += 4) {
      const f32x4_t v = *(const f32x4_t*)&dls[t - t0][i];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i + q] = __builtin_fmaf(v[q], xv, acc[i + q]);
    }
  }
  for (int i = 0; i < ne; ++i) partial[((size_t)chunk * E + e0 + i) * d + c] = acc[i];
}

// dW_g[e][c] = sum of the partials in chunk order
__global__ __launch_bounds__(kThreads) void router_bwd_wg_reduce_kernel(
    int d, int E, int chunks, const float* __restrict__ partial, float* __restrict__ dw) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)E * d) return;
  float acc = 0.f;
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
  const int chunks = (N + kChunkTokens - 1) / kChunkTokens;
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
  const int chunks = (N + kChunkTokens - 1) / kChunkTokens;
  float* partial = (float*)workspace;
  float* dv = w_noise ? (float*)((char*)workspace + align256((size_t)chunks * E * d * 4)) : nullptr;
  const int per_block = kThreads / 64;
  router_bwd_token_kernel<<<(N + per_block - 1) / per_block, kThreads, 0, st>>>(
      N, E, k, C, renormalize, logits, cand_ids, expert_of, row_of, dgates, counts_routed, alpha,
      beta, dlogits, w_noise ? noise_v : nullptr, seed, dv);
  moe_status s = launch_status("router backward (scores)");
  if (s != MOE_OK) return s;
  dim3 gdx((N + kDxTokens - 1) / kDxTokens, (d + kThreads - 1) / kThreads);
  router_bwd_dx_kernel<<<gdx, kThreads, 0, st>>>(N, d, E, k, dlogits, w_gate, row_of, dx_rows,
                                                 dx_shared, dv, w_noise, dx);
  s = launch_status("router backward (dx)");
  if (s != MOE_OK) return s;
  // dW = g^T x for g = dl (-> dW_g) and, with noise, g = dv (-> dW_noise)
  for (int pass = 0; pass < (w_noise ? 2 : 1); ++pass) {
    const float* gsrc = pass == 0 ? dlogits : dv;
    float* out = pass == 0 ? dw_gate : dw_noise;
    dim3 grid((d + kThreads - 1) / kThreads, (E + kWgExperts - 1) / kWgExperts, chunks);
    if (x_dt == MOE_BF16)
      router_bwd_wg_partial_kernel<uint16_t><<<grid, kThreads, 0, st>>>(
          N, d, E, gsrc, (const uint16_t*)x, partial);
    else
      router_bwd_wg_partial_kernel<float><<<grid, kThreads, 0, st>>>(N, d, E, gsrc,
                                                                     (const float*)x, partial);
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
