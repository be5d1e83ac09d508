// combine.hip -- gate-weighted combine back to token order (gfx950).
//
// mkbk-pku.cn, "通信与并行": expert outputs go back to each token's original
// position, weighted by the router's alpha; chiang97912 MoE notes, "专家选择":
// y = sum_i G(x)_i E_i(x). The shared always-on expert ("MoE" on ld246.com,
// Q4) adds its output with gate 1. A dropped assignment adds nothing
// (mkbk-pku.cn "负载均衡": the overflowed token's output is zero).
#include "moe_device.h"

namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  __device__ static void load(const float* p, float v[8]) {
    const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ static void store(float* p, const float v[8]) {
    *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]};
    *(f32x4_t*)(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<uint16_t> {
  __device__ static void load(const uint16_t* p, float v[8]) {
    const u32x4_t a = *(const u32x4_t*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float v[8]) {
    u32x4_t a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = moe::pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *(u32x4_t*)p = a;
  }
};

// One block per token and column slice (blockIdx.y of gridDim.y: a few
// tokens, as in decode, still fill the chip); each thread owns 8 consecutive
// features per pass (k <= 8: the token's rows and gates sit in registers).
template <typename YT, typename ST, typename OT>
__global__ __launch_bounds__(kThreads) void combine_kernel(int d, int k,
                                                           const YT* __restrict__ y_rows,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ gates,
                                                           const ST* __restrict__ ysh,
                                                           OT* __restrict__ y) {
  const int t = blockIdx.x;
  int rows[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? row_of[(size_t)t * k + j] : -1;
    g[j] = j < k ? gates[(size_t)t * k + j] : 0.f;
  }
  // the grid covers d in one pass (gridDim.y * kThreads * 8 >= d): one
  // 8-feature chunk a thread
  const int c = (blockIdx.y * kThreads + threadIdx.x) * 8;
  if (c < d) {
    // every kept row's chunk is requested before the first product (eight
    // loads in flight a thread instead of one row at a time), then summed in
    // slot order
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (rows[j] >= 0) Vec8<YT>::load(y_rows + (size_t)rows[j] * d + c, v[j]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(g[j], v[j][i], acc[i]);
    }
    if (ysh) {
      float v[8];
      Vec8<ST>::load(ysh + (size_t)t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<OT>::store(y + (size_t)t * d + c, acc);
  }
}

// Wide form for k > 8 (expert-choice routing makes k = n_experts): the block
// first packs the token's kept (row, gate) pairs into LDS in slot order, so
// each feature chunk loops over kept rows only, with the same fma order as
// combine_kernel.
template <typename YT, typename ST, typename OT>
__global__ __launch_bounds__(kThreads) void combine_wide_kernel(int d, int k,
                                                                const YT* __restrict__ y_rows,
                                                                const int32_t* __restrict__ row_of,
                                                                const float* __restrict__ gates,
                                                                const ST* __restrict__ ysh,
                                                                OT* __restrict__ y) {
  __shared__ int s_row[kThreads];
  __shared__ float s_g[kThreads];
  __shared__ int s_wave[kThreads / 64];
  const int t = blockIdx.x, j = threadIdx.x, wave = j >> 6;
  const int r = j < k ? row_of[(size_t)t * k + j] : -1;
  const float gj = j < k ? gates[(size_t)t * k + j] : 0.f;
  const uint64_t kept = __ballot(r >= 0);
  if ((j & 63) == 0) s_wave[wave] = __popcll(kept);
  __syncthreads();
  int base = 0, n = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    base += w < wave ? s_wave[w] : 0;
    n += s_wave[w];
  }
  if (r >= 0) {
    const int pos = base + __popcll(kept & moe::lanemask_lt());
    s_row[pos] = r;
    s_g[pos] = gj;
  }
  __syncthreads();
  for (int c = (blockIdx.y * kThreads + threadIdx.x) * 8; c < d; c += gridDim.y * kThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < n; ++q) {
      float v[8];
      Vec8<YT>::load(y_rows + (size_t)s_row[q] * d + c, v);
      const float g = s_g[q];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(g, v[i], acc[i]);
    }
    if (ysh) {
      float v[8];
      Vec8<ST>::load(ysh + (size_t)t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<OT>::store(y + (size_t)t * d + c, acc);
  }
}

template <typename YT, typename ST, typename OT>
void launch_combine(int N, int d, int k, const void* yr, const int32_t* row_of,
                    const float* gates, const void* ysh, void* y, hipStream_t st) {
  // one column slice per 2048 features: each thread combines one 8-feature
  // chunk of one token (more blocks in flight than looping over the slices:
  // DeepSeek-shaped combine 0.448 -> 0.431 ms, Mixtral 0.037 -> 0.035 ms),
  // and a few tokens (decode) still fill the chip
  const int slices = (d + kThreads * 8 - 1) / (kThreads * 8);
  const dim3 grid(N, slices);
  if (k <= 8)
    combine_kernel<YT, ST, OT><<<grid, kThreads, 0, st>>>(d, k, (const YT*)yr, row_of, gates,
                                                          (const ST*)ysh, (OT*)y);
  else
    combine_wide_kernel<YT, ST, OT><<<grid, kThreads, 0, st>>>(d, k, (const YT*)yr, row_of,
                                                               gates, (const ST*)ysh, (OT*)y);
}

template <typename YT, typename ST>
moe_status dispatch_out(int N, int d, int k, const void* yr, const int32_t* row_of,
                        const float* gates, const void* ysh, void* y, moe_dtype out_dt,
                        hipStream_t st) {
  if (out_dt == MOE_BF16)
    launch_combine<YT, ST, uint16_t>(N, d, k, yr, row_of, gates, ysh, y, st);
  else
    launch_combine<YT, ST, float>(N, d, k, yr, row_of, gates, ysh, y, st);
  return moe_host::launch_status("combine");
}

// Backward of the combine, one block per token. y_t = sum_j g_tj o_tj:
// dO_r = g_tj * dy_t (bf16, the data operand of the experts' backward GEMMs)
// for the row r = row_of[t][j] of each kept slot, and dg_tj = <dy_t, o_r>
// (fp32, summed per thread in feature order, then over the block's threads
// in a fixed tree: deterministic). A dropped slot gets dg = 0. With a shared
// expert (gate 1) its output gradient is dy itself, written as bf16 rows.
template <typename YT>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    int d, int k, const float* __restrict__ dy, const YT* __restrict__ y_rows,
    const int32_t* __restrict__ row_of, const float* __restrict__ gates,
    uint16_t* __restrict__ d_rows, float* __restrict__ dgates, uint16_t* __restrict__ d_shared) {
  __shared__ float red[kThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (d_shared)
    for (int c = tid * 8; c < d; c += kThreads * 8) {
      float v[8];
      Vec8<float>::load(dy + (size_t)t * d + c, v);
      Vec8<uint16_t>::store(d_shared + (size_t)t * d + c, v);
    }
  for (int j = 0; j < k; ++j) {
    const int r = row_of[(size_t)t * k + j];
    if (r < 0) {
      if (tid == 0) dgates[(size_t)t * k + j] = 0.f;
      continue;
    }
    const float g = gates[(size_t)t * k + j];
    float dot = 0.f;
    for (int c = tid * 8; c < d; c += kThreads * 8) {
      float v[8], o[8];
      Vec8<float>::load(dy + (size_t)t * d + c, v);
      Vec8<YT>::load(y_rows + (size_t)r * d + c, o);
      float s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot = __builtin_fmaf(v[i], o[i], dot);
        s[i] = g * v[i];
      }
      Vec8<uint16_t>::store(d_rows + (size_t)r * d + c, s);
    }
    dot = moe::wave_tree_sum(dot);
    if ((tid & 63) == 0) red[tid >> 6] = dot;
    __syncthreads();
    if (tid == 0) {
      float sum = 0.f;
      for (int w = 0; w < kThreads / 64; ++w) sum += red[w];
      dgates[(size_t)t * k + j] = sum;
    }
    __syncthreads();
  }
}

}  // namespace

namespace moe_host {

moe_status combine_backward_launch(int N, int d, int k, const float* dy, const void* y_rows,
                                   moe_dtype y_dt, const int32_t* row_of, const float* gates,
                                   uint16_t* d_rows, float* dgates, uint16_t* d_shared,
                                   hipStream_t st) {
  if (y_dt == MOE_BF16)
    combine_backward_kernel<uint16_t><<<N, kThreads, 0, st>>>(
        d, k, dy, (const uint16_t*)y_rows, row_of, gates, d_rows, dgates, d_shared);
  else
    combine_backward_kernel<float><<<N, kThreads, 0, st>>>(
        d, k, dy, (const float*)y_rows, row_of, gates, d_rows, dgates, d_shared);
  return launch_status("combine backward");
}


// Top-1 combine done in the expert GEMM's epilogue, the part before it:
// rows of tokens whose one assignment was dropped get zero output (the
// residual is the caller's), and each kept token's gate goes to its packed
// row (gate_row), where the epilogue that writes the token's row reads it.
__global__ __launch_bounds__(kThreads) void combine_dropped_kernel(int d,
                                                                   const int32_t* __restrict__ row_of,
                                                                   const float* __restrict__ gates,
                                                                   float* __restrict__ gate_row,
                                                                   float* __restrict__ y) {
  const int t = blockIdx.x;
  const int r = row_of[t];
  if (r >= 0) {
    if (blockIdx.y == 0 && threadIdx.x == 0) gate_row[r] = gates[t];
    return;
  }
  for (int c = (blockIdx.y * kThreads + threadIdx.x) * 4; c < d; c += gridDim.y * kThreads * 4)
    *(f32x4_t*)(y + (size_t)t * d + c) = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

moe_status combine_dropped_launch(int N, int d, const int32_t* row_of, const float* gates,
                                  float* gate_row, float* y, hipStream_t st) {
  const int per = kThreads * 4;
  int slices = (d + per - 1) / per;
  slices = slices < 1 ? 1 : (slices > 8 ? 8 : slices);
  combine_dropped_kernel<<<dim3(N, slices), kThreads, 0, st>>>(d, row_of, gates, gate_row, y);
  return launch_status("combine (dropped tokens)");
}

moe_status combine_launch(int N, int d, int k, const void* y_rows, moe_dtype y_dt,
                          const int32_t* row_of, const float* gates, const void* y_shared,
                          moe_dtype sh_dt, void* y, moe_dtype out_dt, hipStream_t st) {
  const bool ybf = y_dt == MOE_BF16, sbf = sh_dt == MOE_BF16;
  if (ybf && sbf) return dispatch_out<uint16_t, uint16_t>(N, d, k, y_rows, row_of, gates, y_shared, y, out_dt, st);
  if (ybf) return dispatch_out<uint16_t, float>(N, d, k, y_rows, row_of, gates, y_shared, y, out_dt, st);
  if (sbf) return dispatch_out<float, uint16_t>(N, d, k, y_rows, row_of, gates, y_shared, y, out_dt, st);
  return dispatch_out<float, float>(N, d, k, y_rows, row_of, gates, y_shared, y, out_dt, st);
}

}  // namespace moe_host
