// balance_stats.hip -- load-balance statistics and the loss-free bias step.
//
// heavensheep.xyz MoE notes, "Training": Switch aux loss from f_i (fraction
// of tokens sent to expert i) and P_i (router probability of i), minimal when
// every expert gets the same share; DeepSeek V3 per-expert bias adjusted
// online by usage (also "MoE" on ld246.com, Q3 item 2: over-used -> bias
// down, idle -> bias up). chiang97912 MoE notes, "辅助损失": Importance =
// sum of G(x) over the batch, CV = sigma / mu, L = w CV^2. "[CS336-04]",
// section 4, names the router z-loss.
#include "moe_device.h"

namespace {

constexpr int kThreads = 256;

__device__ double block_sum(double v, double* buf) {
  buf[threadIdx.x] = v;
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) buf[threadIdx.x] += buf[threadIdx.x + s];
    __syncthreads();
  }
  const double r = buf[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void balance_stats_kernel(
    int N, int E, int k, const int32_t* __restrict__ routed, const int32_t* __restrict__ kept,
    const double* __restrict__ sums, float* __restrict__ f, float* __restrict__ P,
    float* __restrict__ scalars, float* __restrict__ bias, float rate) {
  __shared__ double buf[kThreads];
  const int e = threadIdx.x;
  const double nk = (double)N * (double)k;
  double fe = 0.0, Ie = 0.0, ke = 0.0;
  if (e < E) {
    fe = (double)routed[e] / nk;
    Ie = sums[e];
    ke = (double)kept[e];
    f[e] = (float)fe;
    P[e] = (float)(Ie / (double)N);
  }
  const double aux = block_sum(fe * (Ie / (double)N), buf);
  const double mean = block_sum(Ie, buf) / (double)E;
  const double dev = e < E ? (Ie - mean) : 0.0;
  const double var = block_sum(dev * dev, buf) / (double)E;
  const double sum_kept = block_sum(ke, buf);
  if (e == 0) {
    scalars[0] = (float)((double)E * aux);
    scalars[1] = (float)(var / (mean * mean));
    scalars[2] = (float)(sums[E] / (double)N);
    scalars[3] = (float)((nk - sum_kept) / nk);
  }
  if (bias && e < E) {
    const long long load = (long long)routed[e] * E, target = (long long)N * k;
    if (load > target) bias[e] = bias[e] - rate;
    else if (load < target) bias[e] = bias[e] + rate;
  }
}

}  // namespace

namespace moe_host {

moe_status balance_stats_launch(int N, int E, int k, const int32_t* routed, const int32_t* kept,
                                const double* sums, float* f, float* P, float* scalars,
                                float* bias, float rate, hipStream_t st) {
  balance_stats_kernel<<<1, kThreads, 0, st>>>(N, E, k, routed, kept, sums, f, P, scalars, bias,
                                               rate);
  return launch_status("balance stats");
}

}  // namespace moe_host
