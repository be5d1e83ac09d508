// expert_choice.hip -- expert-choice routing on gfx950: every expert takes
// its top-capacity tokens by router score.
//
// heavensheep.xyz MoE notes, "Routing Function": besides tokens choosing
// experts, experts can choose tokens, which balances the load; "[CS336-04]
// Mixture of Experts", section 3: the routing can be reversed so that
// experts select tokens. Expert e takes the cap tokens with the largest
// s_te (ties to the lower token index) and lists them in token order.
//
// One workgroup per expert. The cap-th largest 64-bit key
// (orderable(s_te) << 32 | ~t: unique, larger = preferred) is found by an
// 8-pass most-significant-digit radix select over the expert's column of
// scores; a token is chosen iff its key is at least that key. A workgroup
// scan over contiguous runs of tokens then gives every chosen token its row
// in token order.
#include "moe_device.h"

namespace {

constexpr int kEcThreads = 1024;

__device__ __forceinline__ uint64_t ec_key(const float* __restrict__ scores, int E, int e, int t) {
  float v = scores[(size_t)t * E + e];
  if (v == 0.0f) v = 0.0f;  // -0 counts as +0
  return ((uint64_t)moe::orderable(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)t);
}

__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(
    int N, int E, int cap, const float* __restrict__ scores, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ row_of, float* __restrict__ gates,
    int32_t* __restrict__ counts) {
  __shared__ int hist[256];
  __shared__ int sums[kEcThreads];
  __shared__ uint64_t s_prefix;
  __shared__ int s_rank, s_done;
  const int e = blockIdx.x, tid = threadIdx.x;

  // radix select: after pass p the top 8(p+1) bits of the cap-th largest key
  // are known; `rank` is its rank among the keys sharing those bits
  uint64_t prefix = 0;
  int rank = cap;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t known = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int i = tid; i < 256; i += kEcThreads) hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < N; t += kEcThreads) {
      const uint64_t k = ec_key(scores, E, e, t);
      if ((k & known) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);  // counts: order-free
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, dgt = 255;
      for (; dgt > 0; --dgt) {
        if (above + hist[dgt] >= rank) break;
        above += hist[dgt];
      }
      s_prefix = prefix | ((uint64_t)dgt << shift);
      s_rank = rank - above;
      // every key in the chosen bucket is taken: the bucket's floor is the
      // threshold and the lower digits need no further pass
      s_done = hist[dgt] == rank - above;
    }
    __syncthreads();
    prefix = s_prefix;
    rank = s_rank;
    const bool done = s_done;
    __syncthreads();
    if (done) break;
  }
  // keys are unique: exactly cap keys are >= kth
  const uint64_t kth = prefix;

  // rows in token order: thread i owns tokens [t0, t1)
  const int chunk = (N + kEcThreads - 1) / kEcThreads;
  const int t0 = min(N, tid * chunk), t1 = min(N, t0 + chunk);
  int mine = 0;
  for (int t = t0; t < t1; ++t) mine += ec_key(scores, E, e, t) >= kth;
  sums[tid] = mine;
  __syncthreads();
  for (int o = 1; o < kEcThreads; o <<= 1) {
    const int v = tid >= o ? sums[tid - o] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  int row = e * cap + sums[tid] - mine;
  for (int t = t0; t < t1; ++t) {
    const size_t te = (size_t)t * E + e;
    if (ec_key(scores, E, e, t) >= kth) {
      perm_token[row] = t;
      row_of[te] = row;
      gates[te] = scores[te];
      ++row;
    } else {
      row_of[te] = -1;
      gates[te] = 0.f;
    }
  }
  if (tid == 0) {
    offsets[e] = e * cap;
    if (e == E - 1) offsets[E] = E * cap;
    if (counts) counts[e] = cap;
  }
}

}  // namespace

namespace moe_host {

moe_status expert_choice_launch(int N, int E, int capacity, const float* scores,
                                int32_t* offsets, int32_t* perm_token, int32_t* row_of,
                                float* gates, int32_t* counts, hipStream_t st) {
  const int cap = capacity < N ? capacity : N;
  ec_select_kernel<<<E, kEcThreads, 0, st>>>(N, E, cap, scores, offsets, perm_token, row_of,
                                            gates, counts);
  return launch_status("expert choice");
}

}  // namespace moe_host
