// expert_choice.hip -- expert-choice routing on gfx950: every expert takes
// its top-capacity tokens by router score.
//
// heavensheep.xyz MoE notes, "Routing Function": besides tokens choosing
// experts, experts can choose tokens, which balances the load; "[CS336-04]
// Mixture of Experts", section 3: the routing can be reversed so that
// experts select tokens. Expert e takes the cap tokens with the largest
// s_te (ties to the lower token index) and lists them in token order.
//
// One workgroup per expert (its column of scores staged in LDS when it
// fits). The cap-th largest 64-bit key
// (orderable(s_te) << 32 | ~t: unique, larger = preferred) is found by an
// 8-pass most-significant-digit radix select over the expert's column of
// scores; a token is chosen iff its key is at least that key. A workgroup
// scan over contiguous runs of tokens then gives every chosen token its row
// in token order.
#include "moe_device.h"

namespace {

constexpr int kEcThreads = 1024;
// columns of up to this many tokens are staged in LDS (4 B each) once; the
// radix passes and the compaction then read LDS instead of L2
constexpr int kEcLdsTokens = 32768;

__device__ __forceinline__ uint32_t ec_score_key(float v) {
  if (v == 0.0f) v = 0.0f;  // -0 counts as +0
  return moe::orderable(v);
}

// key of token t: score bits above, ~t below (unique; larger = preferred)
__device__ __forceinline__ uint64_t ec_key(uint32_t score_key, int t) {
  return ((uint64_t)score_key << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)t);
}

template <bool STAGED>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(
    int N, int E, int cap, const float* __restrict__ scores, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ row_of, float* __restrict__ gates,
    int32_t* __restrict__ counts) {
  extern __shared__ uint32_t s_key[];  // [N] when STAGED
  __shared__ int hist[256];
  __shared__ int sums[kEcThreads];
  __shared__ uint64_t s_prefix;
  __shared__ int s_rank, s_done;
  const int e = blockIdx.x, tid = threadIdx.x;
  if constexpr (STAGED) {
    for (int t = tid; t < N; t += kEcThreads) s_key[t] = ec_score_key(scores[(size_t)t * E + e]);
    __syncthreads();
  }
  auto key = [&](int t) -> uint64_t {
    if constexpr (STAGED) return ec_key(s_key[t], t);
    else return ec_key(ec_score_key(scores[(size_t)t * E + e]), t);
  };

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
      const uint64_t k = key(t);
      if ((k & known) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);  // counts: order-free
    }
    __syncthreads();
    if (tid < 64) {
      // wave 0 picks the digit: lane l holds bins 4l..4l+3; `above` counts
      // the keys in higher bins (a suffix sum across lanes)
      int h[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) tot += h[i] = hist[4 * tid + i];
      int suf = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(suf, o);
        if (tid + o < 64) suf += v;
      }
      int above = suf - tot;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < rank && above + h[i] >= rank) {  // one bin in the wave
          s_prefix = prefix | ((uint64_t)(4 * tid + i) << shift);
          s_rank = rank - above;
          // every key in the chosen bin is taken: the bin's floor is the
          // threshold and the lower digits need no further pass
          s_done = h[i] == rank - above;
        }
        above += h[i];
      }
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
  for (int t = t0; t < t1; ++t) mine += key(t) >= kth;
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
    if (key(t) >= kth) {
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
  if (N <= kEcLdsTokens) {
    static bool configured = false;  // LDS beyond the default per-launch limit
    if (!configured) {
      if (hipFuncSetAttribute((const void*)ec_select_kernel<true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              kEcLdsTokens * 4) != hipSuccess)
        return launch_status("expert choice (LDS attribute)");
      configured = true;
    }
    ec_select_kernel<true><<<E, kEcThreads, (size_t)N * 4, st>>>(N, E, cap, scores, offsets,
                                                                 perm_token, row_of, gates,
                                                                 counts);
  } else {
    ec_select_kernel<false><<<E, kEcThreads, 0, st>>>(N, E, cap, scores, offsets, perm_token,
                                                      row_of, gates, counts);
  }
  return launch_status("expert choice");
}

}  // namespace moe_host
