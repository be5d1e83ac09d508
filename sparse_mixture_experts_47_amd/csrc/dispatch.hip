// dispatch.hip -- bucketize by expert, capacity, reroute, pack rows (gfx950).
//
// Tokens are bucketed by their routed expert and each expert's tokens are
// packed contiguously (mkbk-pku.cn, "MOE的优化": bucketize + contiguous
// packing). An expert takes at most `capacity` assignments; beyond that an
// assignment is dropped, or (top-1) its token tries the next candidate once
// (chiang97912 MoE notes, "专家容量"; mkbk-pku.cn "负载均衡", overflow).
//
// Order is a stable counting sort of the assignments taken rank-major
// (every first choice in ascending token order, then every second choice,
// ...): per-block histograms, an ordered scan over blocks, and in-wave ranks
// from ballots over the expert id's bits. No atomic decides any position.
#include <mutex>

#include "moe_device.h"

namespace {

constexpr int kThreads = 256;  // one assignment per thread, 4 waves per block

struct KeyArgs {
  int N, k, C, mode;        // mode 0: a = j*N + t, key = cand[t][j]
  const int32_t* cand;      // mode 1: a = t, key = cand[t][1] if slot1[t] < 0
  const int32_t* slot1;
  int A;                    // number of items
  int E;
};

// An id outside [0, E) is no candidate: its assignment is dropped.
__device__ __forceinline__ int valid_key(int32_t id, int E) {
  return (uint32_t)id < (uint32_t)E ? id : -1;
}

__device__ __forceinline__ int item_key(const KeyArgs& g, int a) {
  if (a >= g.A) return -1;
  if (g.mode == 0) {
    const int j = a / g.N, t = a - j * g.N;
    return valid_key(g.cand[(size_t)t * g.C + j], g.E);
  }
  return g.slot1[a] < 0 ? valid_key(g.cand[(size_t)a * g.C + 1], g.E) : -1;
}

__global__ __launch_bounds__(kThreads) void disp_count_kernel(KeyArgs g, int E,
                                                              int32_t* __restrict__ blockcnt) {
  __shared__ int hist[256];
  hist[threadIdx.x] = 0;
  __syncthreads();
  const int key = item_key(g, blockIdx.x * kThreads + threadIdx.x);
  if (key >= 0) atomicAdd(&hist[key], 1);  // integer counts: order-free
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) blockcnt[(size_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan over blocks for each expert, in block order: one workgroup
// per expert; thread t owns a contiguous run of blocks, the per-thread sums
// are scanned across the workgroup, then each thread writes its run's
// prefixes. Integer sums, so the order of additions does not matter.
__global__ __launch_bounds__(kThreads) void disp_scan_kernel(int nblk, int E,
                                                             const int32_t* __restrict__ blockcnt,
                                                             int32_t* __restrict__ blockbase,
                                                             int32_t* __restrict__ total) {
  __shared__ int sums[kThreads];
  const int e = blockIdx.x, t = threadIdx.x;
  const int chunk = (nblk + kThreads - 1) / kThreads;
  const int b0 = t * chunk, b1 = min(nblk, b0 + chunk);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += blockcnt[(size_t)b * E + e];
  sums[t] = local;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = t >= o ? sums[t - o] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int run = sums[t] - local;  // exclusive prefix of this thread's run
  for (int b = b0; b < b1; ++b) {
    blockbase[(size_t)b * E + e] = run;
    run += blockcnt[(size_t)b * E + e];
  }
  if (t == kThreads - 1) total[e] = sums[t];
}

// Position of each item among the items with the same key, in item order,
// plus `base[key]`; slot = position if it is below capacity, else -1.
__global__ __launch_bounds__(kThreads) void disp_rank_kernel(KeyArgs g, int E, int cap,
                                                             const int32_t* __restrict__ blockbase,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ slot_out) {
  __shared__ int wcnt[kThreads / MOE_WAVE][256];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (kThreads / MOE_WAVE) * 256; i += kThreads)
    (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int a = blockIdx.x * kThreads + threadIdx.x;
  const int key = item_key(g, a);
  const bool valid = key >= 0;
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  const int rank = __popcll(m & moe::lanemask_lt());
  if (valid && rank == 0) wcnt[wave][key] = __popcll(m);
  __syncthreads();
  if (a < g.A) {
    int slot = -1;
    if (valid) {
      int pos = blockbase[(size_t)blockIdx.x * E + key] + rank + (base ? base[key] : 0);
      for (int w = 0; w < wave; ++w) pos += wcnt[w][key];
      slot = (cap < 0 || pos < cap) ? pos : -1;
    }
    slot_out[a] = slot;
  }
}

// kept counts, offsets (exclusive scan over experts), routed counts.
__global__ __launch_bounds__(kThreads) void disp_finalize_kernel(
    int E, int cap, int reroute, const int32_t* __restrict__ routed,
    const int32_t* __restrict__ demand2, int32_t* __restrict__ kept1_out,
    int32_t* __restrict__ counts_routed, int32_t* __restrict__ counts_kept,
    int32_t* __restrict__ offsets) {
  __shared__ int sc[kThreads];
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E) {
    const int r = routed[e];
    int k1 = (cap < 0) ? r : min(r, cap);
    kept = k1;
    if (reroute) kept += min(demand2[e], max(cap - k1, 0));
    counts_routed[e] = r;
    counts_kept[e] = kept;
    if (kept1_out) kept1_out[e] = k1;
  }
  sc[e] = kept;
  __syncthreads();
  // Hillis-Steele inclusive scan (integers: exact)
  for (int o = 1; o < kThreads; o <<= 1) {
    int v = e >= o ? sc[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e] = sc[e] - kept;
  if (e == E - 1) offsets[E] = sc[e];
}

// kept1 only (needed before the reroute rank pass).
__global__ __launch_bounds__(kThreads) void disp_kept1_kernel(int E, int cap,
                                                              const int32_t* __restrict__ routed,
                                                              int32_t* __restrict__ kept1) {
  const int e = threadIdx.x;
  if (e < E) kept1[e] = min(routed[e], cap);
}

struct ScatterArgs {
  int N, k, C, policy;
  const int32_t* cand;
  const float* cand_s;
  const int32_t* slot1;  // [k*N] rank-major
  const int32_t* slot2;  // [N] or null
  const int32_t* offsets;
  float* gates;
  int32_t* row_of;
  int32_t* expert_of;
  int32_t* perm_token;
};

__global__ __launch_bounds__(kThreads) void disp_scatter_kernel(ScatterArgs s) {
  const int a = blockIdx.x * kThreads + threadIdx.x;  // token-major output index
  if (a >= s.N * s.k) return;
  const int t = a / s.k, j = a - t * s.k;
  int e = s.cand[(size_t)t * s.C + j];
  int slot = s.slot1[(size_t)j * s.N + t];
  if (slot < 0 && s.slot2) {
    const int s2 = s.slot2[t];
    if (s2 >= 0) {
      e = s.cand[(size_t)t * s.C + 1];
      slot = s2;
      s.gates[a] = s.cand_s[(size_t)t * s.C + 1];
    }
  }
  if (slot < 0) {
    s.row_of[a] = -1;
    s.expert_of[a] = -1;
    if (s.policy != MOE_DROPLESS) s.gates[a] = 0.f;
  } else {
    const int row = s.offsets[e] + slot;
    s.row_of[a] = row;
    s.expert_of[a] = e;
    s.perm_token[row] = t;
  }
}

// The whole dispatch in one workgroup for small problems (N*k <= 8192, no
// reroute): the same stable counting sort in rank-major item order. Every
// key is loaded up front (8 per thread, rank-major item a = c*1024 + tid);
// then the items are taken 1024 at a time in order: ranks inside a wave
// from ballots over the key bits, each wave's per-expert count in LDS, and
// per expert an exclusive prefix over the waves plus the count carried from
// the earlier chunks. Capacity, kept counts, offsets and the scatter follow
// in the same workgroup, without the five launches of the general path
// (decode and small batches are launch-bound).
constexpr int kSmallThreads = 1024, kSmallWaves = kSmallThreads / MOE_WAVE;
constexpr int kSmallMaxItems = 8192, kSmallChunks = kSmallMaxItems / kSmallThreads;

__global__ __launch_bounds__(kSmallThreads) void disp_small_kernel(
    int N, int E, int k, int C, int policy, int cap, const int32_t* __restrict__ cand,
    float* __restrict__ gates, int32_t* __restrict__ counts_routed,
    int32_t* __restrict__ counts_kept, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of, int32_t* __restrict__ expert_of,
    int32_t* __restrict__ perm_token) {
  __shared__ int key_s[kSmallMaxItems];   // rank-major keys
  __shared__ int slot_s[kSmallMaxItems];  // rank-major slots (-1: dropped / no key)
  __shared__ int wcnt[kSmallWaves][256];  // this chunk's count per wave and expert
  __shared__ int wpre[kSmallWaves][256];  // items of the expert before this wave
  __shared__ int off_s[256];              // inclusive scan of the kept counts
  const int tid = threadIdx.x, wave = tid >> 6;
  const int A = N * k;
  int bits = 1;
  while ((1 << bits) < E) ++bits;
  int key[kSmallChunks];
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int a = c * kSmallThreads + tid;
    key[c] = -1;
    if (a < A) {
      const int j = a / N, t = a - j * N;
      key[c] = valid_key(cand[(size_t)t * C + j], E);
    }
  }
  for (int i = tid; i < kSmallWaves * 256; i += kSmallThreads) (&wcnt[0][0])[i] = 0;
  int running = 0;  // thread e < E: items of expert e in the chunks so far
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    if (c * kSmallThreads >= A) break;  // uniform
    const int a = c * kSmallThreads + tid;
    const int kc = key[c];
    const bool valid = kc >= 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (kc >> b) & 1;
      const uint64_t bal = __ballot(bit);
      m &= bit ? bal : ~bal;
    }
    const int rank = __popcll(m & moe::lanemask_lt());
    if (valid && rank == 0) wcnt[wave][kc] = __popcll(m);
    __syncthreads();
    if (tid < E) {
      int v[kSmallWaves];
#pragma unroll
      for (int w = 0; w < kSmallWaves; ++w) v[w] = wcnt[w][tid];
#pragma unroll
      for (int w = 0; w < kSmallWaves; ++w) {
        wpre[w][tid] = running;
        running += v[w];
        wcnt[w][tid] = 0;
      }
    }
    __syncthreads();
    if (a < A) {
      key_s[a] = kc;
      int slot = -1;
      if (valid) {
        const int pos = wpre[wave][kc] + rank;
        slot = (cap < 0 || pos < cap) ? pos : -1;
      }
      slot_s[a] = slot;
    }
  }
  // kept counts and offsets (Hillis-Steele scan over at most 256 experts)
  int kept = 0;
  if (tid < E) {
    kept = cap < 0 ? running : min(running, cap);
    counts_routed[tid] = running;
    counts_kept[tid] = kept;
  }
  if (tid < 256) off_s[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = (tid < 256 && tid >= o) ? off_s[tid - o] : 0;
    __syncthreads();
    if (tid < 256) off_s[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid] = off_s[tid] - kept;
  if (tid == E - 1) offsets[E] = off_s[tid];
  // scatter, token-major output index a = t*k + j (reads only LDS written
  // before the scan's barriers)
  for (int a = tid; a < A; a += kSmallThreads) {
    const int t = a / k, j = a - t * k;
    const int e = key_s[j * N + t];
    const int slot = slot_s[j * N + t];
    if (slot < 0) {
      row_of[a] = -1;
      expert_of[a] = -1;
      if (policy != MOE_DROPLESS) gates[a] = 0.f;
    } else {
      const int row = (e == 0 ? 0 : off_s[e - 1]) + slot;  // off_s is inclusive
      row_of[a] = row;
      expert_of[a] = e;
      perm_token[row] = t;
    }
  }
}

// x_perm[r] = x[perm_token[r]] for r < offsets[E]; 16-byte lanes.
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(
    const u32x4_t* __restrict__ x, const int32_t* __restrict__ perm_token,
    const int32_t* __restrict__ offsets, int E, int chunks_per_row, u32x4_t* __restrict__ xp) {
  const int R = offsets[E];
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const size_t src = (size_t)perm_token[r] * chunks_per_row;
    const size_t dst = (size_t)r * chunks_per_row;
    for (int c = threadIdx.x; c < chunks_per_row; c += kThreads) xp[dst + c] = x[src + c];
  }
}

}  // namespace

namespace moe_host {

static size_t disp_nblk(int A) { return (size_t)(A + kThreads - 1) / kThreads; }

static moe_status gather_launch(int N, int E, int k, const void* x, moe_dtype x_dt, int d,
                                const int32_t* perm_token, const int32_t* offsets, void* x_perm,
                                hipStream_t st) {
  const int A = N * k;
  const int esz = x_dt == MOE_BF16 ? 2 : 4;
  const int chunks = d * esz / 16;
  const int grid = A < 4096 ? A : 4096;
  gather_rows_kernel<<<grid, kThreads, 0, st>>>((const u32x4_t*)x, perm_token, offsets, E,
                                                chunks, (u32x4_t*)x_perm);
  return launch_status("dispatch gather");
}

size_t dispatch_workspace_bytes(int N, int E, int k) {
  const size_t A = (size_t)N * k;
  const size_t nb = disp_nblk((int)A);
  size_t s = 0;
  s += 2 * align256(nb * E * sizeof(int32_t));  // blockcnt, blockbase
  s += align256(A * sizeof(int32_t));           // slot1
  s += align256((size_t)N * sizeof(int32_t));   // slot2
  s += 3 * align256((size_t)E * sizeof(int32_t));  // routed, demand2, kept1
  return s;
}

moe_status dispatch_launch(int N, int E, int k, int C, moe_overflow policy, int cap,
                           const int32_t* cand, const float* cand_s, float* gates,
                           const void* x, moe_dtype x_dt, int d, int32_t* counts_routed,
                           int32_t* counts_kept, int32_t* offsets, int32_t* row_of,
                           int32_t* expert_of, int32_t* perm_token, void* x_perm,
                           void* workspace, hipStream_t st) {
  const int A = N * k;
  const int nb = (int)disp_nblk(A);
  char* ws = (char*)workspace;
  int32_t* blockcnt = (int32_t*)ws;
  ws += align256((size_t)nb * E * sizeof(int32_t));
  int32_t* blockbase = (int32_t*)ws;
  ws += align256((size_t)nb * E * sizeof(int32_t));
  int32_t* slot1 = (int32_t*)ws;
  ws += align256((size_t)A * sizeof(int32_t));
  int32_t* slot2 = (int32_t*)ws;
  ws += align256((size_t)N * sizeof(int32_t));
  int32_t* routed = (int32_t*)ws;
  ws += align256((size_t)E * sizeof(int32_t));
  int32_t* demand2 = (int32_t*)ws;
  ws += align256((size_t)E * sizeof(int32_t));
  int32_t* kept1 = (int32_t*)ws;

  const int ecap = (policy == MOE_DROPLESS) ? -1 : cap;
  const bool reroute = policy == MOE_REROUTE_THEN_DROP;

  moe_status s;
  if (!reroute && A <= kSmallMaxItems) {
    disp_small_kernel<<<1, kSmallThreads, 0, st>>>(N, E, k, C, (int)policy, ecap, cand, gates,
                                                   counts_routed, counts_kept, offsets, row_of,
                                                   expert_of, perm_token);
    s = launch_status("dispatch (one workgroup)");
    if (s != MOE_OK || !x_perm) return s;
    return gather_launch(N, E, k, x, x_dt, d, perm_token, offsets, x_perm, st);
  }

  KeyArgs g1{N, k, C, 0, cand, nullptr, A, E};
  disp_count_kernel<<<nb, kThreads, 0, st>>>(g1, E, blockcnt);
  disp_scan_kernel<<<E, kThreads, 0, st>>>(nb, E, blockcnt, blockbase, routed);
  disp_rank_kernel<<<nb, kThreads, 0, st>>>(g1, E, ecap, blockbase, nullptr, slot1);
  s = launch_status("dispatch phase 1");
  if (s != MOE_OK) return s;

  if (reroute) {
    const int nb2 = (int)disp_nblk(N);
    KeyArgs g2{N, k, C, 1, cand, slot1, N, E};
    disp_kept1_kernel<<<1, kThreads, 0, st>>>(E, cap, routed, kept1);
    disp_count_kernel<<<nb2, kThreads, 0, st>>>(g2, E, blockcnt);
    disp_scan_kernel<<<E, kThreads, 0, st>>>(nb2, E, blockcnt, blockbase, demand2);
    disp_rank_kernel<<<nb2, kThreads, 0, st>>>(g2, E, cap, blockbase, kept1, slot2);
    s = launch_status("dispatch reroute phase");
    if (s != MOE_OK) return s;
  }
  disp_finalize_kernel<<<1, kThreads, 0, st>>>(E, ecap, reroute ? 1 : 0, routed, demand2,
                                               nullptr, counts_routed, counts_kept, offsets);
  ScatterArgs sa{N, k, C, (int)policy, cand, cand_s, slot1, reroute ? slot2 : nullptr,
                 offsets, gates, row_of, expert_of, perm_token};
  disp_scatter_kernel<<<(A + kThreads - 1) / kThreads, kThreads, 0, st>>>(sa);
  s = launch_status("dispatch scatter");
  if (s != MOE_OK || !x_perm) return s;
  return gather_launch(N, E, k, x, x_dt, d, perm_token, offsets, x_perm, st);
}

// ---------------------------------------------------------------- no-alloc
// Scratch for moe_dispatch_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends. Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): the address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept per device. Every
// dispatch kernel writes each scratch word it later reads, so nothing needs
// clearing between calls; calls that overlap on one GPU share the array and
// race.
static __device__ __align__(256) char dispatch_scratch[MOE_DISPATCH_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

moe_status dispatch_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("moe_dispatch_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return MOE_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("moe_dispatch_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    return MOE_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(dispatch_scratch));
    if (e != hipSuccess || !p) {
      set_error("moe_dispatch_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
                hipGetErrorString(e));
      return MOE_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe_host
