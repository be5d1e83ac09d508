// grouped_ffn_bwd.hip -- backward pass of the grouped expert FFN (SwiGLU,
// or ReLU / GELU) on gfx950 (bf16 MFMA, fp32 accumulation).
//
// heavensheep.xyz MoE notes, "Training": an expert receives gradient only
// from the tokens routed to it; mkbk-pku.cn "通信与并行", step 5: the
// backward pass follows the forward's routing path back. Per expert e, over
// its packed rows r (x_r its token row, o_r = h_r W2^T its output, dO_r =
// gate * dy of the token, a = x W1^T, u = x W3^T, h = silu(a) * u):
//   dh  = dO W2                      data gradient of GEMM 2
//   da  = dh * u * silu'(a), du = dh * silu(a)     (fused in its epilogue)
//   dW2 = sum_r dO_r^T h_r           weight gradient of GEMM 2
//   dX  = da W1 + du W3              data gradient of GEMM 1 (K = 2 d_ff)
//   dW1 = sum_r da_r^T x_r, dW3 = sum_r du_r^T x_r   (one launch)
// The forward's training call saved a and u (bf16) and h (bf16, the exact
// operand GEMM 2 used). dX stays in packed row order; the router's backward
// sums it back to tokens. ReLU / GELU experts (h = act(a)) have one gate
// plane: da = dh act'(a), dX = da W1, dW1 = sum_r da_r^T x_r.
#include "gemm_bwd.h"

// Tile shapes: 256-row M tiles; N tile width and the wave grid per tile space
#ifndef MOE_BWD_ROWS_BN
#define MOE_BWD_ROWS_BN 256
#endif
#ifndef MOE_BWD_ROWS_WGM
#define MOE_BWD_ROWS_WGM 4
#endif
#ifndef MOE_BWD_DENSE_BN
#define MOE_BWD_DENSE_BN 256
#endif
#ifndef MOE_BWD_DENSE_WGM
#define MOE_BWD_DENSE_WGM 4
#endif
// N tiles that run side by side over consecutive M tiles (L2 reuse of both operands)
#ifndef MOE_BWD_ROWS_GN
#define MOE_BWD_ROWS_GN 2
#endif
#ifndef MOE_BWD_DENSE_GN
#define MOE_BWD_DENSE_GN 16
#endif

namespace {

constexpr int kBwdBM = 256;
constexpr int kRowsBN = MOE_BWD_ROWS_BN, kDenseBN = MOE_BWD_DENSE_BN;
constexpr int kRowsWGM = MOE_BWD_ROWS_WGM, kDenseWGM = MOE_BWD_DENSE_WGM;

// tile_start[e] = sum over e' < e of ceil(rows_e' / bm)
__global__ __launch_bounds__(256) void bwd_tile_table_kernel(const int32_t* __restrict__ offsets,
                                                             int E, int bm,
                                                             int32_t* __restrict__ ts) {
  __shared__ int sc[256];
  const int e = threadIdx.x;
  const int n = e < E ? (offsets[e + 1] - offsets[e] + bm - 1) / bm : 0;
  sc[e] = n;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? sc[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) {
    ts[e] = sc[e] - n;
    if (e == E - 1) ts[E] = sc[e];
  }
}

// x_perm[r] = x[row_index[r]] for r < offsets[E] (bf16 rows, 16 bytes a lane)
__global__ __launch_bounds__(256) void bwd_gather_kernel(const uint16_t* __restrict__ x,
                                                         const int32_t* __restrict__ row_index,
                                                         const int32_t* __restrict__ offsets,
                                                         int E, int d,
                                                         uint16_t* __restrict__ xp) {
  const int R = offsets[E];
  const int vec = d / 8;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < (size_t)R * vec;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / vec, c = i - r * vec;
    ((u32x4_t*)xp)[r * vec + c] = ((const u32x4_t*)x)[(size_t)row_index[r] * vec + c];
  }
}

moe_status bwd_status(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    moe_host::set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace

namespace moe_host {

// workspace: tile table [E+1] int32 | dpre [max_rows][2F] bf16 | x_perm [max_rows][d] bf16
size_t grouped_ffn_backward_workspace_bytes(const moe_ffn_weights* w, int max_rows,
                                            bool gather) {
  return align256((size_t)(w->n_experts + 1) * 4) +
         align256((size_t)max_rows * 2 * w->d_ff * 2) +
         (gather ? align256((size_t)max_rows * w->d_model * 2) : 0);
}

moe_status grouped_ffn_backward_launch(const moe_ffn_weights* w, const void* x_rows,
                                       const int32_t* row_index, const int32_t* offsets,
                                       int max_rows, const uint16_t* preact, const uint16_t* h,
                                       const uint16_t* d_out, float* dx_rows, void* dw1,
                                       void* dw3, void* dw2, moe_dtype dw_dt, void* workspace,
                                       hipStream_t st) {
  using namespace moe_bwd;
  const int E = w->n_experts, d = w->d_model, F = w->d_ff;
  const bool glu = w->act == MOE_SWIGLU;
  const int P = glu ? 2 * F : F;  // columns of the saved pre-activations and of dpre
  char* ws = (char*)workspace;
  int32_t* ts = (int32_t*)ws;
  ws += align256((size_t)(E + 1) * 4);
  uint16_t* dpre = (uint16_t*)ws;
  ws += align256((size_t)max_rows * 2 * F * 2);
  const uint16_t* xp = (const uint16_t*)x_rows;
  if (row_index) {
    uint16_t* g = (uint16_t*)ws;
    bwd_gather_kernel<<<2048, 256, 0, st>>>((const uint16_t*)x_rows, row_index, offsets, E, d, g);
    moe_status s = launch_status("backward gather");
    if (s != MOE_OK) return s;
    xp = g;
  }
  bwd_tile_table_kernel<<<1, 256, 0, st>>>(offsets, E, kBwdBM, ts);
  moe_status s = launch_status("backward tile table");
  if (s != MOE_OK) return s;
  const int max_mt = (max_rows + kBwdBM - 1) / kBwdBM + E;

  // data gradient of GEMM 2 with the SwiGLU backward in its epilogue
  BwdArgs g{};
  g.E = E;
  g.offsets = offsets;
  g.tile_start = ts;
  g.max_mt = max_mt;
  BwdArgs d2 = g;
  d2.group_n = MOE_BWD_ROWS_GN;
  d2.A = d_out;
  d2.lda = d;
  d2.B0 = (const uint16_t*)w->w2;  // [E][d][F]: row k = feature of d
  d2.ldb = F;
  d2.b_expert = (long long)d * F;
  d2.N = F;
  d2.K = d;
  d2.n_tiles_n = F / kRowsBN;
  d2.pre = preact;
  d2.dpre = dpre;
  d2.act = (int)w->act;
  const long long d2_tiles =
      (long long)max_mt * ((d2.n_tiles_n + d2.group_n - 1) / d2.group_n * d2.group_n);
  hipError_t err =
      glu ? launch_bwd<MODE_ROWS, BEPI_DSWIGLU, 256, kRowsBN, 2, kRowsWGM, 8 / kRowsWGM>(
                d2, d2_tiles, st)
          : launch_bwd<MODE_ROWS, BEPI_DACT, 256, kRowsBN, 2, kRowsWGM, 8 / kRowsWGM>(
                d2, d2_tiles, st);
  if (err != hipSuccess) return bwd_status(err, "backward data gradient of GEMM 2");

  // weight gradient of GEMM 2: dW2[e][c][f] = sum_r dO[r][c] h[r][f]
  BwdArgs w2 = g;
  w2.group_n = MOE_BWD_DENSE_GN;
  w2.A = d_out;
  w2.lda = d;
  w2.B0 = h;
  w2.ldb = F;
  w2.M = d;
  w2.N = F;
  w2.mseg = d;
  w2.C0 = dw2;
  w2.c_bf16 = dw_dt == MOE_BF16;
  w2.ldc = F;
  w2.n_tiles_n = F / kDenseBN;
  err = launch_bwd<MODE_DENSE, BEPI_F32, 256, kDenseBN, 2, kDenseWGM, 8 / kDenseWGM>(
      w2, (long long)E * (d / 256) * ((w2.n_tiles_n + w2.group_n - 1) / w2.group_n * w2.group_n), st);
  if (err != hipSuccess) return bwd_status(err, "backward weight gradient of GEMM 2");

  // data gradient of GEMM 1: dX = [da | du] [W1 ; W3], K = 2F
  BwdArgs d1 = g;
  d1.group_n = MOE_BWD_ROWS_GN;
  d1.A = dpre;
  d1.lda = P;
  d1.B0 = (const uint16_t*)w->w1;  // [E][F][d]
  d1.B1 = glu ? (const uint16_t*)w->w3 : nullptr;
  d1.kseg = F;
  d1.ldb = d;
  d1.b_expert = (long long)F * d;
  d1.N = d;
  d1.K = P;
  d1.n_tiles_n = d / kRowsBN;
  d1.C0 = dx_rows;
  d1.ldc = d;
  err = launch_bwd<MODE_ROWS, BEPI_F32, 256, kRowsBN, 2, kRowsWGM, 8 / kRowsWGM>(
      d1, (long long)max_mt * ((d1.n_tiles_n + d1.group_n - 1) / d1.group_n * d1.group_n), st);
  if (err != hipSuccess) return bwd_status(err, "backward data gradient of GEMM 1");

  // weight gradients of GEMM 1: rows m < F of [da | du]^T x -> dW1, the rest -> dW3
  BwdArgs w1 = g;
  w1.group_n = MOE_BWD_DENSE_GN;
  w1.A = dpre;
  w1.lda = P;
  w1.B0 = xp;
  w1.ldb = d;
  w1.M = P;
  w1.N = d;
  w1.mseg = F;
  w1.C0 = dw1;
  w1.C1 = glu ? dw3 : nullptr;
  w1.c_bf16 = dw_dt == MOE_BF16;
  w1.ldc = d;
  w1.n_tiles_n = d / kDenseBN;
  err = launch_bwd<MODE_DENSE, BEPI_F32, 256, kDenseBN, 2, kDenseWGM, 8 / kDenseWGM>(
      w1, (long long)E * (P / 256) * ((w1.n_tiles_n + w1.group_n - 1) / w1.group_n * w1.group_n), st);
  return bwd_status(err, "backward weight gradient of GEMM 1");
}

}  // namespace moe_host
