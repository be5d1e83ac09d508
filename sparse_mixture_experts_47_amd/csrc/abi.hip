// abi.hip -- libmoe's C entry points: host-side validation, workspace
// layout, and the launches on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "moe_device.h"

namespace moe_host {

size_t router_workspace_bytes(int N, int d, int E, int with_noise);
size_t router_planes_bytes(int E, int d, int with_noise);
moe_status router_prepare_launch(const float* w_gate, const float* w_noise, int E, int d,
                                 uint16_t* planes, hipStream_t st);
moe_status router_launch(const moe_router_params* p, const void* x, moe_dtype x_dt,
                         const float* w_gate, const float* logits_in, int32_t* cand_ids,
                         float* cand_scores, float* gates, float* logits_out,
                         double* score_sums, void* workspace, hipStream_t st);
size_t dispatch_workspace_bytes(int N, int E, int k);
moe_status dispatch_scratch_ptr(void** out);
moe_status dispatch_launch(int N, int E, int k, int C, moe_overflow policy, int cap,
                           const int32_t* cand, const float* cand_s, float* gates,
                           const void* x, moe_dtype x_dt, int d, int32_t* counts_routed,
                           int32_t* counts_kept, int32_t* offsets, int32_t* row_of,
                           int32_t* expert_of, int32_t* perm_token, void* x_perm,
                           void* workspace, hipStream_t st);
size_t grouped_ffn_workspace_bytes(const moe_ffn_weights* w, moe_dtype act_dt, int max_rows);
moe_status grouped_ffn_launch(const moe_ffn_weights* w, const void* x_rows, moe_dtype act_dt,
                              const int32_t* row_index, const int32_t* offsets, int max_rows,
                              void* y_rows, moe_dtype y_dt, void* workspace, hipStream_t st,
                              uint16_t* preact = nullptr, uint16_t* h_out = nullptr,
                              const int32_t* out_token = nullptr,
                              const float* out_gate = nullptr);
moe_status combine_dropped_launch(int N, int d, const int32_t* row_of, const float* gates,
                                  float* gate_row, float* y, hipStream_t st);
float* row_gates_ws(const moe_ffn_weights* w, moe_dtype act_dt, int max_rows, void* ws);
size_t grouped_ffn_backward_workspace_bytes(const moe_ffn_weights* w, int max_rows,
                                            bool gather);
moe_status grouped_ffn_backward_launch(const moe_ffn_weights* w, const void* x_rows,
                                       const int32_t* row_index, const int32_t* offsets,
                                       int max_rows, const uint16_t* preact, const uint16_t* h,
                                       const uint16_t* d_out, float* dx_rows, void* dw1,
                                       void* dw3, void* dw2, moe_dtype dw_dt, void* workspace,
                                       hipStream_t st);
moe_status combine_backward_launch(int N, int d, int k, const float* dy, const void* y_rows,
                                   moe_dtype y_dt, const int32_t* row_of, const float* gates,
                                   uint16_t* d_rows, float* dgates, uint16_t* d_shared,
                                   hipStream_t st);
size_t router_backward_workspace_bytes(int N, int d, int E);
moe_status router_backward_launch(int N, int d, int E, int k, int C, int renormalize,
                                  const void* x, moe_dtype x_dt, const float* w_gate,
                                  const float* logits, const int32_t* cand_ids,
                                  const int32_t* expert_of, const int32_t* row_of,
                                  const float* dgates, const int32_t* counts_routed, float alpha,
                                  float beta, const float* dx_rows, const float* dx_shared,
                                  const float* w_noise, const float* noise_v, uint64_t seed,
                                  float* dlogits, float* dw_gate, float* dlogit_bias,
                                  float* dw_noise, float* dx, void* workspace, hipStream_t st);
moe_status combine_launch(int N, int d, int k, const void* y_rows, moe_dtype y_dt,
                          const int32_t* row_of, const float* gates, const void* y_shared,
                          moe_dtype sh_dt, void* y, moe_dtype out_dt, hipStream_t st);
moe_status expert_choice_launch(int N, int E, int capacity, const float* scores,
                                int32_t* offsets, int32_t* perm_token, int32_t* row_of,
                                float* gates, int32_t* counts, hipStream_t st);
moe_status balance_stats_launch(int N, int E, int k, const int32_t* routed, const int32_t* kept,
                                const double* sums, float* f, float* P, float* scalars,
                                float* bias, float rate, hipStream_t st);

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

moe_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace moe_host

using namespace moe_host;

#define CHECK(cond, code, ...)      \
  do {                              \
    if (!(cond)) {                  \
      set_error(__VA_ARGS__);       \
      return code;                  \
    }                               \
  } while (0)

static moe_status check_ws(void* ws, size_t have, size_t need, const char* who) {
  CHECK(need == 0 || (ws != nullptr && have >= need), MOE_EWORKSPACE,
        "%s: workspace of %zu bytes needed, %zu given%s", who, need, have,
        ws ? "" : " (NULL)");
  CHECK(((uintptr_t)ws & 255) == 0, MOE_EINVAL, "%s: workspace must be 256-byte aligned", who);
  return MOE_OK;
}

extern "C" {

const char* moe_version(void) { return "libmoe 0.1 gfx950"; }

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE";
    case MOE_EHIP: return "MOE_EHIP";
  }
  return "MOE_UNKNOWN";
}

int32_t moe_capacity(int32_t n_tokens, int32_t n_experts, int32_t cf_num, int32_t cf_den) {
  if (n_tokens <= 0 || n_experts <= 0 || cf_num < 0 || cf_den <= 0) return -1;
  // ceil(N * num / (E * den)) in exact integer arithmetic: both products fit
  // in 62 bits, so no rounding enters before the one ceiling
  const int64_t p = (int64_t)n_tokens * cf_num, q = (int64_t)n_experts * cf_den;
  const int64_t c = (p + q - 1) / q;
  return c > INT32_MAX ? INT32_MAX : (int32_t)c;
}

size_t moe_router_workspace_bytes(int32_t n_tokens, int32_t d_model, int32_t n_experts,
                                  int32_t with_noise) {
  if (n_tokens <= 0 || n_experts <= 0 || d_model < 0) return 0;
  return router_workspace_bytes(n_tokens, d_model, n_experts, with_noise);
}

size_t moe_dispatch_workspace_bytes(int32_t n_tokens, int32_t n_experts, int32_t top_k) {
  if (n_tokens <= 0 || n_experts <= 0 || top_k <= 0) return 0;
  return dispatch_workspace_bytes(n_tokens, n_experts, top_k);
}

size_t moe_grouped_ffn_workspace_bytes(const moe_ffn_weights* w, moe_dtype act_dt,
                                       int32_t max_rows) {
  if (!w || max_rows <= 0) return 0;
  return grouped_ffn_workspace_bytes(w, act_dt, max_rows);
}

size_t moe_workspace_bytes(int32_t n_tokens, int32_t n_experts, int32_t top_k, int32_t d_model,
                           int32_t d_ff) {
  if (n_tokens <= 0 || n_experts <= 0 || top_k <= 0) return 0;
  size_t a = router_workspace_bytes(n_tokens, d_model, n_experts, 1);
  size_t b = dispatch_workspace_bytes(n_tokens, n_experts, top_k);
  moe_ffn_weights w = {};
  w.n_experts = n_experts;
  w.d_model = d_model;
  w.d_ff = d_ff;
  size_t c = grouped_ffn_workspace_bytes(&w, MOE_F32, n_tokens * top_k);
  size_t m = a > b ? a : b;
  return m > c ? m : c;
}

size_t moe_router_planes_bytes(int32_t n_experts, int32_t d_model, int32_t with_noise) {
  if (n_experts <= 0 || d_model <= 0) return 0;
  return router_planes_bytes(n_experts, d_model, with_noise ? 1 : 0);
}

moe_status moe_router_prepare(const float* w_gate, const float* w_noise, int32_t n_experts,
                              int32_t d_model, void* planes, size_t planes_bytes,
                              void* hip_stream) {
  CHECK(w_gate && planes, MOE_EINVAL, "moe_router_prepare: NULL w_gate or planes");
  CHECK(n_experts >= 1 && d_model >= 1, MOE_EINVAL, "moe_router_prepare: E=%d d=%d", n_experts,
        d_model);
  CHECK(n_experts <= 256, MOE_EUNSUPPORTED, "moe_router_prepare: n_experts %d > 256",
        n_experts);
  CHECK(d_model % 64 == 0, MOE_EINVAL, "moe_router_prepare: d_model %d %% 64 != 0", d_model);
  const size_t need = router_planes_bytes(n_experts, d_model, w_noise ? 1 : 0);
  CHECK(planes_bytes >= need, MOE_EWORKSPACE,
        "moe_router_prepare: %zu bytes of planes needed, %zu given", need, planes_bytes);
  CHECK(((uintptr_t)planes & 15) == 0, MOE_EINVAL,
        "moe_router_prepare: planes not 16-byte aligned");
  return router_prepare_launch(w_gate, w_noise, n_experts, d_model, (uint16_t*)planes,
                               (hipStream_t)hip_stream);
}

moe_status moe_router_topk(const moe_router_params* p, const void* x, moe_dtype x_dt,
                           const float* w_gate, const float* logits_in, int32_t* cand_ids,
                           float* cand_scores, float* gates, float* logits_out,
                           double* score_sums, void* workspace, size_t ws_bytes,
                           void* hip_stream) {
  CHECK(p, MOE_EINVAL, "moe_router_topk: params is NULL");
  const int N = p->n_tokens, d = p->d_model, E = p->n_experts, k = p->top_k, C = p->n_cand;
  CHECK(N >= 1 && E >= 1 && k >= 1, MOE_EINVAL, "moe_router_topk: N=%d E=%d k=%d must be >= 1",
        N, E, k);
  CHECK(k <= E, MOE_EINVAL, "moe_router_topk: top_k %d > n_experts %d", k, E);
  CHECK(C == k || C == k + 1, MOE_EINVAL, "moe_router_topk: n_cand %d must be k or k+1", C);
  CHECK(C <= E, MOE_EINVAL, "moe_router_topk: n_cand %d > n_experts %d", C, E);
  CHECK((long long)N * C < (1ll << 31), MOE_EINVAL, "moe_router_topk: N*n_cand too large");
  CHECK(cand_ids && cand_scores && gates, MOE_EINVAL, "moe_router_topk: NULL output");
  CHECK(E <= 256, MOE_EUNSUPPORTED, "moe_router_topk: n_experts %d > 256", E);
  CHECK(k <= 8, MOE_EUNSUPPORTED, "moe_router_topk: top_k %d > 8", k);
  if (!logits_in) {
    CHECK(x && w_gate, MOE_EINVAL, "moe_router_topk: x and w_gate needed without logits_in");
    CHECK(d >= 1, MOE_EINVAL, "moe_router_topk: d_model %d", d);
    CHECK(x_dt == MOE_F32 || x_dt == MOE_BF16, MOE_EUNSUPPORTED,
          "moe_router_topk: x dtype must be F32 or BF16");
  }
  CHECK(((uintptr_t)p->w_planes & 15) == 0, MOE_EINVAL,
        "moe_router_topk: w_planes not 16-byte aligned");
  const int noise = (!logits_in && p->w_noise) ? 1 : 0;
  moe_status s = check_ws(workspace, ws_bytes, router_workspace_bytes(N, logits_in ? 0 : d, E, noise),
                          "moe_router_topk");
  if (s != MOE_OK) return s;
  return router_launch(p, x, x_dt, w_gate, logits_in, cand_ids, cand_scores, gates, logits_out,
                       score_sums, workspace, (hipStream_t)hip_stream);
}

static moe_status check_dispatch(const char* who, int32_t n_tokens, int32_t n_experts,
                                 int32_t top_k, int32_t n_cand, moe_overflow policy,
                                 int32_t capacity, const int32_t* cand_ids,
                                 const float* cand_scores, const float* gates, const void* x,
                                 moe_dtype x_dt, int32_t d_model, const int32_t* counts_routed,
                                 const int32_t* counts_kept, const int32_t* offsets,
                                 const int32_t* row_of, const int32_t* expert_of,
                                 const int32_t* perm_token, const void* x_perm) {
  const int N = n_tokens, E = n_experts, k = top_k, C = n_cand;
  CHECK(N >= 1 && E >= 1 && k >= 1 && k <= E, MOE_EINVAL,
        "%s: N=%d E=%d k=%d out of range", who, N, E, k);
  CHECK(C == k || C == k + 1, MOE_EINVAL, "%s: n_cand %d must be k or k+1", who, C);
  CHECK((long long)N * C < (1ll << 31), MOE_EINVAL, "%s: N*n_cand too large", who);
  CHECK(policy == MOE_DROPLESS || policy == MOE_DROP || policy == MOE_REROUTE_THEN_DROP,
        MOE_EINVAL, "%s: unknown overflow policy %d", who, (int)policy);
  CHECK(policy == MOE_DROPLESS || capacity >= 0, MOE_EINVAL,
        "%s: capacity %d must be >= 0 with a dropping policy", who, capacity);
  CHECK(capacity >= -1, MOE_EINVAL, "%s: capacity %d < -1", who, capacity);
  CHECK(cand_ids && cand_scores && gates && counts_routed && counts_kept && offsets && row_of &&
            expert_of && perm_token,
        MOE_EINVAL, "%s: NULL argument", who);
  CHECK(E <= 256, MOE_EUNSUPPORTED, "%s: n_experts %d > 256", who, E);
  CHECK(policy != MOE_REROUTE_THEN_DROP || (k == 1 && C == 2), MOE_EUNSUPPORTED,
        "%s: reroute needs top_k == 1 and n_cand == 2", who);
  if (x_perm) {
    CHECK(x, MOE_EINVAL, "%s: x_perm given without x", who);
    CHECK(x_dt == MOE_F32 || x_dt == MOE_BF16, MOE_EUNSUPPORTED, "%s: x dtype", who);
    CHECK(d_model >= 8 && d_model % 8 == 0, MOE_EUNSUPPORTED,
          "%s: d_model %d must be a multiple of 8", who, d_model);
  }
  return MOE_OK;
}

moe_status moe_dispatch(int32_t n_tokens, int32_t n_experts, int32_t top_k, int32_t n_cand,
                        moe_overflow policy, int32_t capacity, const int32_t* cand_ids,
                        const float* cand_scores, float* gates, const void* x, moe_dtype x_dt,
                        int32_t d_model, int32_t* counts_routed, int32_t* counts_kept,
                        int32_t* offsets, int32_t* row_of, int32_t* expert_of,
                        int32_t* perm_token, void* x_perm, void* workspace, size_t ws_bytes,
                        void* hip_stream) {
  moe_status s = check_dispatch("moe_dispatch", n_tokens, n_experts, top_k, n_cand, policy,
                                capacity, cand_ids, cand_scores, gates, x, x_dt, d_model,
                                counts_routed, counts_kept, offsets, row_of, expert_of,
                                perm_token, x_perm);
  if (s != MOE_OK) return s;
  s = check_ws(workspace, ws_bytes, dispatch_workspace_bytes(n_tokens, n_experts, top_k),
               "moe_dispatch");
  if (s != MOE_OK) return s;
  return dispatch_launch(n_tokens, n_experts, top_k, n_cand, policy, capacity, cand_ids,
                         cand_scores, gates, x, x_dt, d_model, counts_routed, counts_kept,
                         offsets, row_of, expert_of, perm_token, x_perm, workspace,
                         (hipStream_t)hip_stream);
}

moe_status moe_dispatch_noalloc(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                                int32_t n_cand, moe_overflow policy, int32_t capacity,
                                const int32_t* cand_ids, const float* cand_scores, float* gates,
                                const void* x, moe_dtype x_dt, int32_t d_model,
                                int32_t* counts_routed, int32_t* counts_kept, int32_t* offsets,
                                int32_t* row_of, int32_t* expert_of, int32_t* perm_token,
                                void* x_perm, void* hip_stream) {
  moe_status s = check_dispatch("moe_dispatch_noalloc", n_tokens, n_experts, top_k, n_cand,
                                policy, capacity, cand_ids, cand_scores, gates, x, x_dt,
                                d_model, counts_routed, counts_kept, offsets, row_of,
                                expert_of, perm_token, x_perm);
  if (s != MOE_OK) return s;
  const size_t need = dispatch_workspace_bytes(n_tokens, n_experts, top_k);
  CHECK(need <= (size_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES, MOE_EWORKSPACE,
        "moe_dispatch_noalloc: N=%d E=%d k=%d needs %zu bytes of scratch, more than the "
        "library's fixed %zu (use moe_dispatch with a workspace)",
        n_tokens, n_experts, top_k, need, (size_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  s = dispatch_scratch_ptr(&scratch);
  if (s != MOE_OK) return s;
  return dispatch_launch(n_tokens, n_experts, top_k, n_cand, policy, capacity, cand_ids,
                         cand_scores, gates, x, x_dt, d_model, counts_routed, counts_kept,
                         offsets, row_of, expert_of, perm_token, x_perm, scratch,
                         (hipStream_t)hip_stream);
}

static moe_status check_ffn(const moe_ffn_weights* w, const void* x_rows, moe_dtype act_dt,
                            const int32_t* offsets, int32_t max_rows, const void* y_rows,
                            moe_dtype y_dt, void* workspace, size_t ws_bytes) {
  CHECK(w, MOE_EINVAL, "moe_grouped_ffn: weights is NULL");
  const int E = w->n_experts, d = w->d_model, F = w->d_ff;
  CHECK(E >= 1 && d >= 1 && F >= 1 && max_rows >= 1, MOE_EINVAL,
        "moe_grouped_ffn: E=%d d=%d d_ff=%d max_rows=%d out of range", E, d, F, max_rows);
  CHECK(x_rows && offsets && y_rows && w->w1 && w->w2, MOE_EINVAL, "moe_grouped_ffn: NULL argument");
  CHECK(w->act == MOE_RELU || w->act == MOE_GELU || w->act == MOE_SWIGLU, MOE_EINVAL,
        "moe_grouped_ffn: unknown activation %d", (int)w->act);
  CHECK(w->act != MOE_SWIGLU || w->w3, MOE_EINVAL, "moe_grouped_ffn: SwiGLU needs w3");
  CHECK((long long)max_rows * (d > F ? d : F) < (1ll << 40), MOE_EINVAL,
        "moe_grouped_ffn: max_rows too large");
  CHECK(E <= 256, MOE_EUNSUPPORTED, "moe_grouped_ffn: n_experts %d > 256", E);
  if (act_dt == MOE_F32) {
    CHECK(w->w_dt == MOE_F32 && y_dt == MOE_F32, MOE_EUNSUPPORTED,
          "moe_grouped_ffn: fp32 activations need fp32 weights and output");
  } else if (act_dt == MOE_BF16) {
    CHECK(w->w_dt == MOE_BF16 || w->w_dt == MOE_FP8_E4M3, MOE_EUNSUPPORTED,
          "moe_grouped_ffn: bf16 activations need bf16 or fp8 weights");
    CHECK(y_dt == MOE_BF16 || y_dt == MOE_F32, MOE_EUNSUPPORTED, "moe_grouped_ffn: output dtype");
    CHECK(d % 64 == 0 && F % 64 == 0, MOE_EUNSUPPORTED,
          "moe_grouped_ffn: d_model %d and d_ff %d must be multiples of 64", d, F);
    if (w->w_dt == MOE_FP8_E4M3) {
      CHECK(w->act != MOE_RELU, MOE_EUNSUPPORTED, "moe_grouped_ffn: fp8 needs SwiGLU or GELU");
      CHECK(!w->b1 && !w->b2, MOE_EUNSUPPORTED, "moe_grouped_ffn: fp8 path has no biases");
      CHECK(w->s1 && w->s2 && (w->act != MOE_SWIGLU || w->s3), MOE_EINVAL,
            "moe_grouped_ffn: fp8 weights need their scales");
    }
  } else {
    CHECK(0, MOE_EUNSUPPORTED, "moe_grouped_ffn: activation dtype %d", (int)act_dt);
  }
  return check_ws(workspace, ws_bytes, grouped_ffn_workspace_bytes(w, act_dt, max_rows),
                  "moe_grouped_ffn");
}

moe_status moe_grouped_ffn(const moe_ffn_weights* w, const void* x_rows, moe_dtype act_dt,
                           const int32_t* row_index, const int32_t* offsets, int32_t max_rows,
                           void* y_rows, moe_dtype y_dt, void* workspace, size_t ws_bytes,
                           void* hip_stream) {
  const moe_status s = check_ffn(w, x_rows, act_dt, offsets, max_rows, y_rows, y_dt, workspace,
                                 ws_bytes);
  if (s != MOE_OK) return s;
  return grouped_ffn_launch(w, x_rows, act_dt, row_index, offsets, max_rows, y_rows, y_dt,
                            workspace, (hipStream_t)hip_stream);
}

moe_status moe_grouped_ffn_combine_top1(const moe_ffn_weights* w, const void* x_rows,
                                        moe_dtype act_dt, const int32_t* row_index,
                                        const int32_t* offsets, int32_t max_rows,
                                        int32_t n_tokens, const int32_t* perm_token,
                                        const int32_t* row_of, const float* gates, float* y,
                                        void* workspace, size_t ws_bytes, void* hip_stream) {
  moe_status s = check_ffn(w, x_rows, act_dt, offsets, max_rows, y, MOE_F32, workspace,
                           ws_bytes);
  if (s != MOE_OK) return s;
  CHECK(n_tokens >= 1 && perm_token && row_of && gates, MOE_EINVAL,
        "moe_grouped_ffn_combine_top1: n_tokens %d, NULL perm_token/row_of/gates", n_tokens);
  CHECK(max_rows <= n_tokens, MOE_EINVAL,
        "moe_grouped_ffn_combine_top1: %d packed rows for %d tokens (top-1: at most one each)",
        max_rows, n_tokens);
  CHECK(w->w_dt != MOE_FP8_E4M3, MOE_EUNSUPPORTED,
        "moe_grouped_ffn_combine_top1: fp8 experts take moe_grouped_ffn + moe_combine");
  CHECK(w->d_model % 4 == 0, MOE_EUNSUPPORTED,
        "moe_grouped_ffn_combine_top1: d_model %d %% 4 != 0", w->d_model);
  const hipStream_t st = (hipStream_t)hip_stream;
  float* gate_row = row_gates_ws(w, act_dt, max_rows, workspace);
  s = combine_dropped_launch(n_tokens, w->d_model, row_of, gates, gate_row, y, st);
  if (s != MOE_OK) return s;
  return grouped_ffn_launch(w, x_rows, act_dt, row_index, offsets, max_rows, y, MOE_F32,
                            workspace, st, nullptr, nullptr, perm_token, gate_row);
}

// ------------------------------------------------------------ training
static moe_status check_train_weights(const moe_ffn_weights* w, const char* who) {
  CHECK(w, MOE_EINVAL, "%s: weights is NULL", who);
  const int E = w->n_experts, d = w->d_model, F = w->d_ff;
  CHECK(E >= 1 && E <= 256 && d >= 1 && F >= 1, MOE_EINVAL, "%s: E=%d d=%d d_ff=%d out of range",
        who, E, d, F);
  CHECK(w->act == MOE_RELU || w->act == MOE_GELU || w->act == MOE_SWIGLU, MOE_EINVAL,
        "%s: unknown activation %d", who, (int)w->act);
  CHECK(w->w1 && w->w2 && (w->act != MOE_SWIGLU || w->w3), MOE_EINVAL, "%s: NULL weight", who);
  CHECK(w->w_dt == MOE_BF16 && !w->b1 && !w->b2 && !w->h_fp32, MOE_EUNSUPPORTED,
        "%s: training covers bf16 experts without biases and with bf16 h", who);
  CHECK(d % 256 == 0 && F % 256 == 0, MOE_EUNSUPPORTED,
        "%s: d_model %d and d_ff %d must be multiples of 256", who, d, F);
  return MOE_OK;
}

moe_status moe_grouped_ffn_train(const moe_ffn_weights* w, const void* x_rows,
                                 const int32_t* row_index, const int32_t* offsets,
                                 int32_t max_rows, void* y_rows, moe_dtype y_dt,
                                 uint16_t* preact, uint16_t* h, void* workspace, size_t ws_bytes,
                                 void* hip_stream) {
  moe_status s = check_train_weights(w, "moe_grouped_ffn_train");
  if (s != MOE_OK) return s;
  CHECK(max_rows >= 1 && (long long)max_rows * 2 * w->d_ff < (1ll << 40), MOE_EINVAL,
        "moe_grouped_ffn_train: max_rows %d out of range", max_rows);
  CHECK(x_rows && offsets && y_rows && preact && h, MOE_EINVAL,
        "moe_grouped_ffn_train: NULL argument");
  CHECK(y_dt == MOE_BF16 || y_dt == MOE_F32, MOE_EUNSUPPORTED,
        "moe_grouped_ffn_train: output dtype");
  s = check_ws(workspace, ws_bytes, grouped_ffn_workspace_bytes(w, MOE_BF16, max_rows),
               "moe_grouped_ffn_train");
  if (s != MOE_OK) return s;
  return grouped_ffn_launch(w, x_rows, MOE_BF16, row_index, offsets, max_rows, y_rows, y_dt,
                            workspace, (hipStream_t)hip_stream, preact, h);
}

size_t moe_grouped_ffn_backward_workspace_bytes(const moe_ffn_weights* w, int32_t max_rows,
                                                int32_t gather) {
  if (!w || max_rows <= 0) return 0;
  return grouped_ffn_backward_workspace_bytes(w, max_rows, gather != 0);
}

moe_status moe_grouped_ffn_backward(const moe_ffn_weights* w, const void* x_rows,
                                    const int32_t* row_index, const int32_t* offsets,
                                    int32_t max_rows, const uint16_t* preact, const uint16_t* h,
                                    const uint16_t* d_rows, float* dx_rows, void* dw1, void* dw3,
                                    void* dw2, moe_dtype dw_dt, void* workspace, size_t ws_bytes,
                                    void* hip_stream) {
  moe_status s = check_train_weights(w, "moe_grouped_ffn_backward");
  if (s != MOE_OK) return s;
  CHECK(max_rows >= 1 && (long long)max_rows * 2 * w->d_ff < (1ll << 40), MOE_EINVAL,
        "moe_grouped_ffn_backward: max_rows %d out of range", max_rows);
  CHECK(x_rows && offsets && preact && h && d_rows && dx_rows && dw1 && dw2 &&
            (w->act != MOE_SWIGLU || dw3),
        MOE_EINVAL, "moe_grouped_ffn_backward: NULL argument");
  CHECK(dw_dt == MOE_F32 || dw_dt == MOE_BF16, MOE_EUNSUPPORTED,
        "moe_grouped_ffn_backward: weight gradients are F32 or BF16");
  s = check_ws(workspace, ws_bytes,
               grouped_ffn_backward_workspace_bytes(w, max_rows, row_index != nullptr),
               "moe_grouped_ffn_backward");
  if (s != MOE_OK) return s;
  return grouped_ffn_backward_launch(w, x_rows, row_index, offsets, max_rows, preact, h, d_rows,
                                     dx_rows, dw1, dw3, dw2, dw_dt, workspace,
                                     (hipStream_t)hip_stream);
}

moe_status moe_combine_backward(int32_t n_tokens, int32_t d_model, int32_t top_k,
                                const float* dy, const void* y_rows, moe_dtype y_dt,
                                const int32_t* row_of, const float* gates, uint16_t* d_rows,
                                float* dgates, uint16_t* d_shared, void* hip_stream) {
  CHECK(n_tokens >= 1 && d_model >= 1 && top_k >= 1 && top_k <= 256, MOE_EINVAL,
        "moe_combine_backward: N=%d d=%d k=%d out of range", n_tokens, d_model, top_k);
  CHECK(dy && y_rows && row_of && gates && d_rows && dgates, MOE_EINVAL,
        "moe_combine_backward: NULL argument");
  CHECK(d_model % 8 == 0, MOE_EUNSUPPORTED, "moe_combine_backward: d_model %d not a multiple of 8",
        d_model);
  CHECK(y_dt == MOE_F32 || y_dt == MOE_BF16, MOE_EUNSUPPORTED,
        "moe_combine_backward: y_rows dtype must be F32 or BF16");
  return combine_backward_launch(n_tokens, d_model, top_k, dy, y_rows, y_dt, row_of, gates,
                                 d_rows, dgates, d_shared, (hipStream_t)hip_stream);
}

size_t moe_router_backward_workspace_bytes(int32_t n_tokens, int32_t d_model,
                                           int32_t n_experts) {
  if (n_tokens <= 0 || d_model <= 0 || n_experts <= 0) return 0;
  return router_backward_workspace_bytes(n_tokens, d_model, n_experts);
}

moe_status moe_router_backward(const moe_router_params* p, const void* x, moe_dtype x_dt,
                               const float* w_gate, const float* logits, const int32_t* cand_ids,
                               const int32_t* expert_of, const int32_t* row_of,
                               const float* dgates, const int32_t* counts_routed, float alpha,
                               float beta, const float* dx_rows, const float* dx_shared,
                               const float* noise_v, float* dlogits, float* dw_gate,
                               float* dlogit_bias, float* dw_noise, float* dx, void* workspace,
                               size_t ws_bytes, void* hip_stream) {
  CHECK(p, MOE_EINVAL, "moe_router_backward: params is NULL");
  const int N = p->n_tokens, d = p->d_model, E = p->n_experts, k = p->top_k, C = p->n_cand;
  CHECK(N >= 1 && d >= 1 && E >= 1 && k >= 1 && C >= k && k <= E, MOE_EINVAL,
        "moe_router_backward: N=%d d=%d E=%d k=%d n_cand=%d out of range", N, d, E, k, C);
  CHECK(E <= 256, MOE_EUNSUPPORTED, "moe_router_backward: n_experts %d > 256", E);
  CHECK(!p->w_noise || (noise_v && dw_noise), MOE_EINVAL,
        "moe_router_backward: noisy gating needs noise_v and dw_noise");
  CHECK(x && w_gate && logits && cand_ids && expert_of && row_of && dgates && counts_routed &&
            dlogits && dw_gate && dx,
        MOE_EINVAL, "moe_router_backward: NULL argument");
  CHECK(x_dt == MOE_F32 || x_dt == MOE_BF16, MOE_EUNSUPPORTED, "moe_router_backward: x dtype");
  CHECK((long long)N * (d > E ? d : E) < (1ll << 40), MOE_EINVAL, "moe_router_backward: too large");
  moe_status s = check_ws(workspace, ws_bytes, router_backward_workspace_bytes(N, d, E),
                          "moe_router_backward");
  if (s != MOE_OK) return s;
  return router_backward_launch(N, d, E, k, C, p->renormalize, x, x_dt, w_gate, logits, cand_ids,
                                expert_of, row_of, dgates, counts_routed, alpha, beta, dx_rows,
                                dx_shared, p->w_noise, noise_v, p->noise_seed, dlogits, dw_gate,
                                dlogit_bias, dw_noise, dx, workspace, (hipStream_t)hip_stream);
}

moe_status moe_combine(int32_t n_tokens, int32_t d_model, int32_t top_k, const void* y_rows,
                       moe_dtype y_dt, const int32_t* row_of, const float* gates,
                       const void* y_shared, moe_dtype sh_dt, void* y, moe_dtype out_dt,
                       void* hip_stream) {
  CHECK(n_tokens >= 1 && d_model >= 1 && top_k >= 1, MOE_EINVAL,
        "moe_combine: N=%d d=%d k=%d out of range", n_tokens, d_model, top_k);
  CHECK(y_rows && row_of && gates && y, MOE_EINVAL, "moe_combine: NULL argument");
  CHECK(top_k <= 256, MOE_EUNSUPPORTED, "moe_combine: top_k %d > 256", top_k);
  CHECK(d_model % 8 == 0, MOE_EUNSUPPORTED, "moe_combine: d_model %d not a multiple of 8", d_model);
  CHECK((y_dt == MOE_F32 || y_dt == MOE_BF16) && (out_dt == MOE_F32 || out_dt == MOE_BF16) &&
            (!y_shared || sh_dt == MOE_F32 || sh_dt == MOE_BF16),
        MOE_EUNSUPPORTED, "moe_combine: dtypes must be F32 or BF16");
  return combine_launch(n_tokens, d_model, top_k, y_rows, y_dt, row_of, gates, y_shared, sh_dt, y,
                        out_dt, (hipStream_t)hip_stream);
}

moe_status moe_expert_choice(int32_t n_tokens, int32_t n_experts, int32_t capacity,
                             const float* scores, int32_t* offsets, int32_t* perm_token,
                             int32_t* row_of, float* gates, int32_t* counts, void* hip_stream) {
  CHECK(n_tokens >= 1 && capacity >= 1, MOE_EINVAL,
        "moe_expert_choice: N=%d capacity=%d out of range", n_tokens, capacity);
  CHECK(n_experts >= 1 && n_experts <= 256, MOE_EINVAL,
        "moe_expert_choice: n_experts %d outside [1, 256]", n_experts);
  const long long cap = capacity < n_tokens ? capacity : n_tokens;
  CHECK((long long)n_tokens * n_experts < (1ll << 31) && cap * n_experts < (1ll << 31),
        MOE_EINVAL, "moe_expert_choice: N*E or E*capacity too large");
  CHECK(scores && offsets && perm_token && row_of && gates, MOE_EINVAL,
        "moe_expert_choice: NULL argument");
  return expert_choice_launch(n_tokens, n_experts, capacity, scores, offsets, perm_token, row_of,
                              gates, counts, (hipStream_t)hip_stream);
}

moe_status moe_balance_stats(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                             const int32_t* counts_routed, const int32_t* counts_kept,
                             const double* score_sums, float* f, float* P, float* scalars,
                             float* select_bias, float bias_rate, void* hip_stream) {
  CHECK(n_tokens >= 1 && n_experts >= 1 && top_k >= 1, MOE_EINVAL,
        "moe_balance_stats: N=%d E=%d k=%d out of range", n_tokens, n_experts, top_k);
  CHECK(counts_routed && counts_kept && score_sums && f && P && scalars, MOE_EINVAL,
        "moe_balance_stats: NULL argument");
  CHECK(n_experts <= 256, MOE_EUNSUPPORTED, "moe_balance_stats: n_experts %d > 256", n_experts);
  return balance_stats_launch(n_tokens, n_experts, top_k, counts_routed, counts_kept, score_sums,
                              f, P, scalars, select_bias, bias_rate, (hipStream_t)hip_stream);
}

}  // extern "C"
