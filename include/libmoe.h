/*
 * libmoe.h -- C ABI of libmoe, the forward pass of one sparse
 * Mixture-of-Experts FFN layer with every expert resident on one MI355X
 * (gfx950) GPU.
 *
 * The layer, as the pages state it: a router scores each token against every
 * expert (dot product with a learned per-expert vector, then a softmax), the
 * token keeps its top-k experts, tokens are bucketed and packed by expert,
 * each expert's FFN runs on its bucket (as one grouped GEMM), and the expert
 * outputs are put back in token order weighted by the router's gate values.
 * Sources: heavensheep.xyz MoE notes, "Routing Function"; mkbk-pku.cn
 * "通信与并行" (router gives expert id and weight alpha, dispatch, bucketize,
 * grouped GEMM, combine back to token order with alpha) and "MOE的优化"
 * (grouped GEMM, bucketize + contiguous packing); chiang97912 MoE notes,
 * "专家选择" (y = sum_i G(x)_i E_i(x)), "KeepTopK 策略", "专家容量".
 *
 * Conventions shared by every call
 *  - All array arguments are DEVICE pointers to memory the caller allocated
 *    and owns (e.g. torch tensors' data_ptr()). libmoe allocates no device
 *    memory and keeps no state between calls; scratch space comes from the
 *    caller's `workspace` (size from the matching *_workspace_bytes query,
 *    alignment 256 bytes) -- except moe_dispatch_noalloc, whose scratch is a
 *    fixed array inside the library (see there). Parameter structs are HOST
 *    memory, read during the call only.
 *  - Layouts are row-major and dense. bf16 is the upper half of an IEEE
 *    binary32; fp8 is OCP E4M3FN (bias 7, max 448, no infinities).
 *  - Every call enqueues its kernels on `hip_stream` (a hipStream_t; NULL is
 *    the default stream) and returns without synchronising: routing counts
 *    and offsets stay on the device.
 *  - Arguments are validated on the host before anything is enqueued. On an
 *    error nothing is enqueued and no output is touched; moe_last_error()
 *    gives a message (per calling thread).
 *      MOE_EINVAL        a required pointer is NULL or a size is out of range
 *      MOE_EUNSUPPORTED  valid but not implemented (limits below)
 *      MOE_EWORKSPACE    workspace NULL or smaller than required
 *      MOE_EHIP          a kernel launch failed; faults inside kernels
 *                        surface at the caller's next synchronisation
 *  - Limits: 1 <= n_experts <= 256, 1 <= top_k <= 8, top_k <= n_experts,
 *    n_tokens * n_cand < 2^31, d_model % 8 == 0 and d_ff % 8 == 0 (16-byte
 *    rows); the bf16 tensor-core path needs d_model % 64 == 0 and
 *    d_ff % 64 == 0. Non-finite inputs are not supported (garbage in).
 *  - Results are deterministic: no atomics decide any value or order.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Expert FFN activation: ReLU and GELU (exact erf form) apply to W1 x + b1;
 * SwiGLU is silu(W1 x) * (W3 x) with w1 the gate and w3 the up projection. */
typedef enum { MOE_RELU = 0, MOE_GELU = 1, MOE_SWIGLU = 2 } moe_act;

/* What happens to an assignment beyond an expert's capacity
 * (mkbk-pku.cn "负载均衡", overflow strategies; chiang97912 "专家容量"):
 *  DROPLESS           no capacity limit;
 *  DROP               the assignment is dropped (gate 0, contributes 0);
 *  REROUTE_THEN_DROP  (top-1 with one spare candidate) after every token's
 *                     first choice is placed, overflowed tokens in ascending
 *                     order try their second candidate once, else drop. */
typedef enum { MOE_DROPLESS = 0, MOE_DROP = 1, MOE_REROUTE_THEN_DROP = 2 } moe_overflow;

/* ---------------------------------------------------------------------- */
/* moe_router_topk                                                         */
/* ---------------------------------------------------------------------- */
/* Router: logits l = x . W_g^T (+ logit_bias); with w_noise, noisy top-k
 * gating H = l + z * softplus(x . W_noise^T) (chiang97912 "KeepTopK 策略"),
 * z a standard-normal draw from a counter hash of (noise_seed, token,
 * expert); then an fp32 softmax (heavensheep "Training": exponentials need
 * the higher precision) and top-k selection ("Routing Function"), keys =
 * score + select_bias (ld246.com Q3: per-expert bias added to the softmax
 * score before top-k). Gates: renormalize ? s_j / sum of the kept s (equal
 * to softmax(KeepTopK(H,k))) : s_j.
 *
 * Numerics, fixed so that integer decisions are reproducible:
 *  - softmax: m = max; d = l - m; u = 0 if d < -87 else exp(d) with a
 *    Cody-Waite reduced, degree-7 Taylor fp32 exponential; S = halving-tree
 *    sum of u padded to a power of two; s = u / S (IEEE divide);
 *  - key ties go to the lower expert index; -0 counts as +0;
 *  - renormalising sum in rank order, fp32.
 */
typedef struct {
  int32_t n_tokens;     /* N >= 1 */
  int32_t d_model;      /* d, % 8 == 0 */
  int32_t n_experts;    /* E in [1, 256] */
  int32_t top_k;        /* k in [1, min(8, E)] */
  int32_t n_cand;       /* candidates kept per token: k, or k+1 for reroute */
  int32_t renormalize;  /* 1: gates renormalised over the k; 0: gate = score */
  const float* logit_bias;  /* [E] added to the logits, or NULL */
  const float* select_bias; /* [E] added to scores for selection only, or NULL */
  const float* w_noise;     /* [E][d] fp32 noise projection, or NULL */
  uint64_t noise_seed;
  float* scores_out;        /* [N][E] fp32 out: every softmax score s_te (the
                               values cand_scores takes them from), or NULL;
                               the input of moe_expert_choice */
  float* noise_out;         /* [N][E] fp32 out with w_noise: v = x.W_noise^T
                               before the softplus (the backward pass's
                               input), or NULL. Not written when logits_in
                               is given (the router computes no logits) */
  const void* w_planes;     /* w_gate (and w_noise) as three bf16 planes from
                               moe_router_prepare, or NULL: then every call
                               splits them into the workspace first. Used
                               when x is bf16 and d % 64 == 0 (the matrix-
                               core router), ignored otherwise; must match
                               w_gate / w_noise (the caller re-prepares after
                               changing them) */
} moe_router_params;

/*  x          [N][d] activations, x_dt = MOE_F32 or MOE_BF16
 *  w_gate     [E][d] fp32 router weights (each expert's vector)
 *  logits_in  [N][E] fp32 or NULL. When set, x, w_gate, logit_bias and
 *             w_noise are ignored and these are the logits the softmax sees.
 *  cand_ids   [N][n_cand] int32 out: experts by descending key
 *  cand_scores[N][n_cand] fp32 out: their unbiased softmax scores
 *  gates      [N][top_k]  fp32 out
 *  logits_out [N][E] fp32 out (the logits the softmax saw), or NULL
 *  score_sums [E+1] fp64 out, or NULL: [e] = sum over tokens of s_te,
 *             [E] = sum over tokens of lse_t^2 (lse = m + ln S). Inputs of
 *             moe_balance_stats. Summed in a fixed order. */
moe_status moe_router_topk(const moe_router_params* p, const void* x, moe_dtype x_dt,
                           const float* w_gate, const float* logits_in, int32_t* cand_ids,
                           float* cand_scores, float* gates, float* logits_out,
                           double* score_sums, void* workspace, size_t ws_bytes,
                           void* hip_stream);
size_t moe_router_workspace_bytes(int32_t n_tokens, int32_t d_model, int32_t n_experts,
                                  int32_t with_noise);

/* The router weights w_gate (rows 0..E-1) and w_noise (rows E..2E-1, if
 * given) as three bf16 planes whose sum is the fp32 weight exactly:
 * hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid), so that the
 * router GEMM with bf16 x runs on bf16 matrix cores with every product
 * exact (the fp32 router of heavensheep "Training": the scores must not be
 * computed in bf16). Layout [3][E2pad][d], E2pad = E (2E with w_noise)
 * rounded up to a multiple of 64, zero rows past the weights; size from
 * moe_router_planes_bytes. The caller owns `planes` and passes it as
 * moe_router_params.w_planes on later calls; libmoe keeps no state.
 * Needs d_model % 64 == 0 and 1 <= n_experts <= 256 (else EINVAL /
 * EUNSUPPORTED), planes_bytes >= moe_router_planes_bytes (else
 * EWORKSPACE), 16-byte aligned planes. Asynchronous on hip_stream. */
size_t moe_router_planes_bytes(int32_t n_experts, int32_t d_model, int32_t with_noise);
moe_status moe_router_prepare(const float* w_gate, const float* w_noise, int32_t n_experts,
                              int32_t d_model, void* planes, size_t planes_bytes,
                              void* hip_stream);

/* ---------------------------------------------------------------------- */
/* moe_dispatch                                                            */
/* ---------------------------------------------------------------------- */
/* Bucketize assignments by expert and pack each expert's tokens
 * contiguously (mkbk-pku.cn "MOE的优化": bucketize + contiguous packing),
 * applying the expert capacity (chiang97912 "专家容量").
 * Order: assignments are taken rank-major -- every token's first choice in
 * ascending token order, then every second choice, ... An assignment whose
 * expert already holds `capacity` assignments overflows (policy above).
 * Rows: offsets = exclusive prefix sum of counts_kept; the assignment's row
 * is offsets[e] + its slot (its position among e's kept assignments).
 *  cand_ids, cand_scores [N][n_cand] from moe_router_topk; an id outside
 *              [0, n_experts) is no candidate (its assignment, or its
 *              reroute, is dropped; it takes no capacity)
 *  gates       [N][top_k] in/out: rerouted -> second candidate's score,
 *              dropped -> 0 (DROPLESS leaves it untouched)
 *  capacity    -1 for DROPLESS, else >= 0 (see moe_capacity)
 *  x           [N][d_model] (x_dt) rows to gather, or NULL with x_perm NULL
 *  counts_routed [E] out: demand of the first top_k candidates (pre-capacity)
 *  counts_kept   [E] out
 *  offsets     [E+1] out, offsets[E] = R = kept assignments
 *  row_of      [N][top_k] out: row in the packed order, -1 if dropped
 *  expert_of   [N][top_k] out: expert actually used, -1 if dropped
 *  perm_token  [N*top_k] out: token of each packed row (first R entries)
 *  x_perm      [N*top_k][d_model] out (x_dt): x rows in packed order (first
 *              R rows), or NULL to skip the gather.
 * REROUTE_THEN_DROP needs top_k == 1 and n_cand == 2 (else EUNSUPPORTED). */
moe_status moe_dispatch(int32_t n_tokens, int32_t n_experts, int32_t top_k, int32_t n_cand,
                        moe_overflow policy, int32_t capacity, const int32_t* cand_ids,
                        const float* cand_scores, float* gates, const void* x, moe_dtype x_dt,
                        int32_t d_model, int32_t* counts_routed, int32_t* counts_kept,
                        int32_t* offsets, int32_t* row_of, int32_t* expert_of,
                        int32_t* perm_token, void* x_perm, void* workspace, size_t ws_bytes,
                        void* hip_stream);
size_t moe_dispatch_workspace_bytes(int32_t n_tokens, int32_t n_experts, int32_t top_k);

/* moe_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as moe_dispatch, without the
 * workspace: its scratch is a fixed device array inside libmoe, one per GPU,
 * MOE_DISPATCH_NOALLOC_SCRATCH_BYTES long and held until the process ends;
 * no call allocates. Sizes whose moe_dispatch_workspace_bytes exceed it are
 * rejected with MOE_EWORKSPACE before any launch (4 MiB covers, e.g., the
 * DeepSeek-shaped 8192 tokens x top-8 over 256 experts, 0.8 MB). Every call
 * on one GPU shares that GPU's array: calls that overlap on the same GPU
 * (other streams, other threads) race; calls in stream order do not (no
 * part of the array has to start at zero). */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_dispatch_noalloc(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                                int32_t n_cand, moe_overflow policy, int32_t capacity,
                                const int32_t* cand_ids, const float* cand_scores, float* gates,
                                const void* x, moe_dtype x_dt, int32_t d_model,
                                int32_t* counts_routed, int32_t* counts_kept, int32_t* offsets,
                                int32_t* row_of, int32_t* expert_of, int32_t* perm_token,
                                void* x_perm, void* hip_stream);

/* capacity = ceil(n_tokens / n_experts * capacity_factor) (chiang97912
 * "专家容量": tokens per batch / number of experts x capacity factor; the
 * rounding up is this library's choice). The factor is the exact fraction
 * cf_num / cf_den (1.25 = 5/4, 1.1 = 11/10), so a decimal factor is never
 * replaced by its nearest binary value; the result is exact integer
 * arithmetic, clamped to INT32_MAX. Expert-choice routing takes
 * moe_capacity(N, E, top_k, 1) = ceil(N * top_k / E) tokens per expert.
 * Returns -1 if n_tokens <= 0, n_experts <= 0, cf_num < 0 or cf_den <= 0.
 * Host function, no GPU work. */
int32_t moe_capacity(int32_t n_tokens, int32_t n_experts, int32_t cf_num, int32_t cf_den);

/* ---------------------------------------------------------------------- */
/* moe_expert_choice                                                       */
/* ---------------------------------------------------------------------- */
/* Expert-choice routing: instead of every token picking its top-k experts,
 * every expert picks its tokens, which balances the load by construction
 * (heavensheep.xyz MoE notes, "Routing Function"; "[CS336-04] Mixture of
 * Experts", section 3). Expert e takes cap = min(capacity, N) tokens: the
 * ones with the largest score s_te, ties to the lower token index; its rows
 * are those tokens in token order, rows e*cap .. e*cap+cap-1. The gate of a
 * chosen (token, expert) pair is s_te; a token no expert chose gets 0 from
 * the combine (the residual is the caller's).
 *  scores     [N][E] fp32 (moe_router_params.scores_out)
 *  offsets    [E+1] int32 out: e * cap
 *  perm_token [E*cap] int32 out: token of each row (row_index of
 *             moe_grouped_ffn)
 *  row_of     [N][E] int32 out: row of (t, e), or -1 (moe_combine with
 *             top_k = E)
 *  gates      [N][E] fp32 out: s_te where chosen, else 0
 *  counts     [E] int32 out (cap each), or NULL
 * Errors: EINVAL for N < 1, capacity < 1, E outside [1, 256], N*E or E*cap
 * of 2^31 or more, or a NULL required pointer. No workspace. */
moe_status moe_expert_choice(int32_t n_tokens, int32_t n_experts, int32_t capacity,
                             const float* scores, int32_t* offsets, int32_t* perm_token,
                             int32_t* row_of, float* gates, int32_t* counts,
                             void* hip_stream);

/* ---------------------------------------------------------------------- */
/* moe_grouped_ffn                                                         */
/* ---------------------------------------------------------------------- */
/* Every expert's FFN on its packed rows, as one grouped GEMM pair
 * (mkbk-pku.cn "MOE的优化", Grouped GEMM): rows offsets[e] .. offsets[e+1]
 * of x_rows go through expert e:
 *   ReLU/GELU: y = W2 act(W1 x + b1) + b2;  SwiGLU: y = W2 (silu(W1 x) * W3 x)
 * The intermediate h is kept in the workspace in bf16, or fp32 when
 * act_dt is MOE_F32 or h_fp32 is set. fp8 weights carry one fp32 scale per output channel (row of
 * W1/W3/W2), applied after the K sum; activations stay bf16 (W8A16).
 * Shared always-on expert: the same call with n_experts = 1,
 * offsets = {0, N}, row_index NULL, on x.
 * Supported: (act_dt, w_dt, y_dt) = (F32, F32, F32), (BF16, BF16, BF16|F32),
 * (BF16, FP8_E4M3, BF16|F32); fp8 weights need SwiGLU or GELU and no bias. */
typedef struct {
  int32_t n_experts, d_model, d_ff;
  moe_act act;
  moe_dtype w_dt;
  const void* w1; /* [E][d_ff][d_model] */
  const void* w3; /* [E][d_ff][d_model], SwiGLU only, else NULL */
  const void* w2; /* [E][d_model][d_ff] */
  const float* b1; /* [E][d_ff] or NULL */
  const float* b2; /* [E][d_model] or NULL */
  const float* s1; /* [E][d_ff] fp8 scales, else NULL */
  const float* s3; /* [E][d_ff] fp8 scales (SwiGLU), else NULL */
  const float* s2; /* [E][d_model] fp8 scales, else NULL */
  /* Precision of the intermediate h between the two GEMMs (bf16 paths):
   * 0 = bf16; 1 = fp32, with GEMM 2 run as two bf16 MFMA passes over the
   * high and low bf16 parts of h (twice the GEMM 2 MFMA work, about 16 more
   * bits of h). Meant for layers bound by weight traffic, where MFMA time is
   * spare. Ignored for the fp32 path (h is fp32 there). */
  int32_t h_fp32;
} moe_ffn_weights;

/*  x_rows    activations (act_dt), row-major with d_model columns: the
 *            packed rows [max_rows][d_model] when row_index is NULL, or any
 *            row set (e.g. the token rows x [N][d_model]) when row_index is
 *            given
 *  row_index [max_rows] device int32 or NULL: packed row r reads
 *            x_rows[row_index[r]] -- pass perm_token from moe_dispatch to
 *            fuse the token gather into GEMM 1's operand loads (the fused
 *            dispatch + GEMM of mkbk-pku.cn "MOE的优化", Fused MoE kernel)
 *  offsets   [E+1] device int32 row offsets (from moe_dispatch); rows past
 *            offsets[E] are not read or written
 *  max_rows  upper bound on offsets[E] used to size the launch (N*top_k)
 *  y_rows    [max_rows][d_model] out (y_dt), in packed row order */
moe_status moe_grouped_ffn(const moe_ffn_weights* w, const void* x_rows, moe_dtype act_dt,
                           const int32_t* row_index, const int32_t* offsets, int32_t max_rows,
                           void* y_rows, moe_dtype y_dt, void* workspace, size_t ws_bytes,
                           void* hip_stream);
size_t moe_grouped_ffn_workspace_bytes(const moe_ffn_weights* w, moe_dtype act_dt,
                                       int32_t max_rows);

/* moe_grouped_ffn followed by moe_combine for top-1 routing without a
 * shared expert, in one call: the combine is done where the expert outputs
 * are made (mkbk-pku.cn "MOE的优化", Fused MoE kernel: no round trip of the
 * expert outputs through memory). With one assignment per token, GEMM 2's
 * epilogue writes fmaf(gates[t], value, 0) straight to y[t] for the token
 * t = perm_token[r] of each packed row r, and the rows of tokens whose
 * assignment was dropped (row_of[t] < 0) are set to 0 -- the same bits
 * moe_combine would produce from y_rows. A first small kernel zeroes the
 * dropped rows and puts each kept gate at its packed row (in the
 * workspace), so the epilogue's gate and token loads do not depend on each
 * other. Arguments as moe_grouped_ffn,
 * plus n_tokens, perm_token [max_rows], row_of [N][1] and gates [N][1]
 * from moe_dispatch (top_k = 1), y [N][d_model] fp32 out instead of
 * y_rows. Needs max_rows <= n_tokens (EINVAL), no fp8 weights and
 * d_model % 4 == 0 (EUNSUPPORTED); perm_token's first offsets[E] entries
 * must be distinct tokens (dispatch's output is). Workspace: as
 * moe_grouped_ffn. */
moe_status moe_grouped_ffn_combine_top1(const moe_ffn_weights* w, const void* x_rows,
                                        moe_dtype act_dt, const int32_t* row_index,
                                        const int32_t* offsets, int32_t max_rows,
                                        int32_t n_tokens, const int32_t* perm_token,
                                        const int32_t* row_of, const float* gates, float* y,
                                        void* workspace, size_t ws_bytes, void* hip_stream);

/* ---------------------------------------------------------------------- */
/* moe_combine                                                             */
/* ---------------------------------------------------------------------- */
/* Back to token order, weighted by the gates (mkbk-pku.cn "通信与并行",
 * combine with alpha; chiang97912 "专家选择": y = sum_i G(x)_i E_i(x)), plus
 * the shared expert's output with gate 1 ("MoE" on ld246.com, Q4):
 *   y[t] = sum over j < top_k with row_of[t][j] >= 0 of
 *          gates[t][j] * y_rows[row_of[t][j]]  (+ y_shared[t]),
 * accumulated in fp32 in rank order, rounded once. A token whose
 * assignments were all dropped gets 0 (+ shared): it skips the layer, the
 * residual add is the caller's.
 *  y_rows [R][d_model] (y_dt), row_of/gates [N][top_k], y_shared [N][d_model]
 *  (sh_dt) or NULL, y [N][d_model] out (out_dt). Dtypes: F32 or BF16.
 *  top_k in [1, 256]: up to 8 for token choice, up to E with the [N][E]
 *  row_of/gates of moe_expert_choice (rows still summed in j order). */
moe_status moe_combine(int32_t n_tokens, int32_t d_model, int32_t top_k, const void* y_rows,
                       moe_dtype y_dt, const int32_t* row_of, const float* gates,
                       const void* y_shared, moe_dtype sh_dt, void* y, moe_dtype out_dt,
                       void* hip_stream);

/* ---------------------------------------------------------------------- */
/* moe_balance_stats                                                       */
/* ---------------------------------------------------------------------- */
/* Load-balance statistics of one forward, computed in fp64:
 *  f[e] = counts_routed[e] / (N k)   fraction of assignments sent to e, and
 *  P[e] = score_sums[e] / N          mean router probability of e
 *                                    (heavensheep "Training": f_i and P_i)
 *  scalars[0] = E * sum_e f_e P_e    Switch aux loss, unscaled (1 when uniform)
 *  scalars[1] = CV^2 of Importance = sum_t G(x_t) (population variance over
 *               mean^2; chiang97912 "辅助损失")
 *  scalars[2] = router z-loss = mean_t lse_t^2 ("[CS336-04]" section 4 names it)
 *  scalars[3] = drop rate = (N k - sum counts_kept) / (N k)
 * With select_bias non-NULL, the loss-free balancing step is applied in
 * place: bias_e -= bias_rate * sign(counts_routed[e] - N k / E), sign(0) = 0
 * (ld246.com Q3 item 2; heavensheep "Training", DeepSeek V3 bias).
 *  counts_*: [E] int32; score_sums [E+1] fp64 from moe_router_topk;
 *  f, P [E] fp32 out; scalars [4] fp32 out. */
moe_status moe_balance_stats(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                             const int32_t* counts_routed, const int32_t* counts_kept,
                             const double* score_sums, float* f, float* P, float* scalars,
                             float* select_bias, float bias_rate, void* hip_stream);

/* ====================================================================== */
/* Training: the layer's backward pass                                     */
/* ====================================================================== */
/* The backward pass differentiates, with the forward's discrete decisions
 * (selected experts, capacity drops) fixed,
 *   L = sum_t <dy_t, y_t> + alpha * switch_aux + beta * z_loss
 * (switch_aux and z_loss as in moe_balance_stats; f_e is a count and gets
 * no gradient). heavensheep.xyz MoE notes, "Training": with top-k routing
 * an unselected expert gets no gradient from the main loss, and the
 * auxiliary loss gives the router a gradient for every expert;
 * mkbk-pku.cn "通信与并行", step 5: gradients go back along the forward's
 * routing path. Order of the calls: moe_combine_backward ->
 * moe_grouped_ffn_backward (routed experts, and the shared expert if any) ->
 * moe_router_backward. Scope: token-choice routing (with or without noisy
 * gating, capacity and reroute) and expert choice; bf16 SwiGLU, ReLU or
 * GELU experts without biases (h kept in bf16); d_model and d_ff multiples
 * of 256. Expert choice runs as E slots per token: row_of [N][E] and the
 * gates [N][E] of moe_expert_choice go to moe_combine_backward with
 * top_k = E, and moe_router_backward takes top_k = n_cand = E,
 * renormalize = 0, cand_ids = expert_of = [N][E] with column j holding j
 * (slot j is expert j; a chosen pair's gate is its score) and
 * counts_routed = the capacity of every expert.
 * Gradients come out in fp32 (expert weight gradients optionally bf16) and
 * overwrite their buffers (no accumulation). */

/* Forward of the routed (or shared) experts that also keeps what the
 * backward needs: as moe_grouped_ffn (bf16 activations), plus
 *  preact [max_rows][2 d_ff] bf16 out (SwiGLU: per packed row the gate
 *         pre-activation a = x W1^T then the up projection u = x W3^T), or
 *         [max_rows][d_ff] (ReLU / GELU: a)
 *  h      [max_rows][d_ff] bf16 out: silu(a) * u or act(a), the operand of
 *         GEMM 2
 * Rows past offsets[E] are untouched. Workspace: moe_grouped_ffn's. */
moe_status moe_grouped_ffn_train(const moe_ffn_weights* w, const void* x_rows,
                                 const int32_t* row_index, const int32_t* offsets,
                                 int32_t max_rows, void* y_rows, moe_dtype y_dt,
                                 uint16_t* preact, uint16_t* h, void* workspace, size_t ws_bytes,
                                 void* hip_stream);

/* Backward of the gate-weighted combine y_t = sum_j g_tj o_{row_of[t][j]}
 * (+ the shared expert's output with gate 1):
 *  dy     [N][d] fp32 upstream gradient
 *  y_rows [R][d] (y_dt F32 or BF16) the expert outputs o of the forward
 *  row_of, gates [N][k] as given to moe_combine
 *  d_rows [R][d] bf16 out: g_tj * dy_t on the row of each kept slot
 *  dgates [N][k] fp32 out: <dy_t, o_row>, 0 for a dropped slot
 *  d_shared [N][d] bf16 out (dy rounded: the shared expert's output
 *           gradient) or NULL without a shared expert
 * Deterministic (fixed reduction order). */
moe_status moe_combine_backward(int32_t n_tokens, int32_t d_model, int32_t top_k,
                                const float* dy, const void* y_rows, moe_dtype y_dt,
                                const int32_t* row_of, const float* gates, uint16_t* d_rows,
                                float* dgates, uint16_t* d_shared, void* hip_stream);

/* Backward of the grouped expert FFN. The shared expert is the same call
 * with one expert, offsets {0, N}, row_index NULL and d_rows =
 * moe_combine_backward's d_shared. Per expert e over its packed rows
 * (a = x W1^T, u = x W3^T, h = silu(a) u, o = h W2^T):
 *  dh = dO W2; da = dh u silu'(a); du = dh silu(a); dX = da W1 + du W3;
 *  dW2_e = sum_r dO_r^T h_r; dW1_e = sum_r da_r^T x_r; dW3_e = sum_r du_r^T x_r.
 *  ReLU / GELU (h = act(a)): da = dh act'(a), dX = da W1, no dW3 (dw3 may be
 *  NULL); GELU' = Phi(a) + a phi(a) (exact erf form).
 *  x_rows, row_index, offsets, max_rows: as given to moe_grouped_ffn_train
 *  preact, h: what moe_grouped_ffn_train saved
 *  d_rows [R][d] bf16: dO (moe_combine_backward's d_rows)
 *  dx_rows [max_rows][d] fp32 out: dX per packed row (rows >= offsets[E]
 *          untouched)
 *  dw1, dw3 [E][d_ff][d], dw2 [E][d][d_ff] out in dw_dt (F32, or BF16:
 *          the fp32 sums rounded once; every element written, zero for an
 *          expert without rows)
 * Workspace: moe_grouped_ffn_backward_workspace_bytes(w, max_rows,
 * row_index != NULL). bf16 MFMA products with fp32 accumulation; the
 * intermediate da, du are bf16. */
size_t moe_grouped_ffn_backward_workspace_bytes(const moe_ffn_weights* w, int32_t max_rows,
                                                int32_t gather);
moe_status moe_grouped_ffn_backward(const moe_ffn_weights* w, const void* x_rows,
                                    const int32_t* row_index, const int32_t* offsets,
                                    int32_t max_rows, const uint16_t* preact, const uint16_t* h,
                                    const uint16_t* d_rows, float* dx_rows, void* dw1, void* dw3,
                                    void* dw2, moe_dtype dw_dt, void* workspace, size_t ws_bytes,
                                    void* hip_stream);

/* Backward of the router (chiang97912 "KeepTopK 策略": gates renormalised
 * over the kept k, noisy logits H(x); "[CS336-04]" section 4: z-loss); it
 * also assembles the token gradient dx. Per token, with s the softmax of
 * the logits the forward's softmax saw:
 *  renormalised gates: ds_{c_j} = (dg_j - sum_i dg_i g_i) / sum_i s_{c_i}
 *  Switch gate (renormalize = 0): ds_e += dg_j for the expert used
 *  auxiliary: ds_te += alpha E f_e / N, f_e = counts_routed[e] / (N k)
 *  dl_te = s_te (ds_te - sum_e s_te ds_te) + beta 2 lse_t s_te / N
 *  noise (p->w_noise set): dv_te = dl_te z_te sigmoid(v_te) (1 for v > 20),
 *  dW_noise = dv^T x
 *  dW_g = dl^T x; dlogit_bias = sum_t dl_t; dx_t = sum over the token's
 *  kept slots j (in order) of dx_rows[row_of[t][j]] + dx_shared[t]
 *  + dl_t W_g + dv_t W_noise.
 *  p: n_tokens, d_model, n_experts, top_k, n_cand, renormalize, w_noise and
 *     noise_seed as in the forward
 *  logits [N][E] fp32: the forward's logits_out; cand_ids [N][n_cand],
 *  expert_of, row_of [N][k], counts_routed [E]: the forward's
 *  dgates [N][k] from moe_combine_backward; dx_rows from
 *  moe_grouped_ffn_backward or NULL (router part only); dx_shared [N][d]
 *  fp32 (the shared expert's moe_grouped_ffn_backward) or NULL; noise_v
 *  [N][E] fp32 (the forward's noise_out) with noise, else NULL
 *  dlogits [N][E], dw_gate [E][d], dlogit_bias [E] (or NULL), dw_noise
 *  [E][d] (with noise, else NULL), dx [N][d]: fp32 out. Deterministic.
 *  Workspace: moe_router_backward_workspace_bytes. */
size_t moe_router_backward_workspace_bytes(int32_t n_tokens, int32_t d_model,
                                           int32_t n_experts);
moe_status moe_router_backward(const moe_router_params* p, const void* x, moe_dtype x_dt,
                               const float* w_gate, const float* logits, const int32_t* cand_ids,
                               const int32_t* expert_of, const int32_t* row_of,
                               const float* dgates, const int32_t* counts_routed, float alpha,
                               float beta, const float* dx_rows, const float* dx_shared,
                               const float* noise_v, float* dlogits, float* dw_gate,
                               float* dlogit_bias, float* dw_noise, float* dx, void* workspace,
                               size_t ws_bytes, void* hip_stream);

/* ---------------------------------------------------------------------- */
/* Helpers                                                                 */
/* ---------------------------------------------------------------------- */
/* Largest workspace any call of one layer forward needs. */
size_t moe_workspace_bytes(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                           int32_t d_model, int32_t d_ff);
const char* moe_status_string(moe_status s);
/* Message of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_H */
