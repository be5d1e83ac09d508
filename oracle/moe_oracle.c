/*
 * moe_oracle.c -- plain, slow CPU oracle for the forward pass of one sparse
 * Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, calls or
 * loads this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header or constant table with the GPU
 * path: every formula here is written out from the pages' statement of the
 * method and from the number-format definitions.
 *
 * What it follows (page title, section):
 *  - Router = a learned vector per expert, dot product with the token, then a
 *    softmax, then keep the top-k experts ("heavensheep MoE notes", section
 *    "Routing Function"; "MoE" on ld246.com, Q1: router is FFN + softmax;
 *    chiang97912 "混合专家模型笔记", section "专家选择": G(x)=softmax(x.W_g)).
 *  - The softmax is kept in fp32 because bf16 round-off of shifted logits
 *    distorts scores ("heavensheep", section "Training", the 10-logit example).
 *  - Noisy gating H = x.W_g + StandardNormal() * Softplus(x.W_noise), and
 *    KeepTopK then softmax (chiang97912, section "KeepTopK 策略").
 *  - Per-expert selection bias added to scores before top-k, moved against
 *    load (ld246.com Q3 item 2; heavensheep "Training", DeepSeek V3 bias).
 *  - Expert capacity = tokens/experts x capacity factor; overflow goes to the
 *    next candidate, else the token skips the layer (chiang97912, section
 *    "专家容量"); dropped tokens output zero (mkbk-pku.cn, "负载均衡",
 *    overflow strategies).
 *  - y = sum_i G(x)_i E_i(x) (chiang97912, section "专家选择").
 *  - Shared always-on experts ("MoE" on ld246.com, Q4; heavensheep "Routing
 *    Function", last paragraph).
 *  - Switch aux loss from f_i and P_i (heavensheep, section "Training");
 *    importance and CV^2 (chiang97912, section "辅助损失"); router z-loss
 *    named in "[CS336-04] Mixture of Experts", section 4.
 *
 * Precision: routing in fp32 with a fully specified operation order (so its
 * integer decisions are reproducible); logits, FFNs, combine and statistics
 * accumulate in fp64. Build with -ffp-contract=off so no multiply-add is
 * fused behind the code's back.
 *
 * Parity pins: every function here is pinned by the CPU tests against closed
 * forms, the pages' worked softmax example, library routines or brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2

#define ORC_RELU 0
#define ORC_GELU 1
#define ORC_SWIGLU 2

#define ORC_DROPLESS 0
#define ORC_DROP 1
#define ORC_REROUTE 2

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the top 16 bits of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, S.1111.111 is NaN. Exponent field 0 is subnormal:
 * m/8 * 2^-6. */
double orc_e4m3_to_f64(uint8_t q) {
    int s = (q >> 7) & 1;
    int e = (q >> 3) & 15;
    int m = q & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

static double load_val(const void* p, int dt, size_t i) {
    if (dt == ORC_F32) return (double)((const float*)p)[i];
    if (dt == ORC_BF16) return (double)orc_bf16_to_f32(((const uint16_t*)p)[i]);
    return orc_e4m3_to_f64(((const uint8_t*)p)[i]);
}

/* ------------------------------------------------------------------ */
/* fp32 exponential for the softmax                                    */
/* ------------------------------------------------------------------ */
/* Cody & Waite range reduction (Software Manual for the Elementary
 * Functions, 1980): x = n*ln2 + r with n = nearest integer to x*log2(e) and
 * ln2 split into a short high part (exact products n*hi) and a low part;
 * e^r by its Taylor series to degree 7 (|r| <= ln2/2, truncation < 0.1 ulp)
 * in Horner form with explicit fused multiply-adds; then scaling by 2^n by
 * building the exponent bits. Valid for x in [-87, 0], where 2^n stays
 * normal. Coefficients are 1/i! rounded to fp32 from double. */
float orc_exp_spec(float x) {
    const float log2e = 1.44269504088896341f;
    const float ln2_hi = 0.693359375f;            /* 355/512 */
    const float ln2_lo = -2.12194440054690583e-4f; /* ln2 - 355/512 */
    const float c7 = (float)(1.0 / 5040.0);
    const float c6 = (float)(1.0 / 720.0);
    const float c5 = (float)(1.0 / 120.0);
    const float c4 = (float)(1.0 / 24.0);
    const float c3 = (float)(1.0 / 6.0);
    const float c2 = 0.5f;
    const float c1 = 1.0f;
    const float c0 = 1.0f;
    float t = x * log2e;
    float n = rintf(t);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = c7;
    p = fmaf(p, r, c6);
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, c2);
    p = fmaf(p, r, c1);
    p = fmaf(p, r, c0);
    int ni = (int)n;
    uint32_t bits = (uint32_t)(ni + 127) << 23;
    float two_n;
    memcpy(&two_n, &bits, 4);
    return p * two_n;
}

/* Max-subtracted softmax over one token's E logits, fp32 throughout:
 *   m = max_e l_e;  d_e = l_e - m;  u_e = 0 if d_e < -87 else exp(d_e);
 *   S = halving-tree sum of u padded with zeros to a power of two
 *       (a_i += a_{i+h} for h = P/2, P/4, ..., 1);
 *   s_e = u_e / S (IEEE division).
 * Also returns m and S. */
void orc_softmax_spec(const float* l, int E, float* s, float* m_out, float* S_out) {
    float m = l[0];
    for (int e = 1; e < E; ++e)
        if (l[e] > m) m = l[e];
    int P = 1;
    while (P < E) P <<= 1;
    float* a = (float*)calloc((size_t)P, sizeof(float));
    float* u = (float*)malloc(sizeof(float) * (size_t)E);
    for (int e = 0; e < E; ++e) {
        float d = l[e] - m;
        u[e] = (d < -87.0f) ? 0.0f : orc_exp_spec(d);
        a[e] = u[e];
    }
    for (int h = P / 2; h >= 1; h /= 2)
        for (int i = 0; i < h; ++i) a[i] = a[i] + a[i + h];
    float S = a[0];
    for (int e = 0; e < E; ++e) s[e] = u[e] / S;
    if (m_out) *m_out = m;
    if (S_out) *S_out = S;
    free(a);
    free(u);
}

/* ------------------------------------------------------------------ */
/* Counter-based standard normal for noisy gating                      */
/* ------------------------------------------------------------------ */
/* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): one step of the generator whose state is x,
 * i.e. advance by the golden gamma then apply the mixing function. */
uint64_t orc_splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Irwin-Hall approximation of N(0,1): the sum of 12 independent U(0,1) has
 * mean 6 and variance 1. Each uniform is the top 24 bits of one SplitMix64
 * output on counter c*12+i, c = t*E + e. The integer sum is exact; one
 * rounding to fp32 at the end. */
float orc_hash_normal(uint64_t seed, int64_t t, int32_t e, int32_t E) {
    uint64_t c = (uint64_t)t * (uint64_t)E + (uint64_t)e;
    int64_t S = 0;
    for (int i = 0; i < 12; ++i) {
        uint64_t w = orc_splitmix64(seed ^ (c * 12ull + (uint64_t)i));
        S += (int64_t)(w >> 40);
    }
    double v = (double)(S - 6ll * 16777216ll) * (1.0 / 16777216.0);
    return (float)v;
}

/* z[t][e] for t < N, e < E (used to pin the generator's statistics). */
void orc_hash_normal_grid(uint64_t seed, int N, int E, float* z) {
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < N; ++t)
        for (int e = 0; e < E; ++e) z[(size_t)t * E + e] = orc_hash_normal(seed, t, e, E);
}

/* ------------------------------------------------------------------ */
/* Router logits                                                       */
/* ------------------------------------------------------------------ */
/* l[t][e] = fp32( sum_i x[t][i]*Wg[e][i] ) accumulated in fp64, then
 * + logit_bias[e] in fp32. With w_noise (noisy top-k gating):
 *   v = fp32(sum x*Wn) in fp64;  sp = fp32(softplus(v)) computed in fp64
 *   (v itself when v > 20);  z = hash normal(seed, t, e);
 *   H = fma(z, sp, l) in fp32.
 * token_ids (optional) gives each row's index in the full batch (the noise
 * counter); raw_out (optional) receives l before noise. */
void orc_router_logits(int N, int d, int E, const void* x, int x_dt, const float* wg,
                       const float* logit_bias, const float* w_noise, uint64_t noise_seed,
                       const int32_t* token_ids, float* H_out, float* raw_out) {
    #pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(static)
        for (int t = 0; t < N; ++t) {
            /* token index for the noise counter: position in the full batch */
            int64_t tok = token_ids ? (int64_t)token_ids[t] : (int64_t)t;
            for (int i = 0; i < d; ++i) xr[i] = load_val(x, x_dt, (size_t)t * d + i);
            for (int e = 0; e < E; ++e) {
                double acc = 0.0;
                const float* w = wg + (size_t)e * d;
                for (int i = 0; i < d; ++i) acc += xr[i] * (double)w[i];
                float l = (float)acc;
                if (logit_bias) l = l + logit_bias[e];
                if (raw_out) raw_out[(size_t)t * E + e] = l;
                if (w_noise) {
                    double av = 0.0;
                    const float* wn = w_noise + (size_t)e * d;
                    for (int i = 0; i < d; ++i) av += xr[i] * (double)wn[i];
                    float v = (float)av;
                    float sp = (v > 20.0f) ? v : (float)log1p(exp((double)v));
                    float z = orc_hash_normal(noise_seed, tok, e, E);
                    l = fmaf(z, sp, l);
                }
                H_out[(size_t)t * E + e] = l;
            }
        }
        free(xr);
    }
}

/* ------------------------------------------------------------------ */
/* Routing: softmax, selection, gates                                  */
/* ------------------------------------------------------------------ */
/* Per token: s = softmax_spec(l); key_e = s_e + select_bias[e] (fp32; -0
 * counts as +0); candidates = the C experts with the largest key, ties to
 * the lower expert index; cand_s = the unbiased s of each candidate.
 * Gates for the first k candidates: renormalize ? s_j / S_k with
 * S_k = ((s_0 + s_1) + ...) in rank order (KeepTopK then softmax equals
 * this) : s_j.
 * s_out [N][E] and lse_out [N] (fp64 log-sum-exp of the fp32 logits) are
 * optional. */
void orc_route(int N, int E, int k, int C, int renormalize, const float* logits,
               const float* select_bias, float* s_out, int32_t* cand, float* cand_s,
               float* gates, double* lse_out) {
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < N; ++t) {
        const float* l = logits + (size_t)t * E;
        float* s = (float*)malloc(sizeof(float) * (size_t)E);
        float* key = (float*)malloc(sizeof(float) * (size_t)E);
        char* taken = (char*)calloc((size_t)E, 1);
        orc_softmax_spec(l, E, s, NULL, NULL);
        for (int e = 0; e < E; ++e) {
            float kv = select_bias ? s[e] + select_bias[e] : s[e];
            key[e] = (kv == 0.0f) ? 0.0f : kv;
        }
        for (int j = 0; j < C; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e;  /* strict: ties keep lower index */
            }
            taken[best] = 1;
            cand[(size_t)t * C + j] = best;
            cand_s[(size_t)t * C + j] = s[best];
        }
        if (renormalize) {
            float Sk = cand_s[(size_t)t * C];
            for (int j = 1; j < k; ++j) Sk = Sk + cand_s[(size_t)t * C + j];
            for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = cand_s[(size_t)t * C + j] / Sk;
        } else {
            for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = cand_s[(size_t)t * C + j];
        }
        if (s_out) memcpy(s_out + (size_t)t * E, s, sizeof(float) * (size_t)E);
        if (lse_out) {
            double m = (double)l[0];
            for (int e = 1; e < E; ++e)
                if ((double)l[e] > m) m = (double)l[e];
            double acc = 0.0;
            for (int e = 0; e < E; ++e) acc += exp((double)l[e] - m);
            lse_out[t] = m + log(acc);
        }
        free(s);
        free(key);
        free(taken);
    }
}

/* ------------------------------------------------------------------ */
/* Dispatch: capacity, overflow, slots, rows                           */
/* ------------------------------------------------------------------ */
/* Walk the assignments (rank j, token t) with j outer and t inner. For
 * expert e = cand[t][j]: if it has room (dropless, or fewer than `cap`
 * assignments so far) the assignment takes the next slot; otherwise it
 * overflows. Policy DROP: overflowed assignments are dropped (gate 0).
 * Policy REROUTE (top-1 with one spare candidate): the overflowed tokens, in
 * ascending order, try their second candidate the same way, taking its
 * score as the gate; if that is full too the token is dropped.
 * Rows: offsets = exclusive prefix sum of kept counts; row = offsets[e] +
 * slot; perm_token[row] = t. Dropped assignments get row -1, expert -1.
 * counts_routed = demand of the first k candidates before capacity.
 * Returns the number of kept assignments R. */
int orc_dispatch(int N, int E, int k, int C, int policy, int cap, const int32_t* cand,
                 const float* cand_s, float* gates, int32_t* counts_routed,
                 int32_t* counts_kept, int32_t* offsets, int32_t* row_of,
                 int32_t* expert_of, int32_t* perm_token) {
    int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * k);
    int32_t* cnt = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int e = 0; e < E; ++e) counts_routed[e] = 0;
    for (int j = 0; j < k; ++j) {
        for (int t = 0; t < N; ++t) {
            int e = cand[(size_t)t * C + j];
            size_t a = (size_t)t * k + j;
            counts_routed[e] += 1;
            if (policy == ORC_DROPLESS || cnt[e] < cap) {
                slot[a] = cnt[e]++;
                expert_of[a] = e;
            } else {
                slot[a] = -1;
                expert_of[a] = -1;
            }
        }
    }
    if (policy == ORC_REROUTE) {
        for (int t = 0; t < N; ++t) {
            size_t a = (size_t)t * k;  /* top-1: the only rank */
            if (slot[a] >= 0) continue;
            int e2 = cand[(size_t)t * C + 1];
            if (cnt[e2] < cap) {
                slot[a] = cnt[e2]++;
                expert_of[a] = e2;
                gates[a] = cand_s[(size_t)t * C + 1];
            } else {
                gates[a] = 0.0f;
            }
        }
    } else if (policy == ORC_DROP) {
        for (size_t a = 0; a < (size_t)N * k; ++a)
            if (slot[a] < 0) gates[a] = 0.0f;
    }
    int R = 0;
    for (int e = 0; e < E; ++e) {
        counts_kept[e] = cnt[e];
        offsets[e] = R;
        R += cnt[e];
    }
    offsets[E] = R;
    for (int t = 0; t < N; ++t) {
        for (int j = 0; j < k; ++j) {
            size_t a = (size_t)t * k + j;
            if (slot[a] >= 0) {
                int row = offsets[expert_of[a]] + slot[a];
                row_of[a] = row;
                perm_token[row] = t;
            } else {
                row_of[a] = -1;
            }
        }
    }
    free(slot);
    free(cnt);
    return R;
}

/* ------------------------------------------------------------------ */
/* Expert FFN in fp64                                                  */
/* ------------------------------------------------------------------ */
static double act_f64(int act, double a) {
    if (act == ORC_RELU) return a > 0.0 ? a : 0.0;
    /* GELU, exact erf form: 0.5 a (1 + erf(a / sqrt 2)) */
    return 0.5 * a * (1.0 + erf(a / sqrt(2.0)));
}

static double silu_f64(double a) { return a / (1.0 + exp(-a)); }

/* One expert's FFN on n rows X [n][d] (fp64):
 *   ReLU/GELU: y = W2 act(W1 x + b1) + b2
 *   SwiGLU:    y = W2 (silu(W1 x) * (W3 x))
 * W1, W3 are [f][d], W2 is [d][f] (each row is one output channel). fp8
 * weights carry one fp32 scale per output channel (row): w = code * scale.
 * b1 [f], b2 [d] optional (NULL). Y [n][d] fp64. */
void orc_expert_ffn(int n, int d, int f, int act, int w_dt, const double* X,
                    const void* w1, const void* w3, const void* w2, const float* b1,
                    const float* b2, const float* s1, const float* s3, const float* s2,
                    double* Y) {
    double* H = (double*)malloc(sizeof(double) * (size_t)n * f);
    #pragma omp parallel
    {
        double* wa = (double*)malloc(sizeof(double) * (size_t)(d > f ? d : f));
        double* wb = (double*)malloc(sizeof(double) * (size_t)d);
        /* hidden layer: one output channel (row of W1, W3) at a time */
        #pragma omp for schedule(static)
        for (int o = 0; o < f; ++o) {
            for (int i = 0; i < d; ++i) wa[i] = load_val(w1, w_dt, (size_t)o * d + i);
            if (act == ORC_SWIGLU)
                for (int i = 0; i < d; ++i) wb[i] = load_val(w3, w_dt, (size_t)o * d + i);
            for (int r = 0; r < n; ++r) {
                const double* x = X + (size_t)r * d;
                double a = 0.0;
                for (int i = 0; i < d; ++i) a += wa[i] * x[i];
                if (w_dt == ORC_FP8) a *= (double)s1[o];
                if (b1) a += (double)b1[o];
                if (act == ORC_SWIGLU) {
                    double g = 0.0;
                    for (int i = 0; i < d; ++i) g += wb[i] * x[i];
                    if (w_dt == ORC_FP8) g *= (double)s3[o];
                    H[(size_t)r * f + o] = silu_f64(a) * g;
                } else {
                    H[(size_t)r * f + o] = act_f64(act, a);
                }
            }
        }
        /* output layer: one output channel (row of W2) at a time */
        #pragma omp for schedule(static)
        for (int o = 0; o < d; ++o) {
            for (int i = 0; i < f; ++i) wa[i] = load_val(w2, w_dt, (size_t)o * f + i);
            for (int r = 0; r < n; ++r) {
                const double* h = H + (size_t)r * f;
                double a = 0.0;
                for (int i = 0; i < f; ++i) a += wa[i] * h[i];
                if (w_dt == ORC_FP8) a *= (double)s2[o];
                if (b2) a += (double)b2[o];
                Y[(size_t)r * d + o] = a;
            }
        }
        free(wa);
        free(wb);
    }
    free(H);
}

/* ------------------------------------------------------------------ */
/* Combine                                                             */
/* ------------------------------------------------------------------ */
/* y_t = sum over kept ranks j of gate[t][j] * Yexp[t][j] + Ysh[t] (fp64).
 * Yexp [N][k][d] holds each assignment's expert output (its values are
 * ignored for dropped assignments, row_of = -1). Ysh [N][d] optional. */
void orc_combine(int N, int d, int k, const int32_t* row_of, const float* gates,
                 const double* Yexp, const double* Ysh, double* y) {
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < N; ++t) {
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                size_t a = (size_t)t * k + j;
                if (row_of[a] < 0) continue;
                acc += (double)gates[a] * Yexp[a * (size_t)d + i];
            }
            if (Ysh) acc += Ysh[(size_t)t * d + i];
            y[(size_t)t * d + i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Balance statistics                                                  */
/* ------------------------------------------------------------------ */
/* f_e = routed_e / (N k)             fraction of assignments sent to e
 * P_e = (1/N) sum_t s_te             mean router probability of e
 * switch_aux = E * sum_e f_e P_e     (1 under perfectly uniform routing)
 * I_e = sum_t s_te, CV^2 = var_pop(I) / mean(I)^2
 * z_loss = (1/N) sum_t lse_t^2
 * drop_rate = (N k - sum kept) / (N k)
 * scalars = {switch_aux, importance_cv2, z_loss, drop_rate}. fp64. */
void orc_balance_stats(int N, int E, int k, const int32_t* routed, const int32_t* kept,
                       const float* s, const double* lse, double* f, double* P,
                       double* scalars) {
    double nk = (double)N * (double)k;
    double aux = 0.0, sum_kept = 0.0;
    double* I = (double*)calloc((size_t)E, sizeof(double));
    for (int t = 0; t < N; ++t)
        for (int e = 0; e < E; ++e) I[e] += (double)s[(size_t)t * E + e];
    for (int e = 0; e < E; ++e) {
        f[e] = (double)routed[e] / nk;
        P[e] = I[e] / (double)N;
        aux += f[e] * P[e];
        sum_kept += (double)kept[e];
    }
    double mean = 0.0;
    for (int e = 0; e < E; ++e) mean += I[e];
    mean /= (double)E;
    double var = 0.0;
    for (int e = 0; e < E; ++e) var += (I[e] - mean) * (I[e] - mean);
    var /= (double)E;
    double z = 0.0;
    for (int t = 0; t < N; ++t) z += lse[t] * lse[t];
    scalars[0] = (double)E * aux;
    scalars[1] = var / (mean * mean);
    scalars[2] = z / (double)N;
    scalars[3] = (nk - sum_kept) / nk;
    free(I);
}

/* Loss-free balancing bias step: an over-used expert's bias goes down, an
 * idle one's goes up: b_e <- b_e - rate * sign(routed_e - N k / E), sign(0)=0,
 * in fp32. The comparison is done in integers: routed_e * E vs N * k. */
void orc_bias_update(int N, int E, int k, const int32_t* routed, float* bias, float rate) {
    int64_t target = (int64_t)N * k;
    for (int e = 0; e < E; ++e) {
        int64_t load = (int64_t)routed[e] * E;
        if (load > target) bias[e] = bias[e] - rate;
        else if (load < target) bias[e] = bias[e] + rate;
    }
}
