"""CPU oracle for the sparse MoE FFN layer forward -- TEST INFRASTRUCTURE.

Only the tests, `__graft_entry__.smoke()` and the benchmark's `cpu_baseline`
leg may import this package. The product library (sparse_mixture_experts_47_amd)
never imports it and shares no code with it.

The arithmetic lives in `moe_oracle.c` (plain C, gcc -O2 -ffp-contract=off,
OpenMP over independent rows); this module compiles it, loads it with ctypes
and composes the layer forward from its steps in the pages' order:
router logits -> fp32 softmax -> top-k selection -> gates -> dispatch with
capacity -> per-expert FFN (fp64) -> gate-weighted combine (+ shared expert)
-> balance statistics.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD_DIR, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, FP8 = 0, 1, 2
RELU, GELU, SWIGLU = 0, 1, 2
DROPLESS, DROP, REROUTE = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/_build/libmoe_oracle.so."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_SO)
            P = ctypes.c_void_p
            i32, u64, f32 = ctypes.c_int, ctypes.c_uint64, ctypes.c_float
            L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
            L.orc_bf16_to_f32.restype = f32
            L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
            L.orc_e4m3_to_f64.restype = ctypes.c_double
            L.orc_exp_spec.argtypes = [f32]
            L.orc_exp_spec.restype = f32
            L.orc_softmax_spec.argtypes = [P, i32, P, P, P]
            L.orc_splitmix64.argtypes = [u64]
            L.orc_splitmix64.restype = u64
            L.orc_hash_normal.argtypes = [u64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
            L.orc_hash_normal.restype = f32
            L.orc_hash_normal_grid.argtypes = [u64, i32, i32, P]
            L.orc_router_logits.argtypes = [i32, i32, i32, P, i32, P, P, P, u64, P, P, P]
            L.orc_route.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
            L.orc_dispatch.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
            L.orc_dispatch.restype = i32
            L.orc_expert_ffn.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
            L.orc_combine.argtypes = [i32, i32, i32, P, P, P, P, P]
            L.orc_balance_stats.argtypes = [i32, i32, i32, P, P, P, P, P, P, P]
            L.orc_bias_update.argtypes = [i32, i32, i32, P, P, f32]
            _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_bf16_to_f32(int(b)) for b in flat], dtype=np.float32).reshape(
        np.shape(bits))


def e4m3_to_f64(codes) -> np.ndarray:
    L = lib()
    flat = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e4m3_to_f64(int(q)) for q in flat]).reshape(np.shape(codes))


def exp_spec(x) -> np.ndarray:
    L = lib()
    flat = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.orc_exp_spec(float(v)) for v in flat], dtype=np.float32).reshape(
        np.shape(x))


def softmax_spec(l):
    """One token's fp32 softmax: returns (s, m, S)."""
    l = _c(l, np.float32)
    s = np.empty_like(l)
    m = np.zeros(1, np.float32)
    S = np.zeros(1, np.float32)
    lib().orc_softmax_spec(_p(l), l.shape[0], _p(s), _p(m), _p(S))
    return s, float(m[0]), float(S[0])


def splitmix64(x: int) -> int:
    return int(lib().orc_splitmix64(x))


def hash_normal(seed: int, t: int, e: int, E: int) -> float:
    return float(lib().orc_hash_normal(seed, t, e, E))


def hash_normal_grid(seed: int, N: int, E: int) -> np.ndarray:
    z = np.empty((N, E), np.float32)
    lib().orc_hash_normal_grid(seed, N, E, _p(z))
    return z


# ---------------------------------------------------------------- routing
def _x_arg(x: np.ndarray, x_dt: int):
    if x_dt == BF16:
        return _c(x, np.uint16)
    return _c(x, np.float32)


def router_logits(x, x_dt, w_gate, logit_bias=None, w_noise=None, noise_seed=0, token_ids=None):
    """Returns (H, raw): logits the softmax sees, and the logits before noise.
    token_ids: each row's token index in the full batch (noise counter)."""
    x = _x_arg(x, x_dt)
    N, d = x.shape
    wg = _c(w_gate, np.float32)
    E = wg.shape[0]
    H = np.empty((N, E), np.float32)
    raw = np.empty((N, E), np.float32)
    lib().orc_router_logits(N, d, E, _p(x), x_dt, _p(wg), _p(_c(logit_bias, np.float32)),
                            _p(_c(w_noise, np.float32)), int(noise_seed),
                            _p(_c(token_ids, np.int32)), _p(H), _p(raw))
    return H, raw


def route(logits, top_k, n_cand, renormalize, select_bias=None):
    """Returns dict(s, cand_ids, cand_scores, gates, lse)."""
    l = _c(logits, np.float32)
    N, E = l.shape
    s = np.empty((N, E), np.float32)
    cand = np.empty((N, n_cand), np.int32)
    cand_s = np.empty((N, n_cand), np.float32)
    gates = np.empty((N, top_k), np.float32)
    lse = np.empty(N, np.float64)
    lib().orc_route(N, E, top_k, n_cand, int(bool(renormalize)), _p(l),
                    _p(_c(select_bias, np.float32)), _p(s), _p(cand), _p(cand_s), _p(gates),
                    _p(lse))
    return dict(s=s, cand_ids=cand, cand_scores=cand_s, gates=gates, lse=lse)


def capacity(n_tokens, n_experts, capacity_factor):
    """Expert capacity: (tokens per batch / number of experts) x capacity
    factor, rounded up (chiang97912 MoE notes, section "专家容量"; the page
    gives no rounding, the upward one is this library's reading). Exact
    rational arithmetic: a float factor is taken as the decimal it prints as
    (1.25 is 5/4, 1.1 is 11/10), never as its binary approximation, so the
    one rounding is the ceiling itself. None means dropless: -1."""
    if capacity_factor is None:
        return -1
    f = Fraction(repr(capacity_factor)) if isinstance(capacity_factor, float) else \
        Fraction(capacity_factor)
    q = Fraction(int(n_tokens)) / int(n_experts) * f
    return -((-q.numerator) // q.denominator)  # ceiling of a fraction


def expert_choice_capacity(n_tokens, n_experts, top_k):
    """Tokens per expert under expert-choice routing: the number that gives
    every expert the average load of top-k token choice, N*k/E, rounded up
    (the rounding is this library's reading)."""
    return capacity(n_tokens, n_experts, int(top_k))


def expert_choice(s, capacity):
    """Expert-choice routing (heavensheep "Routing Function": experts choose
    tokens, which balances the load by construction; "[CS336-04] Mixture of
    Experts" section 3: the routing can be reversed so that experts select
    tokens). Plain definition: expert e takes the min(capacity, N) tokens
    with the largest router score s[t][e], ties to the lower token index; its
    rows list those tokens in token order; the gate of a chosen (token,
    expert) pair is s[t][e]. Returns dict(offsets [E+1], perm_token [E*cap],
    row_of [N][E] (-1 = not chosen), gates [N][E] (0 = not chosen))."""
    s = np.asarray(s, np.float32)
    N, E = s.shape
    cap = min(int(capacity), N)
    offsets = (np.arange(E + 1) * cap).astype(np.int32)
    perm = np.empty(E * cap, np.int32)
    row_of = np.full((N, E), -1, np.int32)
    gates = np.zeros((N, E), np.float32)
    tok = np.arange(N)
    for e in range(E):
        order = np.lexsort((tok, -s[:, e].astype(np.float64)))  # score desc, then token asc
        chosen = np.sort(order[:cap])
        perm[e * cap:(e + 1) * cap] = chosen
        row_of[chosen, e] = e * cap + np.arange(cap)
        gates[chosen, e] = s[chosen, e]
    return dict(offsets=offsets, perm_token=perm, row_of=row_of, gates=gates, capacity=cap)


def dispatch(cand_ids, cand_scores, gates, n_experts, top_k, policy, capacity):
    cand = _c(cand_ids, np.int32)
    cs = _c(cand_scores, np.float32)
    N, C = cand.shape
    if policy == REROUTE:
        assert top_k == 1 and C == 2, "reroute is defined for top-1 with one spare candidate"
    g = np.array(gates, dtype=np.float32, copy=True, order="C")
    routed = np.empty(n_experts, np.int32)
    kept = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    row_of = np.empty((N, top_k), np.int32)
    expert_of = np.empty((N, top_k), np.int32)
    perm = np.full(N * top_k, -1, np.int32)
    R = lib().orc_dispatch(N, n_experts, top_k, C, policy, int(capacity), _p(cand), _p(cs),
                           _p(g), _p(routed), _p(kept), _p(offsets), _p(row_of),
                           _p(expert_of), _p(perm))
    return dict(gates=g, counts_routed=routed, counts_kept=kept, offsets=offsets,
                row_of=row_of, expert_of=expert_of, perm_token=perm[:R], R=int(R))


# ---------------------------------------------------------------- FFN
def expert_ffn(X, act, w_dt, w1, w3, w2, b1=None, b2=None, s1=None, s3=None, s2=None):
    """One expert's FFN on rows X [n][d] in fp64. w1/w3 [f][d], w2 [d][f] in their
    storage form (fp32 array, uint16 bf16 bits, or uint8 e4m3 codes)."""
    X = _c(X, np.float64)
    n, d = X.shape
    wt = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[w_dt]
    w1 = _c(w1, wt)
    f = w1.shape[0]
    Y = np.empty((n, d), np.float64)
    if n == 0:
        return Y
    lib().orc_expert_ffn(n, d, f, act, w_dt, _p(X), _p(w1), _p(_c(w3, wt)), _p(_c(w2, wt)),
                         _p(_c(b1, np.float32)), _p(_c(b2, np.float32)),
                         _p(_c(s1, np.float32)), _p(_c(s3, np.float32)),
                         _p(_c(s2, np.float32)), _p(Y))
    return Y


def combine(row_of, gates, Yexp, Ysh=None):
    row_of = _c(row_of, np.int32)
    N, k = row_of.shape
    Yexp = _c(Yexp, np.float64)
    d = Yexp.shape[-1]
    y = np.empty((N, d), np.float64)
    lib().orc_combine(N, d, k, _p(row_of), _p(_c(gates, np.float32)), _p(Yexp),
                      _p(_c(Ysh, np.float64)), _p(y))
    return y


def balance_stats(top_k, counts_routed, counts_kept, s, lse):
    s = _c(s, np.float32)
    N, E = s.shape
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    sc = np.empty(4, np.float64)
    lib().orc_balance_stats(N, E, top_k, _p(_c(counts_routed, np.int32)),
                            _p(_c(counts_kept, np.int32)), _p(s), _p(_c(lse, np.float64)),
                            _p(f), _p(P), _p(sc))
    return dict(f=f, P=P, switch_aux=sc[0], importance_cv2=sc[1], z_loss=sc[2],
                drop_rate=sc[3])


def bias_update(n_tokens, top_k, counts_routed, bias, rate):
    b = np.array(bias, dtype=np.float32, copy=True, order="C")
    r = _c(counts_routed, np.int32)
    lib().orc_bias_update(n_tokens, r.shape[0], top_k, _p(r), _p(b), float(rate))
    return b


# ---------------------------------------------------------------- layer
def decode_rows(x, x_dt) -> np.ndarray:
    """Activations in their storage form -> fp64 (exact)."""
    if x_dt == BF16:
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


class ExpertSource:
    """Gives one expert's weights in storage form as numpy arrays. `get(e)`
    returns dict(w1, w3, w2, b1, b2, s1, s3, s2). Subclassed by callers that
    fetch experts lazily (e.g. from device memory)."""

    def __init__(self, arrays: dict):
        self.a = arrays

    def get(self, e):
        out = {}
        for k in ("w1", "w3", "w2", "b1", "b2", "s1", "s3", "s2"):
            v = self.a.get(k)
            out[k] = None if v is None else v[e]
        return out


def ffn_for_assignments(tokens, experts, X64, act, w_dt, source: ExpertSource):
    """Expert outputs for a list of (token, expert) assignments, fp64 [n][d]."""
    tokens = np.asarray(tokens)
    experts = np.asarray(experts)
    d = X64.shape[1]
    Y = np.zeros((len(tokens), d), np.float64)
    for e in np.unique(experts):
        idx = np.nonzero(experts == e)[0]
        w = source.get(int(e))
        Y[idx] = expert_ffn(X64[tokens[idx]], act, w_dt, w["w1"], w["w3"], w["w2"], w["b1"],
                            w["b2"], w["s1"], w["s3"], w["s2"])
    return Y


def layer_forward(cfg, x, x_dt, w_gate, experts: ExpertSource, shared: ExpertSource = None,
                  logit_bias=None, select_bias=None, w_noise=None, logits=None,
                  tokens=None):
    """Full layer forward. If `logits` is given the router GEMM is skipped.
    If `tokens` is given, outputs are computed only for those token rows
    (routing and dispatch always run over all N tokens, since capacity
    couples tokens). Returns a dict with every intermediate."""
    if logits is None:
        H, raw = router_logits(x, x_dt, w_gate, logit_bias, w_noise, cfg.noise_seed)
    else:
        H, raw = np.ascontiguousarray(logits, np.float32), None
    if getattr(cfg, "expert_choice", False):
        return _expert_choice_forward(cfg, x, x_dt, H, raw, experts, shared, tokens)
    r = route(H, cfg.top_k, cfg.n_cand, cfg.renormalize, select_bias)
    cap = -1 if cfg.overflow == DROPLESS else capacity(H.shape[0], cfg.n_experts,
                                                        cfg.capacity_factor)
    dsp = dispatch(r["cand_ids"], r["cand_scores"], r["gates"], cfg.n_experts, cfg.top_k,
                   cfg.overflow, cap)
    st = balance_stats(cfg.top_k, dsp["counts_routed"], dsp["counts_kept"], r["s"], r["lse"])
    N = H.shape[0]
    rows = np.arange(N) if tokens is None else np.asarray(tokens)
    X64 = decode_rows(np.asarray(x)[rows], x_dt)
    k = cfg.top_k
    row_of = dsp["row_of"][rows]
    exp_of = dsp["expert_of"][rows]
    gates = dsp["gates"][rows]
    local_t, local_j = np.nonzero(row_of >= 0)
    Yexp = np.zeros((len(rows), k, X64.shape[1]), np.float64)
    if len(local_t):
        Yk = ffn_for_assignments(local_t, exp_of[local_t, local_j], X64, cfg.act,
                                 cfg.w_dtype, experts)
        Yexp[local_t, local_j] = Yk
    Ysh = None
    if shared is not None:
        Ysh = ffn_for_assignments(np.arange(len(rows)), np.zeros(len(rows), np.int64), X64,
                                  cfg.act, cfg.w_dtype, shared)
    y = combine(row_of, gates, Yexp, Ysh)
    return dict(logits=H, raw_logits=raw, route=r, dispatch=dsp, stats=st, y=y, rows=rows,
                Yexp=Yexp, Ysh=Ysh)


def _expert_choice_forward(cfg, x, x_dt, H, raw, experts, shared, tokens):
    """Layer forward with expert-choice routing: softmax scores as for token
    choice, every expert takes its ceil(N*top_k/E) top tokens, the FFNs run
    on those rows, and a token's output sums gate x expert output over the
    experts that chose it (in expert order), plus the shared expert."""
    r = route(H, 1, 1, False)  # the full score matrix s; its top-1 is unused
    ec = expert_choice(r["s"], expert_choice_capacity(H.shape[0], cfg.n_experts, cfg.top_k))
    E = cfg.n_experts
    N = H.shape[0]
    rows = np.arange(N) if tokens is None else np.asarray(tokens)
    X64 = decode_rows(np.asarray(x)[rows], x_dt)
    row_of = ec["row_of"][rows]
    gates = ec["gates"][rows]
    local_t, local_e = np.nonzero(row_of >= 0)
    Yexp = np.zeros((len(rows), E, X64.shape[1]), np.float64)
    if len(local_t):
        Yexp[local_t, local_e] = ffn_for_assignments(local_t, local_e, X64, cfg.act,
                                                     cfg.w_dtype, experts)
    Ysh = None
    if shared is not None:
        Ysh = ffn_for_assignments(np.arange(len(rows)), np.zeros(len(rows), np.int64), X64,
                                  cfg.act, cfg.w_dtype, shared)
    y = combine(row_of, gates, Yexp, Ysh)
    counts = np.full(E, ec["capacity"], np.int32)
    st = balance_stats(cfg.top_k, counts, counts, r["s"], r["lse"])
    return dict(logits=H, raw_logits=raw, route=r, ec=ec, stats=st, y=y, rows=rows,
                Yexp=Yexp, Ysh=Ysh)
