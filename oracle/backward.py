"""CPU oracle for the backward pass of the MoE FFN layer -- TEST INFRASTRUCTURE.

Only the tests and the benchmark's `cpu_baseline` leg may import this
module; the product library never does and shares no code with it.

What it differentiates. The layer forward of `oracle.layer_forward` with the
discrete decisions (which experts a token selects, which assignments a
capacity drops) held fixed, and the scalar

    L = sum_t <dy_t, y_t> + alpha * switch_aux + beta * z_loss

where dy is the upstream gradient, switch_aux = E * sum_e f_e * P_e with
f_e = routed_e / (N k) a count (no gradient) and P_e = (1/N) sum_t s_te, and
z_loss = (1/N) sum_t lse_t^2 over the logits the softmax sees.

Passages. heavensheep.xyz MoE notes, section "Training": with top-k
selection the experts a token did not select get zero gradient from the main
loss, and the auxiliary loss of f_i and P_i is what gives the router of an
unselected expert a gradient. mkbk-pku.cn, "通信与并行", step 5: the
backward pass sends gradients back along the same routing path (expert
output -> expert -> the token's position). chiang97912 MoE notes, "专家选择":
y = sum_i G(x)_i E_i(x), so the gate and the expert output each take the
other as the factor of their gradient. CS336 notes section 4: the z-loss.

Everything here is plain fp64 numpy, written from the chain rule in the
order the forward runs backwards:
  combine -> (gate gradient, expert-output gradient)
  expert FFN: W2, activation, W1/W3 (and biases) -> token-row gradient
  gates -> scores (renormalisation Jacobian, or the Switch identity)
  + auxiliary-loss term on the scores
  softmax -> logits, + z-loss term on the logits
  (noise: logits of the softmax -> raw logits and W_noise)
  router GEMM -> W_g, logit bias and the token rows.

Expert choice (heavensheep "Routing Function"; CS336 notes section 3: the
experts select tokens): the selections of every expert are held fixed, a
chosen (token, expert) pair's gate is the score s_te itself, so the gate
gradient is the score gradient of that pair; f_e = capacity / (N k) is the
same for every expert, and the auxiliary term then adds the same amount to
every score of a token, which the softmax Jacobian removes.
"""
from __future__ import annotations

import numpy as np

from . import (BF16, F32, FP8, GELU, RELU, SWIGLU, decode_rows, hash_normal_grid)


def decode_weight(w, w_dt):
    """Weights in storage form (fp32, or bf16 bits as uint16) -> fp64."""
    if w is None:
        return None
    if w_dt == BF16:
        return decode_rows(w, BF16)
    if w_dt == F32:
        return np.asarray(w, np.float32).astype(np.float64)
    raise ValueError("the backward oracle covers fp32 and bf16 weights (fp8 is inference-only)")


def _phi(a):
    return np.exp(-0.5 * a * a) / np.sqrt(2.0 * np.pi)


def _Phi(a):
    from scipy.special import erf
    return 0.5 * (1.0 + erf(a / np.sqrt(2.0)))


def expert_backward(X, dO, act, w1, w3, w2, b1=None, b2=None):
    """One expert on rows X [n][d] (fp64) with output gradient dO [n][d].
    Forward: a = X W1^T (+b1); SwiGLU: u = X W3^T, h = silu(a) * u; ReLU /
    GELU: h = act(a); o = h W2^T (+b2).
    Returns dict(dX, dW1, dW3, dW2, db1, db2) in fp64 (dW3 None unless SwiGLU)
    and the intermediates a, u, h, dh, da, du (u, du None unless SwiGLU)."""
    a = X @ w1.T
    if b1 is not None:
        a = a + b1
    if act == SWIGLU:
        sig = 1.0 / (1.0 + np.exp(-a))
        u = X @ w3.T
        h = a * sig * u
    elif act == RELU:
        u = None
        h = np.maximum(a, 0.0)
    else:  # GELU, exact erf form
        u = None
        h = a * _Phi(a)
    dh = dO @ w2              # o = h W2^T  ->  dh = dO W2
    dW2 = dO.T @ h            # dW2[c][f] = sum_rows dO[c] h[f]
    db2 = dO.sum(axis=0) if b2 is not None else None
    dW3 = du = None
    if act == SWIGLU:
        # h = silu(a) u: dh/da = u silu'(a), silu'(a) = sig (1 + a (1 - sig)); dh/du = silu(a)
        da = dh * u * sig * (1.0 + a * (1.0 - sig))
        du = dh * a * sig
        dW3 = du.T @ X
        dX = da @ w1 + du @ w3
    elif act == RELU:
        da = dh * (a > 0.0)
        dX = da @ w1
    else:
        da = dh * (_Phi(a) + a * _phi(a))
        dX = da @ w1
    dW1 = da.T @ X
    db1 = da.sum(axis=0) if b1 is not None else None
    return dict(dX=dX, dW1=dW1, dW3=dW3, dW2=dW2, db1=db1, db2=db2, a=a, u=u, h=h, dh=dh, da=da,
                du=du)


def layer_backward(cfg, x, x_dt, w_gate, experts, fwd, dy, alpha=0.0, beta=0.0,
                   shared=None, logit_bias=None, w_noise=None, keep_terms=False):
    """Gradients of L (module docstring) for a token-choice layer.

    cfg, x, x_dt, w_gate, experts (an ExpertSource), shared, logit_bias and
    w_noise are the forward's inputs; fwd is `oracle.layer_forward`'s result
    over all tokens (its routing, dispatch and statistics are reused as the
    fixed discrete decisions); dy [N][d] is the upstream gradient.
    Returns dict with dx [N][d], dw_gate [E][d], dlogit_bias [E] (or None),
    dw_noise [E][d] (or None), dl [N][E] (gradient of the logits the softmax
    sees), dg [N][k] (gate gradients), ds [N][E] (score gradients) and, per
    expert e, dW1/dW3/dW2/db1/db2 [E][...] (zeros for experts with no rows),
    and the shared expert's dW (shared_dW1, ...). keep_terms: also
    `terms`, per expert dict(tokens, slots, X, dO, w1, w3, w2, a, u, h, dh,
    da, du): its rows' token and slot indices and fp64 intermediates (and
    `shared_terms` for the shared expert, every token with gate 1)."""
    if getattr(cfg, "expert_choice", False):
        return _expert_choice_backward(cfg, x, x_dt, w_gate, experts, fwd, dy, alpha, beta,
                                       shared, logit_bias, w_noise, keep_terms)
    X = decode_rows(x, x_dt)
    N, d = X.shape
    E, k = cfg.n_experts, cfg.top_k
    dy = np.asarray(dy, np.float64)
    r, dsp = fwd["route"], fwd["dispatch"]
    row_of, exp_of = dsp["row_of"], dsp["expert_of"]
    gates_used = dsp["gates"]   # the gate each kept assignment was scaled by
    Yexp = fwd["Yexp"]          # [N][k][d] fp64 expert outputs (0 where dropped)

    # ---- combine: y_t = sum_j g_tj o_tj (+ shared); kept slots only
    kept = row_of >= 0
    dg = np.where(kept, np.einsum("td,tjd->tj", dy, Yexp), 0.0)

    # ---- experts (routed), grouped by expert
    dX = np.zeros((N, d))
    grads = {n: [] for n in ("dW1", "dW3", "dW2", "db1", "db2")}
    terms = []
    for e in range(E):
        tt, jj = np.nonzero(kept & (exp_of == e))
        w = experts.get(e)
        w1 = decode_weight(w["w1"], cfg.w_dtype)
        w3 = decode_weight(w["w3"], cfg.w_dtype)
        w2 = decode_weight(w["w2"], cfg.w_dtype)
        b1 = None if w["b1"] is None else np.asarray(w["b1"], np.float64)
        b2 = None if w["b2"] is None else np.asarray(w["b2"], np.float64)
        dO = gates_used[tt, jj].astype(np.float64)[:, None] * dy[tt]
        g = expert_backward(X[tt], dO, cfg.act, w1, w3, w2, b1, b2)
        np.add.at(dX, tt, g["dX"])
        for n in grads:
            grads[n].append(g[n])
        if keep_terms:
            terms.append(dict(tokens=tt, slots=jj, X=X[tt], dO=dO, w1=w1, w3=w3, w2=w2,
                              **{n: g[n] for n in ("a", "u", "h", "dh", "da", "du")}))
    out = {n: (None if grads[n][0] is None else np.stack(grads[n])) for n in grads}
    if keep_terms:
        out["terms"] = terms

    if shared is not None:
        dX += _shared_backward(cfg, X, dy, shared, out, keep_terms)

    rb = router_backward(cfg, X, w_gate, fwd, dg, alpha, beta, logit_bias, w_noise)
    dX += rb.pop("dx")
    out.update(rb)
    out["dx"] = dX
    out["dg"] = dg
    return out


def _shared_backward(cfg, X, dy, shared, out, keep_terms):
    """The shared expert (gate 1 on every token): stores its weight
    gradients (and terms) in out, returns its token-row gradient."""
    w = shared.get(0)
    w1s, w3s, w2s = (decode_weight(w[n], cfg.w_dtype) for n in ("w1", "w3", "w2"))
    g = expert_backward(X, dy, cfg.act, w1s, w3s, w2s)
    for n in ("dW1", "dW3", "dW2"):
        out["shared_" + n] = g[n]
    if keep_terms:
        out["shared_terms"] = dict(tokens=np.arange(X.shape[0]), X=X, dO=dy, w1=w1s, w3=w3s,
                                   w2=w2s, **{n: g[n] for n in ("a", "u", "h", "dh", "da", "du")})
    return g["dX"]


def _expert_choice_backward(cfg, x, x_dt, w_gate, experts, fwd, dy, alpha, beta, shared,
                            logit_bias, w_noise, keep_terms):
    """layer_backward for expert-choice routing (see the module docstring).
    fwd["ec"] holds row_of and gates [N][E] of the chosen pairs; dg is then
    [N][E] (0 where expert e did not choose token t) and the terms' slots
    are expert indices."""
    X = decode_rows(x, x_dt)
    N, d = X.shape
    E = cfg.n_experts
    dy = np.asarray(dy, np.float64)
    ec = fwd["ec"]
    row_of, gates = ec["row_of"], ec["gates"]
    kept = row_of >= 0
    dg = np.where(kept, np.einsum("td,ted->te", dy, fwd["Yexp"]), 0.0)
    dX = np.zeros((N, d))
    grads = {n: [] for n in ("dW1", "dW3", "dW2", "db1", "db2")}
    terms = []
    for e in range(E):
        tt = np.nonzero(kept[:, e])[0]  # an expert's rows list its tokens in token order
        w = experts.get(e)
        w1, w3, w2 = (decode_weight(w[n], cfg.w_dtype) for n in ("w1", "w3", "w2"))
        b1 = None if w["b1"] is None else np.asarray(w["b1"], np.float64)
        b2 = None if w["b2"] is None else np.asarray(w["b2"], np.float64)
        dO = gates[tt, e].astype(np.float64)[:, None] * dy[tt]
        g = expert_backward(X[tt], dO, cfg.act, w1, w3, w2, b1, b2)
        np.add.at(dX, tt, g["dX"])
        for n in grads:
            grads[n].append(g[n])
        if keep_terms:
            terms.append(dict(tokens=tt, slots=np.full(len(tt), e), X=X[tt], dO=dO, w1=w1,
                              w3=w3, w2=w2, **{n: g[n] for n in ("a", "u", "h", "dh", "da", "du")}))
    out = {n: (None if grads[n][0] is None else np.stack(grads[n])) for n in grads}
    if keep_terms:
        out["terms"] = terms
    if shared is not None:
        dX += _shared_backward(cfg, X, dy, shared, out, keep_terms)
    # gate of a chosen pair = s_te: dL/ds_te = dg_te
    f = np.full(E, ec["capacity"] / (N * cfg.top_k))
    rb = _logits_backward(cfg, X, w_gate, fwd["route"], dg.copy(), f, alpha, beta, logit_bias,
                          w_noise, np.arange(N), N)
    dX += rb.pop("dx")
    out.update(rb)
    out["dx"] = dX
    out["dg"] = dg
    return out


def weight_grad_features(X, dO, w1, w3, w2, fs, want_dW=True):
    """One SwiGLU expert's weight gradients restricted to the features fs
    (indices into d_ff): rows fs of dW1 and dW3 ([len(fs)][d]) and columns fs
    of dW2 ([d][len(fs)]), from its rows X [n][d] and output gradients dO
    [n][d] (fp64). The same definitions as expert_backward, evaluated only
    where asked, so full-size layers can be sampled. Also returns the
    intermediates a, u, h, dh, da, du [n][len(fs)] (only these when
    want_dW is false)."""
    fs = np.asarray(fs)
    a = X @ w1[fs].T
    u = X @ w3[fs].T
    sig = 1.0 / (1.0 + np.exp(-a))
    h = a * sig * u
    dh = dO @ w2[:, fs]
    da = dh * u * sig * (1.0 + a * (1.0 - sig))
    du = dh * a * sig
    out = dict(a=a, u=u, h=h, dh=dh, da=da, du=du)
    if want_dW:
        out.update(dW1=da.T @ X, dW3=du.T @ X, dW2=dO.T @ h)
    return out


def router_backward(cfg, X, w_gate, fwd, dg, alpha=0.0, beta=0.0, logit_bias=None,
                    w_noise=None, rows=None, n_total=None):
    """Router part of the backward pass for given gate gradients dg [N][k]
    (fp64; 0 for dropped slots): gates -> scores (+ auxiliary loss) ->
    logits (+ z-loss) -> (noise) -> W_g, logit bias and the token rows X
    (fp64 [N][d]). fwd gives the forward's route (s, lse, cand_ids) and
    dispatch (expert_of, row_of, counts_routed). Returns dict(ds, dl, dw_gate,
    dlogit_bias, dw_noise, dx) with dx the router's share of the token
    gradient. rows (optional): X and dg hold only these tokens of the batch
    (its size n_total sets the 1/N of the auxiliary and z-loss terms and of
    f_e); the per-token formulas are evaluated for them alone."""
    r, dsp = fwd["route"], fwd["dispatch"]
    rows = np.arange(X.shape[0]) if rows is None else np.asarray(rows)
    N = X.shape[0] if n_total is None else int(n_total)
    E, k = cfg.n_experts, cfg.top_k
    kept = dsp["row_of"][rows] >= 0
    exp_of = dsp["expert_of"][rows]
    dg = np.where(kept, np.asarray(dg, np.float64), 0.0)
    s = r["s"][rows].astype(np.float64)
    n = len(rows)
    ds = np.zeros((n, E))
    if cfg.renormalize:
        # g_j = s_{c_j} / S, S = sum over the k selected candidates:
        # dL/ds_{c_i} = (dg_i - sum_j dg_j g_j) / S
        cand = r["cand_ids"][rows][:, :k]
        sel = np.take_along_axis(s, cand, axis=1)
        S = sel.sum(axis=1, keepdims=True)
        gk = sel / S
        ds_sel = (dg - (dg * gk).sum(axis=1, keepdims=True)) / S
        np.put_along_axis(ds, cand, ds_sel, axis=1)
    else:
        # Switch gate: g = s of the expert actually used (after a reroute)
        for j in range(k):
            np.add.at(ds, (np.arange(n), np.maximum(exp_of[:, j], 0)), dg[:, j])
    f = dsp["counts_routed"].astype(np.float64) / (N * k)
    return _logits_backward(cfg, X, w_gate, r, ds, f, alpha, beta, logit_bias, w_noise, rows, N)


def _logits_backward(cfg, X, w_gate, r, ds, f, alpha, beta, logit_bias, w_noise, rows, N):
    """From score gradients ds [n][E] (the tokens `rows` of a batch of N):
    + the auxiliary-loss term (f_e the routed fractions), softmax -> logits,
    + z-loss, (noise), router GEMM. Returns dict(ds, dl, dw_gate,
    dlogit_bias, dw_noise, dx)."""
    E = cfg.n_experts
    s = r["s"][rows].astype(np.float64)
    # auxiliary loss: d(alpha E sum_e f_e P_e)/ds_te = alpha E f_e / N
    ds = ds + alpha * E * np.asarray(f, np.float64)[None, :] / N

    # softmax -> logits (+ z-loss: d(lse_t^2 / N)/dl_te = 2 lse_t s_te / N)
    dl = s * (ds - (s * ds).sum(axis=1, keepdims=True))
    dl += beta * 2.0 * r["lse"][rows][:, None] * s / N

    # noise: H = l + z * softplus(v); dH/dl = 1, dH/dv = z * sigmoid(v)
    wg = np.asarray(w_gate, np.float32).astype(np.float64)
    dx = np.zeros_like(X)
    dw_noise = None
    if w_noise is not None:
        wn = np.asarray(w_noise, np.float32).astype(np.float64)
        v = X @ wn.T
        z = hash_normal_grid(cfg.noise_seed, N, E)[rows].astype(np.float64)
        dv = dl * z / (1.0 + np.exp(-v))
        dw_noise = dv.T @ X
        dx += dv @ wn
    # router GEMM l = X W_g^T (+ b)
    dx += dl @ wg
    return dict(ds=ds, dl=dl, dw_gate=dl.T @ X,
                dlogit_bias=None if logit_bias is None else dl.sum(axis=0),
                dw_noise=dw_noise, dx=dx)
