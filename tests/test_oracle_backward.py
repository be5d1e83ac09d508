"""Pins of the backward oracle (oracle/backward.py) against things it does not
compute itself: torch's automatic differentiation of the layer forward
written out in fp64 with the oracle's discrete decisions fixed, central
finite differences of the C oracle's fp64 expert FFN, and the pages'
statement that with top-k routing the unselected experts get no gradient
from the main loss while the auxiliary loss gives them one."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import backward as B


def _tiny(act=W.ACT_SWIGLU, w_dt=W.F32, renorm=True, k=2, E=4, overflow=W.DROPLESS, cf=None,
          noise=False, N=24, d=16, F=12, seed=7, shared=False, ec=False):
    cfg = W.C2.with_(name="bwd_tiny", n_tokens=N, d_model=d, n_experts=E, d_ff=F, top_k=k,
                     act=act, w_dtype=w_dt, x_dtype=W.F32 if w_dt == W.F32 else W.BF16,
                     renormalize=renorm and not ec, overflow=overflow, capacity_factor=cf,
                     seed=seed, noise_seed=44 if noise else 0, expert_choice=ec)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, d)).astype(np.float32)
    w = dict(w1=(rng.standard_normal((E, F, d)) / np.sqrt(d)).astype(np.float32),
             w3=(rng.standard_normal((E, F, d)) / np.sqrt(d)).astype(np.float32)
             if act == W.ACT_SWIGLU else None,
             w2=(rng.standard_normal((E, d, F)) / np.sqrt(F)).astype(np.float32),
             b1=(rng.standard_normal((E, F)) * 0.1).astype(np.float32) if act != W.ACT_SWIGLU
             else None,
             b2=(rng.standard_normal((E, d)) * 0.1).astype(np.float32) if act != W.ACT_SWIGLU
             else None)
    wg = (rng.standard_normal((E, d)) * 0.5).astype(np.float32)
    lb = (rng.standard_normal(E) * 0.1).astype(np.float32)
    wn = (rng.standard_normal((E, d)) * 0.3).astype(np.float32) if noise else None
    dy = rng.standard_normal((N, d))
    if shared:  # one always-on SwiGLU expert, gate 1
        w["shared"] = dict(w1=(rng.standard_normal((1, F, d)) / np.sqrt(d)).astype(np.float32),
                           w3=(rng.standard_normal((1, F, d)) / np.sqrt(d)).astype(np.float32),
                           w2=(rng.standard_normal((1, d, F)) / np.sqrt(F)).astype(np.float32))
    return cfg, x, w, wg, lb, wn, dy


def _autograd(cfg, x, w, wg, lb, wn, fwd, dy, alpha, beta):
    """The layer forward in torch fp64 with the oracle's selections and drops
    held fixed; torch differentiates L = <dy, y> + alpha aux + beta z."""
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    X, Wg, Lb = T(x), T(wg), T(lb)
    W1, W2 = T(w["w1"]), T(w["w2"])
    W3 = T(w["w3"]) if w["w3"] is not None else None
    B1 = T(w["b1"]) if w["b1"] is not None else None
    B2 = T(w["b2"]) if w["b2"] is not None else None
    Wn = T(wn) if wn is not None else None
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    l = X @ Wg.T + Lb
    if Wn is not None:
        z = torch.tensor(oracle.hash_normal_grid(cfg.noise_seed, N, E).astype(np.float64))
        l = l + z * torch.nn.functional.softplus(X @ Wn.T)
    s = torch.softmax(l, dim=1)
    lse = torch.logsumexp(l, dim=1)
    r = fwd["route"]
    if cfg.expert_choice:
        # every expert's chosen tokens fixed; a chosen pair's gate is s_te
        ec = fwd["ec"]
        row_of = ec["row_of"]
        exp_of = np.tile(np.arange(E, dtype=np.int64), (N, 1))
        g = s
        counts = np.full(E, ec["capacity"])
        slots = E
    else:
        dsp = fwd["dispatch"]
        cand = torch.tensor(r["cand_ids"][:, :k].astype(np.int64))
        exp_of = dsp["expert_of"]
        row_of = dsp["row_of"]
        if cfg.renormalize:
            sel = torch.gather(s, 1, cand)
            g = sel / sel.sum(dim=1, keepdim=True)
        else:
            g = torch.gather(s, 1, torch.tensor(np.maximum(exp_of, 0).astype(np.int64)))
        counts = dsp["counts_routed"]
        slots = k
    y = torch.zeros((N, cfg.d_model), dtype=torch.float64)
    for t in range(N):
        for j in range(slots):
            if row_of[t, j] < 0:
                continue
            e = int(exp_of[t, j])
            a = W1[e] @ X[t] + (B1[e] if B1 is not None else 0)
            if cfg.act == W.ACT_SWIGLU:
                h = torch.nn.functional.silu(a) * (W3[e] @ X[t])
            elif cfg.act == W.ACT_RELU:
                h = torch.relu(a)
            else:
                h = torch.nn.functional.gelu(a)
            o = W2[e] @ h + (B2[e] if B2 is not None else 0)
            y[t] = y[t] + g[t, j] * o
    if "shared" in w:
        S1, S3, S2 = (T(w["shared"][n][0]) for n in ("w1", "w3", "w2"))
        y = y + (torch.nn.functional.silu(X @ S1.T) * (X @ S3.T)) @ S2.T
    f = torch.tensor(counts.astype(np.float64) / (N * k))
    aux = E * (f * s.mean(dim=0)).sum()
    zl = (lse ** 2).mean()
    L = (torch.tensor(dy) * y).sum() + alpha * aux + beta * zl
    L.backward()
    out = dict(dx=X.grad, dw_gate=Wg.grad, dlogit_bias=Lb.grad, dW1=W1.grad, dW2=W2.grad)
    if W3 is not None:
        out["dW3"] = W3.grad
    if B1 is not None:
        out["db1"], out["db2"] = B1.grad, B2.grad
    if Wn is not None:
        out["dw_noise"] = Wn.grad
    if "shared" in w:
        out.update(shared_dW1=S1.grad, shared_dW3=S3.grad, shared_dW2=S2.grad)
    return {n: v.numpy() for n, v in out.items()}


def _run(cfg, x, w, wg, lb, wn, dy, alpha, beta):
    experts = oracle.ExpertSource(w)
    shared = oracle.ExpertSource(w["shared"]) if "shared" in w else None
    fwd = oracle.layer_forward(cfg, x, cfg.x_dtype, wg, experts, shared, lb, None, wn)
    got = B.layer_backward(cfg, x, cfg.x_dtype, wg, experts, fwd, dy, alpha, beta,
                           shared=shared, logit_bias=lb, w_noise=wn)
    return fwd, got


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("case", ["swiglu_renorm", "relu_switch_drop", "gelu_switch_noise",
                                  "swiglu_top1_reroute", "swiglu_top2_shared"])
def test_backward_matches_autograd(case):
    kw = dict(swiglu_renorm={}, relu_switch_drop=dict(act=W.ACT_RELU, renorm=False, k=1,
                                                      overflow=W.DROP, cf=0.75),
              gelu_switch_noise=dict(act=W.ACT_GELU, renorm=False, k=1, noise=True),
              swiglu_top1_reroute=dict(renorm=False, k=1, overflow=W.REROUTE_THEN_DROP,
                                       cf=0.5),
              swiglu_top2_shared=dict(shared=True))[case]
    cfg, x, w, wg, lb, wn, dy = _tiny(**kw)
    alpha, beta = 0.3, 0.05
    fwd, got = _run(cfg, x, w, wg, lb, wn, dy, alpha, beta)
    if cfg.overflow != W.DROPLESS:
        assert (fwd["dispatch"]["row_of"] < 0).any()  # the case has drops
    ref = _autograd(cfg, x, w, wg, lb, wn, fwd, dy, alpha, beta)
    for n, v in ref.items():
        # the oracle's softmax scores are the fp32 values of the forward,
        # torch's are fp64: agreement to a few fp32 ulps
        assert _rel(got[n], v) < 2e-6, (n, _rel(got[n], v))


@pytest.mark.parametrize("case", ["swiglu_shared", "relu_bias_logit_bias", "gelu_noise"])
def test_expert_choice_backward_matches_autograd(case):
    """Expert-choice routing: the experts' selections held fixed, a chosen
    pair's gate is its score."""
    kw = dict(swiglu_shared=dict(shared=True), relu_bias_logit_bias=dict(act=W.ACT_RELU),
              gelu_noise=dict(act=W.ACT_GELU, noise=True))[case]
    cfg, x, w, wg, lb, wn, dy = _tiny(ec=True, E=5, k=2, N=30, **kw)
    alpha, beta = 0.3, 0.05
    fwd, got = _run(cfg, x, w, wg, lb, wn, dy, alpha, beta)
    row_of = fwd["ec"]["row_of"]
    assert ((row_of >= 0).sum(axis=0) == fwd["ec"]["capacity"]).all()
    assert ((row_of >= 0).sum(axis=1) != cfg.top_k).any()  # tokens get uneven expert counts
    ref = _autograd(cfg, x, w, wg, lb, wn, fwd, dy, alpha, beta)
    for n, v in ref.items():
        assert _rel(got[n], v) < 2e-6, (n, _rel(got[n], v))
    # the auxiliary term is the same for every score of a token (f_e is
    # uniform), so the logit gradients do not depend on alpha -- up to the
    # fp32 scores summing to 1 within ~1e-7
    _, got0 = _run(cfg, x, w, wg, lb, wn, dy, 0.0, beta)
    assert _rel(got0["dl"], got["dl"]) < 1e-8


def test_expert_backward_matches_finite_differences():
    """Central differences of the C oracle's fp64 expert FFN (fp32 weights):
    <dX, V> and <dW, V_W> against (f(+) - f(-)) / 2 projected on dO."""
    rng = np.random.default_rng(3)
    n, d, F = 5, 8, 6
    X = rng.standard_normal((n, d))
    dO = rng.standard_normal((n, d))
    for act in (W.ACT_SWIGLU, W.ACT_RELU, W.ACT_GELU):
        w1 = (rng.standard_normal((F, d)) / 3).astype(np.float32)
        w3 = (rng.standard_normal((F, d)) / 3).astype(np.float32) if act == W.ACT_SWIGLU else None
        w2 = (rng.standard_normal((d, F)) / 3).astype(np.float32)
        b1 = None if act == W.ACT_SWIGLU else (rng.standard_normal(F) * 0.1).astype(np.float32)
        b2 = None if act == W.ACT_SWIGLU else (rng.standard_normal(d) * 0.1).astype(np.float32)

        def f(X_, w1_=w1, w3_=w3, w2_=w2):
            return np.sum(dO * oracle.expert_ffn(X_, act, W.F32, w1_, w3_, w2_, b1, b2))

        g = B.expert_backward(X, dO, act, w1.astype(np.float64),
                              None if w3 is None else w3.astype(np.float64),
                              w2.astype(np.float64),
                              None if b1 is None else b1.astype(np.float64),
                              None if b2 is None else b2.astype(np.float64))
        V = rng.standard_normal(X.shape)
        eps = 1e-6
        fd = (f(X + eps * V) - f(X - eps * V)) / (2 * eps)
        assert abs(fd - np.sum(g["dX"] * V)) < 1e-6 * max(1.0, abs(fd)), act
        for name in ("w1", "w2") + (("w3",) if w3 is not None else ()):
            base = dict(w1=w1, w3=w3, w2=w2)[name]
            Vw = rng.standard_normal(base.shape)
            wp = (base + 1e-3 * Vw).astype(np.float32)
            wm = (base - 1e-3 * Vw).astype(np.float32)
            delta = (wp.astype(np.float64) - wm.astype(np.float64)) / 2  # exact step taken
            kw_p, kw_m = {name + "_": wp}, {name + "_": wm}
            fd = f(X, **kw_p) - f(X, **kw_m)
            dW = g["d" + name.upper()]
            assert abs(fd / 2 - np.sum(dW * delta)) < 2e-6 * max(1.0, abs(fd)), (act, name)


def test_unselected_experts_get_no_main_loss_gradient():
    """heavensheep "Training": with top-k the experts a token did not select
    get zero gradient; the auxiliary loss is what gives them one."""
    cfg, x, w, wg, lb, wn, dy = _tiny(k=2, E=6)
    fwd, got = _run(cfg, x, w, wg, lb, wn, dy, 0.0, 0.0)
    sel = np.zeros((cfg.n_tokens, cfg.n_experts), bool)
    np.put_along_axis(sel, fwd["route"]["cand_ids"][:, :2], True, axis=1)
    assert np.all(got["ds"][~sel] == 0.0)
    assert np.all(got["ds"][sel] != 0.0)
    _, got_aux = _run(cfg, x, w, wg, lb, wn, dy, 0.5, 0.0)
    assert np.all(got_aux["ds"][~sel] != 0.0)
    # an expert that received no rows gets exactly zero weight gradients
    counts = fwd["dispatch"]["counts_kept"]
    for e in np.nonzero(counts == 0)[0]:
        assert not got["dW1"][e].any() and not got["dW2"][e].any()


def test_renormalised_gate_gradient_is_orthogonal_to_scores():
    """With renormalised gates the selected scores enter only through their
    ratios, so the gradient of the gate part (alpha = beta = 0) is orthogonal
    to the selected scores: sum_j s_cj dL/ds_cj = 0 for every token."""
    cfg, x, w, wg, lb, wn, dy = _tiny(k=3, E=5)
    fwd, got = _run(cfg, x, w, wg, lb, wn, dy, 0.0, 0.0)
    s = fwd["route"]["s"].astype(np.float64)
    dots = (s * got["ds"]).sum(axis=1)
    assert np.max(np.abs(dots)) < 1e-12 * np.max(np.abs(got["ds"]))


def test_sampled_evaluations_equal_full_ones():
    """The sampled forms used at full size (features of one expert, tokens of
    the router part) agree with the full computations pinned above."""
    cfg, x, w, wg, lb, wn, dy = _tiny(k=2, E=4, N=30)
    fwd, got = _run(cfg, x, w, wg, lb, wn, dy, 0.2, 0.03)
    X = x.astype(np.float64)
    dsp = fwd["dispatch"]
    e = int(np.argmax(dsp["counts_kept"]))
    tt, jj = np.nonzero((dsp["row_of"] >= 0) & (dsp["expert_of"] == e))
    dO = dsp["gates"][tt, jj].astype(np.float64)[:, None] * dy[tt]
    fs = np.array([0, 5, 11])
    part = B.weight_grad_features(X[tt], dO, w["w1"][e].astype(np.float64),
                                  w["w3"][e].astype(np.float64), w["w2"][e].astype(np.float64), fs)
    assert np.allclose(part["dW1"], got["dW1"][e][fs], rtol=1e-12, atol=1e-14)
    assert np.allclose(part["dW3"], got["dW3"][e][fs], rtol=1e-12, atol=1e-14)
    assert np.allclose(part["dW2"], got["dW2"][e][:, fs], rtol=1e-12, atol=1e-14)
    rows = np.array([3, 17, 29])
    sub = B.router_backward(cfg, X[rows], wg, fwd, got["dg"][rows], 0.2, 0.03, lb, rows=rows,
                            n_total=cfg.n_tokens)
    full = B.router_backward(cfg, X, wg, fwd, got["dg"], 0.2, 0.03, lb)
    for name in ("dl", "ds", "dx"):
        assert np.allclose(sub[name], full[name][rows], rtol=1e-12, atol=1e-15), name
