"""GPU parity of expert-choice routing (every expert takes its top-capacity
tokens by router score) against the oracle: the selection alone on edge
shapes and ties, the router's full score output, the wide combine (k = E),
and the whole layer on the reduced expert-choice workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import (MARGIN, TOL_REL, experts_of, host_inputs, out_tol, rel_err,
                          require_gpu, to_device, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    require_gpu()
    import sparse_mixture_experts_47_amd as m
    return m


def _softmax_scores(N, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, E))
    if ties:  # quantised logits: many exactly equal scores in a column
        x = np.round(x * 2) / 2
    s = np.exp(x - x.max(1, keepdims=True))
    return (s / s.sum(1, keepdims=True)).astype(np.float32)


def _ec_gpu(moe, s, cap):
    N, E = s.shape
    i32 = dict(dtype=torch.int32, device="cuda")
    c = min(cap, N)
    out = dict(offsets=torch.full((E + 1,), -5, **i32), perm_token=torch.full((E * c,), -5, **i32),
               row_of=torch.full((N, E), -5, **i32),
               gates=torch.full((N, E), 9.0, dtype=torch.float32, device="cuda"),
               counts=torch.full((E,), -5, **i32))
    moe.moe_expert_choice(torch.from_numpy(s).cuda(), cap, **out)
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in out.items()}


@pytest.mark.parametrize("N,E,cap,ties", [(1, 1, 1, False), (37, 8, 10, False),
                                          (600, 8, 150, True), (1000, 64, 40, False),
                                          (3000, 8, 5000, False), (2049, 4, 2049, True),
                                          (65, 256, 1, False), (8192, 8, 2048, False),
                                          (5000, 3, 1667, True), (40000, 4, 10000, True)])
def test_expert_choice_selection_bit_exact(moe, N, E, cap, ties):
    # N = 40000 takes the kernel form that reads scores from global memory
    print("ec select", N, E, cap, ties, flush=True)
    s = _softmax_scores(N, E, N + E, ties)
    ref = oracle.expert_choice(s, cap)
    got = _ec_gpu(moe, s, cap)
    for k in ("offsets", "perm_token", "row_of"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.array_equal(got["gates"].view(np.uint32), ref["gates"].view(np.uint32))
    assert np.all(got["counts"] == ref["capacity"])


def test_expert_choice_all_equal_scores_takes_first_tokens(moe):
    # every score equal: ties go to the lower token index
    N, E, cap = 300, 3, 100
    s = np.full((N, E), 1.0 / E, np.float32)
    got = _ec_gpu(moe, s, cap)
    for e in range(E):
        assert got["perm_token"][e * cap:(e + 1) * cap].tolist() == list(range(cap))
    assert np.all(got["row_of"][cap:] == -1)


def test_router_scores_out_is_the_softmax(moe):
    g = torch.Generator().manual_seed(11)
    N, E = 333, 16
    logits = torch.randn((N, E), generator=g) * 2
    ref = oracle.route(logits.numpy(), 1, 1, False)
    i32 = dict(dtype=torch.int32, device="cuda")
    scores = torch.empty((N, E), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(None, torch.zeros((E, 8), device="cuda"), top_k=1, renormalize=False,
                        logits_in=logits.cuda(), cand_ids=torch.empty((N, 1), **i32),
                        cand_scores=torch.empty((N, 1), device="cuda"),
                        gates=torch.empty((N, 1), device="cuda"), scores_out=scores)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(scores).view(np.uint32), ref["s"].view(np.uint32))


@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_wide_combine_matches_narrow_and_oracle(moe, ydt):
    """k = 12 slots with at most 8 kept per token: the wide kernel must equal
    the k <= 8 kernel run on the same kept slots packed in order (same fma
    order), and the oracle's combine."""
    rng = np.random.default_rng(5)
    N, d, k = 70, 264, 12
    R = N * k
    row_of = rng.permutation(R).astype(np.int32).reshape(N, k)
    gates = rng.random((N, k)).astype(np.float32)
    for t in range(N):
        drop = rng.choice(k, size=k - int(rng.integers(0, 9)), replace=False)
        row_of[t, drop] = -1
    row_of[3] = -1
    narrow_rows = np.full((N, 8), -1, np.int32)
    narrow_g = np.zeros((N, 8), np.float32)
    for t in range(N):
        j = np.nonzero(row_of[t] >= 0)[0]
        narrow_rows[t, :len(j)] = row_of[t, j]
        narrow_g[t, :len(j)] = gates[t, j]
    yr = torch.randn((R, d)).to(ydt)
    ysh = torch.randn((N, d)).to(ydt)
    outs = []
    for ro, gg in ((row_of, gates), (narrow_rows, narrow_g)):
        out = torch.empty((N, d), dtype=torch.float32, device="cuda")
        moe.moe_combine(yr.cuda(), torch.from_numpy(ro).cuda(), torch.from_numpy(gg).cuda(), out,
                        y_shared=ysh.cuda())
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    yr64 = yr.double().numpy()
    Yexp = np.zeros((N, k, d))
    for t in range(N):
        for j in range(k):
            if row_of[t, j] >= 0:
                Yexp[t, j] = yr64[row_of[t, j]]
    ref = oracle.combine(row_of, gates, Yexp, ysh.double().numpy())
    assert rel_err(to_np(outs[0]), ref) <= 1e-6


def _layer(moe, cfg, dev):
    spec = moe.spec_from_config(cfg)
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    return moe.MoELayer(spec, dev, x_dtype=xdt)


def _oracle_forward(cfg, host, logits=None):
    shared = experts_of(host, "shared_") if cfg.shared_d_ff else None
    return oracle.layer_forward(cfg, host["x"], cfg.x_dtype, host["w_gate"], experts_of(host),
                                shared, host["logit_bias"], host["select_bias"],
                                host["w_noise"], logits=logits)


def _check_ec(layer, ec):
    assert np.array_equal(to_np(layer.offsets), ec["offsets"])
    assert np.array_equal(to_np(layer.perm_token), ec["perm_token"])
    assert np.array_equal(to_np(layer.row_of), ec["row_of"])
    assert np.array_equal(to_np(layer.ec_gates).view(np.uint32), ec["gates"].view(np.uint32))


EC_LAYERS = {
    "c6": W.REDUCED["c6"],
    # fine-grained experts (64, capacity ceil(320*8/64) = 40) plus a shared expert
    "c3_expert_choice": W.REDUCED["c3"].with_(name="deepseek_reduced_expert_choice",
                                              expert_choice=True, select_bias=False),
}


@pytest.mark.parametrize("key", list(EC_LAYERS))
def test_expert_choice_layer_level1(moe, key):
    cfg = EC_LAYERS[key]
    print("ec level1", cfg, flush=True)
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    ref = _oracle_forward(cfg, host)
    dev = to_device(inp)
    layer = _layer(moe, cfg, dev)
    y = layer.forward(dev["x"], logits_in=torch.from_numpy(ref["logits"]).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_np(layer.scores).view(np.uint32), ref["route"]["s"].view(np.uint32))
    _check_ec(layer, ref["ec"])
    err = rel_err(to_np(y), ref["y"])
    print("  max|dy|/rms =", err)
    assert err <= out_tol(cfg)
    st = ref["stats"]
    assert np.allclose(to_np(layer.f), st["f"], rtol=TOL_REL, atol=0)
    assert np.allclose(to_np(layer.P), st["P"], rtol=TOL_REL, atol=1e-12)
    sc = to_np(layer.scalars)
    for i, name in enumerate(("switch_aux", "importance_cv2", "z_loss", "drop_rate")):
        assert abs(sc[i] - st[name]) <= TOL_REL * abs(st[name]) + 1e-7, (name, sc[i], st[name])


def test_expert_choice_layer_level2(moe):
    """GPU router GEMM: every (token, expert) pair whose score is at least
    MARGIN away from that expert's selection threshold is chosen alike, and
    tokens chosen by the same experts get the same output."""
    cfg = W.REDUCED["c6"]
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    ref = _oracle_forward(cfg, host)
    dev = to_device(inp)
    layer = _layer(moe, cfg, dev)
    y = layer.forward(dev["x"])
    torch.cuda.synchronize()
    assert rel_err(to_np(layer.logits), ref["logits"]) <= TOL_REL
    s = ref["route"]["s"].astype(np.float64)
    cap = ref["ec"]["capacity"]
    thr = np.sort(s, axis=0)[::-1][cap - 1]  # each expert's cap-th largest score
    far = np.abs(s - thr[None, :]) >= MARGIN * thr[None, :]
    gsel, rsel = to_np(layer.row_of) >= 0, ref["ec"]["row_of"] >= 0
    assert np.all(gsel[far] == rsel[far])
    alike = np.all(gsel == rsel, axis=1)
    assert alike.mean() > 0.5
    assert rel_err(to_np(y)[alike], ref["y"][alike]) <= out_tol(cfg)
