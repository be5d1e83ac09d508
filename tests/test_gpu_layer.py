"""GPU parity of libmoe against the CPU oracle on reduced-size workloads.

Level 1: the GPU gets the oracle's fp32 logits (logits_in); every routing
and dispatch output must be bit-identical and the layer output must agree
within the dtype's tolerance. Level 2: the GPU computes its own logits; they
must agree with the oracle's, ids must agree for every token whose key
margin is at least 1e-3, and outputs of tokens routed alike must agree.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import (MARGIN, TOL_FP8, TOL_REL, DeviceExperts, experts_of, host_inputs, margins,
                          oracle_keys, out_tol, rel_err, require_gpu, to_device, to_np)

pytestmark = pytest.mark.gpu

CFG_KEYS = ["c1", "c2", "c3", "c4", "c5"]


@pytest.fixture(scope="module")
def moe():
    require_gpu()
    import sparse_mixture_experts_47_amd as m
    return m


def _layer(moe, cfg, dev):
    spec = moe.spec_from_config(cfg)
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    return moe.MoELayer(spec, dev, x_dtype=xdt)


def _oracle_forward(cfg, host, logits=None):
    shared = experts_of(host, "shared_") if cfg.shared_d_ff else None
    return oracle.layer_forward(cfg, host["x"], cfg.x_dtype, host["w_gate"], experts_of(host),
                                shared, host["logit_bias"], host["select_bias"],
                                host["w_noise"], logits=logits)


def _check_stats(layer, ref, cfg):
    st = ref["stats"]
    torch.cuda.synchronize()
    f, P, sc = to_np(layer.f), to_np(layer.P), to_np(layer.scalars)
    assert np.allclose(f, st["f"], rtol=TOL_REL, atol=0)
    assert np.allclose(P, st["P"], rtol=TOL_REL, atol=1e-12)
    for i, name in enumerate(("switch_aux", "importance_cv2", "z_loss", "drop_rate")):
        assert abs(sc[i] - st[name]) <= TOL_REL * abs(st[name]) + 1e-7, (name, sc[i], st[name])


@pytest.mark.parametrize("key", CFG_KEYS)
def test_level1_routing_bit_exact_and_outputs(moe, key):
    cfg = W.REDUCED[key]
    print("level1", key, cfg, flush=True)
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    ref = _oracle_forward(cfg, host)
    dev = to_device(inp)
    layer = _layer(moe, cfg, dev)
    logits_in = torch.from_numpy(ref["logits"]).cuda()
    y = layer.forward(dev["x"], logits_in=logits_in)
    torch.cuda.synchronize()
    r, d = ref["route"], ref["dispatch"]
    assert np.array_equal(to_np(layer.cand_ids), r["cand_ids"])
    assert np.array_equal(to_np(layer.cand_scores).view(np.uint32),
                          r["cand_scores"].view(np.uint32))
    assert np.array_equal(to_np(layer.gates).view(np.uint32), d["gates"].view(np.uint32))
    assert np.array_equal(to_np(layer.counts_routed), d["counts_routed"])
    assert np.array_equal(to_np(layer.counts_kept), d["counts_kept"])
    assert np.array_equal(to_np(layer.offsets), d["offsets"])
    assert np.array_equal(to_np(layer.row_of), d["row_of"])
    assert np.array_equal(to_np(layer.expert_of), d["expert_of"])
    R = d["R"]
    assert np.array_equal(to_np(layer.perm_token)[:R], d["perm_token"])
    if layer.x_perm is not None:  # explicit gather path: rows are exact copies
        xp = to_np(layer.x_perm.float() if layer.x_perm.dtype == torch.bfloat16 else layer.x_perm)
        xs = to_np(dev["x"].float())
        assert np.array_equal(xp[:R], xs[d["perm_token"]])
    err = rel_err(to_np(y), ref["y"])
    print("  max|dy|/rms =", err)
    assert err <= out_tol(cfg)
    _check_stats(layer, ref, cfg)


@pytest.mark.parametrize("key", CFG_KEYS)
def test_level2_router_gemm(moe, key):
    cfg = W.REDUCED[key]
    print("level2", key, flush=True)
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    ref = _oracle_forward(cfg, host)
    dev = to_device(inp)
    layer = _layer(moe, cfg, dev)
    y = layer.forward(dev["x"])
    torch.cuda.synchronize()
    l_gpu, l_ref = to_np(layer.logits), ref["logits"]
    # logits: fp32 accumulation vs fp64; relative to the logits' RMS
    lerr = rel_err(l_gpu, l_ref)
    print("  logits max|dl|/rms =", lerr)
    assert lerr <= TOL_REL
    keys = oracle_keys(ref["route"], host["select_bias"])
    mg = margins(keys, cfg.top_k)
    ok = mg >= MARGIN
    gid = np.sort(to_np(layer.cand_ids)[:, :cfg.top_k], axis=1)
    rid = np.sort(ref["route"]["cand_ids"][:, :cfg.top_k], axis=1)
    same = np.all(gid == rid, axis=1)
    assert np.all(same[ok]), np.nonzero(~same & ok)
    print("  tokens inside margin:", int((~ok).sum()), "of", len(ok),
          "; id match inside margin:", float(same[~ok].mean()) if (~ok).any() else 1.0)
    # outputs of tokens whose final routing (expert set, drops) is identical
    ge = np.sort(to_np(layer.expert_of), axis=1)
    re = np.sort(ref["dispatch"]["expert_of"], axis=1)
    alike = np.all(ge == re, axis=1)
    assert alike.mean() > 0.5
    err = rel_err(to_np(y)[alike], ref["y"][alike])
    assert err <= out_tol(cfg), err


@pytest.mark.parametrize("E,k,C,N,scale", [(5, 2, 3, 37, 1.0), (100, 8, 8, 70, 1.5),
                                           (256, 8, 9, 65, 2.0), (64, 1, 2, 1, 1.0),
                                           (3, 3, 3, 8, 0.0), (256, 1, 1, 130, 30.0)])
def test_router_select_edge_shapes_bit_exact(moe, E, k, C, N, scale):
    g = torch.Generator().manual_seed(E * 1000 + N)
    logits = (torch.randn((N, E), generator=g) * scale)
    # quantise half the rows so that exact ties occur
    logits[::2] = torch.round(logits[::2] * 2) / 2
    bias = (torch.rand(E, generator=g) * 0.02 - 0.01) if E % 2 == 0 else None
    ref = oracle.route(logits.numpy(), k, C, True, None if bias is None else bias.numpy())
    dev = logits.cuda()
    cand = torch.empty((N, C), dtype=torch.int32, device="cuda")
    cs = torch.empty((N, C), dtype=torch.float32, device="cuda")
    gates = torch.empty((N, k), dtype=torch.float32, device="cuda")
    sums = torch.empty(E + 1, dtype=torch.float64, device="cuda")
    wg = torch.zeros((E, 8), device="cuda")
    moe.moe_router_topk(None, wg, top_k=k, n_cand=C, renormalize=True,
                        select_bias=None if bias is None else bias.cuda(), logits_in=dev,
                        cand_ids=cand, cand_scores=cs, gates=gates, score_sums=sums)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(cand), ref["cand_ids"])
    assert np.array_equal(to_np(cs).view(np.uint32), ref["cand_scores"].view(np.uint32))
    assert np.array_equal(to_np(gates).view(np.uint32), ref["gates"].view(np.uint32))
    I = ref["s"].astype(np.float64).sum(axis=0)
    assert np.allclose(to_np(sums)[:E], I, rtol=1e-12, atol=1e-300)
    assert abs(to_np(sums)[E] - np.sum(ref["lse"] ** 2)) <= 1e-6 * np.sum(ref["lse"] ** 2)


def _dispatch_gpu(moe, cand, cs, gates, E, k, policy, cap, x=None):
    N, C = cand.shape
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(counts_routed=torch.empty(E, **i32), counts_kept=torch.empty(E, **i32),
               offsets=torch.empty(E + 1, **i32), row_of=torch.empty((N, k), **i32),
               expert_of=torch.empty((N, k), **i32),
               perm_token=torch.full((N * k,), -7, **i32))
    g = torch.from_numpy(gates.copy()).cuda()
    xp = None if x is None else torch.empty((N * k, x.shape[1]), dtype=x.dtype, device="cuda")
    moe.moe_dispatch(torch.from_numpy(cand).cuda(), torch.from_numpy(cs).cuda(), g,
                     n_experts=E, top_k=k, policy=policy, capacity=cap, x=x, x_perm=xp, **out)
    torch.cuda.synchronize()
    res = {kk: to_np(v) for kk, v in out.items()}
    res["gates"] = to_np(g)
    res["x_perm"] = xp
    return res


@pytest.mark.parametrize("N,E,k,policy,cf", [(4096, 8, 2, W.DROPLESS, None),
                                             (3000, 64, 8, W.DROP, 1.0),
                                             (16384, 64, 1, W.REROUTE_THEN_DROP, 1.0),
                                             (777, 256, 8, W.DROPLESS, None),
                                             (1, 4, 1, W.DROP, 1.0),
                                             (513, 7, 3, W.DROP, 0.5)])
def test_dispatch_bit_exact(moe, N, E, k, policy, cf):
    g = torch.Generator().manual_seed(N + E)
    skew = torch.tensor([-1.1 * np.log(e + 1) for e in range(E)], dtype=torch.float32)
    logits = torch.randn((N, E), generator=g) + skew
    C = k + 1 if policy == W.REROUTE_THEN_DROP else k
    r = oracle.route(logits.numpy(), k, C, policy == W.DROPLESS)
    cap = -1 if cf is None else moe.capacity(N, E, cf)
    ref = oracle.dispatch(r["cand_ids"], r["cand_scores"], r["gates"], E, k, policy, cap)
    got = _dispatch_gpu(moe, r["cand_ids"], r["cand_scores"], r["gates"], E, k, policy, cap)
    for name in ("counts_routed", "counts_kept", "offsets", "row_of", "expert_of"):
        assert np.array_equal(got[name], ref[name]), name
    assert np.array_equal(got["perm_token"][:ref["R"]], ref["perm_token"])
    assert np.array_equal(got["gates"].view(np.uint32), ref["gates"].view(np.uint32))


def test_dispatch_forced_collapse(moe):
    # every token to expert 0: kept = capacity, kept tokens are exactly 0..cap-1
    N, E = 256, 4
    cap = moe.capacity(N, E, 1.25)
    cand = np.zeros((N, 1), np.int32)
    cs = np.ones((N, 1), np.float32)
    got = _dispatch_gpu(moe, cand, cs, cs.copy(), E, 1, W.DROP, cap)
    assert got["counts_kept"].tolist() == [cap, 0, 0, 0]
    assert np.nonzero(got["row_of"][:, 0] >= 0)[0].tolist() == list(range(cap))
    assert np.all(got["gates"][cap:] == 0)


@pytest.mark.parametrize("key", ["c2", "c4", "c5", "c1"])
def test_grouped_ffn_ragged_with_empty_experts(moe, key):
    """Grouped FFN alone on hand-made ragged row counts (some experts empty,
    one with a single row, one larger than a tile)."""
    cfg = W.REDUCED[key]
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    dev = to_device(inp)
    E = cfg.n_experts
    rng = np.random.default_rng(3)
    counts = rng.integers(0, 40, size=E)
    counts[0] = 0
    counts[-1] = 0
    counts[1 % E] = 1
    counts[2 % E] = 300
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    tok = rng.integers(0, cfg.n_tokens, size=R)
    x = dev["x"][torch.from_numpy(tok).cuda()].contiguous()
    ydt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    y = torch.full((R + 5, cfg.d_model), 7.0, dtype=ydt, device="cuda")
    w, keep = moe.ffn_weights(dev["w1"], dev["w2"], dev["w3"], cfg.act, dev["b1"], dev["b2"],
                              dev["s1"], dev["s3"], dev["s2"])
    moe.moe_grouped_ffn(w, x, torch.from_numpy(offs).cuda(), y, max_rows=R)
    torch.cuda.synchronize()
    X64 = oracle.decode_rows(host["x"][tok], cfg.x_dtype)
    experts = np.repeat(np.arange(E), counts)
    ref = oracle.ffn_for_assignments(np.arange(R), experts, X64, cfg.act, cfg.w_dtype,
                                     experts_of(host))
    got = to_np(y)
    assert rel_err(got[:R], ref) <= out_tol(cfg)
    assert np.all(got[R:] == 7.0)  # rows past offsets[E] untouched


def test_combine_matches_oracle(moe):
    rng = np.random.default_rng(8)
    N, d, k = 50, 256, 3
    R = N * k
    perm = rng.permutation(R).astype(np.int32)
    row_of = perm.reshape(N, k).copy()
    row_of[rng.random((N, k)) < 0.2] = -1
    row_of[5] = -1  # a token whose assignments all dropped
    gates = rng.random((N, k)).astype(np.float32)
    yr = torch.randn((R, d)).to(torch.bfloat16)
    ysh = torch.randn((N, d)).to(torch.bfloat16)
    out = torch.empty((N, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(yr.cuda(), torch.from_numpy(row_of).cuda(), torch.from_numpy(gates).cuda(),
                    out, y_shared=ysh.cuda())
    torch.cuda.synchronize()
    yr64 = yr.double().numpy()
    Yexp = np.zeros((N, k, d))
    for t in range(N):
        for j in range(k):
            if row_of[t, j] >= 0:
                Yexp[t, j] = yr64[row_of[t, j]]
    ref = oracle.combine(row_of, gates, Yexp, ysh.double().numpy())
    assert rel_err(to_np(out), ref) <= 2e-2
    # fp32 output: only fp32 rounding
    out32 = torch.empty((N, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(yr.cuda(), torch.from_numpy(row_of).cuda(), torch.from_numpy(gates).cuda(),
                    out32, y_shared=ysh.cuda())
    torch.cuda.synchronize()
    assert rel_err(to_np(out32), ref) <= 1e-6


def test_bias_update_and_stats_closed_forms(moe):
    N, E, k = 12, 4, 2
    routed = torch.tensor([9, 6, 3, 6], dtype=torch.int32, device="cuda")
    kept = routed.clone()
    sums = torch.tensor([3.0, 3.0, 3.0, 3.0, 0.0], dtype=torch.float64, device="cuda")
    bias = torch.tensor([0.0, 0.5, -0.25, 1e-3], dtype=torch.float32, device="cuda")
    f = torch.empty(E, device="cuda")
    P = torch.empty(E, device="cuda")
    sc = torch.empty(4, device="cuda")
    moe.moe_balance_stats(N, k, routed, kept, sums, f, P, sc, select_bias=bias, bias_rate=1e-3)
    torch.cuda.synchronize()
    ref_b = oracle.bias_update(N, k, np.array([9, 6, 3, 6]), np.array([0.0, 0.5, -0.25, 1e-3]),
                               1e-3)
    assert np.array_equal(to_np(bias).view(np.uint32), ref_b.view(np.uint32))
    assert np.allclose(to_np(f), [9 / 24, 6 / 24, 3 / 24, 6 / 24])
    assert abs(to_np(sc)[0] - 1.0) < 1e-6 and to_np(sc)[1] == 0.0 and to_np(sc)[3] == 0.0


@pytest.mark.parametrize("key", ["c3", "c4"])
def test_deterministic_bitwise(moe, key):
    cfg = W.REDUCED[key]
    dev = to_device(W.make_inputs(cfg, "cpu"))
    layer = _layer(moe, cfg, dev)
    outs = []
    for _ in range(2):
        y = layer.forward(dev["x"]).clone()
        outs.append((y, layer.row_of.clone(), layer.score_sums.clone(), layer.scalars.clone()))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


def test_dropped_token_passes_residual(moe):
    # a dropped token's layer output is 0, so x + y == x exactly
    cfg = W.C1.with_(n_tokens=64, capacity_factor=0.25)
    inp = W.make_inputs(cfg, "cpu")
    dev = to_device(inp)
    layer = _layer(moe, cfg, dev)
    y = layer.forward(dev["x"])
    torch.cuda.synchronize()
    dropped = to_np(layer.row_of)[:, 0] < 0
    assert dropped.sum() >= 64 - 4 * moe.capacity(64, 4, 0.25)
    x = dev["x"]
    assert torch.equal((x + y)[torch.from_numpy(dropped).cuda()],
                       x[torch.from_numpy(dropped).cuda()])


def test_abi_errors_leave_outputs_untouched(moe):
    N, E, k = 16, 4, 2
    cand = torch.full((N, k), -5, dtype=torch.int32, device="cuda")
    cs = torch.full((N, k), -5.0, device="cuda")
    gates = torch.full((N, k), -5.0, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_router_topk(None, torch.zeros((E, 8), device="cuda"), top_k=5, n_cand=5,
                            logits_in=torch.zeros((N, E), device="cuda"), cand_ids=cand,
                            cand_scores=cs, gates=gates)
    assert ei.value.status == 1
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_router_topk(None, torch.zeros((E, 8), device="cuda"), top_k=2, n_cand=2,
                            logits_in=torch.zeros((N, E), device="cuda"), cand_ids=cand,
                            cand_scores=cs, gates=gates,
                            ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(cand == -5) and torch.all(gates == -5.0)


def test_grouped_ffn_fp32_intermediate_is_tighter(moe):
    """With h kept in fp32 (GEMM 2 as hi + lo bf16 passes) the grouped FFN
    error falls well below the bf16-h error (about 2^-9 relative per h
    element), down to the fp32 accumulation level."""
    cfg = W.REDUCED["c4"]
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    dev = to_device(inp)
    E = cfg.n_experts
    counts = np.full(E, 37)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    tok = np.arange(R) % cfg.n_tokens
    x = dev["x"][torch.from_numpy(tok).cuda()].contiguous()
    X64 = oracle.decode_rows(host["x"][tok], cfg.x_dtype)
    ref = oracle.ffn_for_assignments(np.arange(R), np.repeat(np.arange(E), counts), X64,
                                     cfg.act, cfg.w_dtype, experts_of(host))
    errs = {}
    for h32 in (False, True):
        y = torch.empty((R, cfg.d_model), dtype=torch.float32, device="cuda")
        w, keep = moe.ffn_weights(dev["w1"], dev["w2"], dev["w3"], cfg.act, h_fp32=h32)
        moe.moe_grouped_ffn(w, x, torch.from_numpy(offs).cuda(), y, max_rows=R)
        torch.cuda.synchronize()
        errs[h32] = rel_err(to_np(y), ref)
    print("bf16 h:", errs[False], " fp32 h:", errs[True])
    assert errs[True] <= 1e-3 and errs[True] < errs[False] / 8


@pytest.mark.parametrize("d_model", [192, 256, 320, 512])
def test_grouped_ffn_fp32_h_column_tilings(moe, d_model):
    """GEMM 2 with fp32 h (hi + lo bf16 planes) on 128-row tiles runs
    256-column tiles when d_model is a multiple of 256 (256, 512) and
    64-column tiles otherwise (192, 320). Ragged experts (empty ones, a
    single row, one past a tile), rows gathered through a row index; both
    tilings reach the fp32-h bar, and rows past offsets[E] stay untouched."""
    cfg = W.REDUCED["c4"].with_(name="switch_fp32h_d%d" % d_model, d_model=d_model)
    print("fp32 h, d_model", d_model, flush=True)
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    dev = to_device(inp)
    E = cfg.n_experts
    rng = np.random.default_rng(d_model)
    counts = rng.integers(0, 60, size=E)
    counts[0] = 0
    counts[3] = 1
    counts[5] = 200
    counts[-1] = 0
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    tok = rng.integers(0, cfg.n_tokens, size=R)
    y = torch.full((R + 3, d_model), 7.0, dtype=torch.float32, device="cuda")
    w, keep = moe.ffn_weights(dev["w1"], dev["w2"], dev["w3"], cfg.act, h_fp32=True)
    moe.moe_grouped_ffn(w, dev["x"], torch.from_numpy(offs).cuda(), y,
                        row_index=torch.from_numpy(tok.astype(np.int32)).cuda(), max_rows=R)
    torch.cuda.synchronize()
    X64 = oracle.decode_rows(host["x"][tok], cfg.x_dtype)
    ref = oracle.ffn_for_assignments(np.arange(R), np.repeat(np.arange(E), counts), X64,
                                     cfg.act, cfg.w_dtype, experts_of(host))
    got = to_np(y)
    assert rel_err(got[:R], ref) <= 1e-3
    assert np.all(got[R:] == 7.0)


@pytest.mark.parametrize("key", ["c2", "c4", "c5", "c1"])
def test_fused_gather_matches_explicit_gather(moe, key):
    """GEMM 1 reading token rows through perm_token gives bit-identical
    outputs to gathering x_perm first in dispatch."""
    cfg = W.REDUCED[key]
    dev = to_device(W.make_inputs(cfg, "cpu"))
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    outs = []
    for fused in (False, True):
        layer = moe.MoELayer(moe.spec_from_config(cfg), dev, x_dtype=xdt, fused_gather=fused)
        outs.append(layer.forward(dev["x"]).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("gather", [False, True])
def test_fp8_stream_and_row_group_paths(moe, gather):
    """fp8 weights, few rows per expert: the streaming path (16-row tiles,
    chosen while max_rows <= 8 per expert) and the 64-row-group path (forced
    by a larger max_rows) on the same ragged counts, including experts that
    span one, two and three 16-row tiles. Both match the oracle, agree
    bitwise with each other (same MFMA accumulation order), and leave rows
    past offsets[E] untouched."""
    cfg = W.REDUCED["c5"]
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    dev = to_device(inp)
    E, d = cfg.n_experts, cfg.d_model
    rng = np.random.default_rng(11)
    counts = rng.integers(0, 9, size=E)
    counts[0] = 0
    counts[-1] = 0
    counts[1], counts[2], counts[3], counts[4] = 1, 16, 17, 40
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    assert R <= 8 * E
    tok = rng.integers(0, cfg.n_tokens, size=R)
    w, keep = moe.ffn_weights(dev["w1"], dev["w2"], dev["w3"], cfg.act, None, None,
                              dev["s1"], dev["s3"], dev["s2"])
    X64 = oracle.decode_rows(host["x"][tok], cfg.x_dtype)
    experts = np.repeat(np.arange(E), counts)
    ref = oracle.ffn_for_assignments(np.arange(R), experts, X64, cfg.act, cfg.w_dtype,
                                     experts_of(host))
    outs = []
    for max_rows in (R, 8 * E + 1):
        idx = np.zeros(max_rows, np.int32)
        idx[:R] = tok
        if gather:
            x_rows = dev["x"]
            row_index = torch.from_numpy(idx).cuda()
        else:
            x_rows = dev["x"][torch.from_numpy(idx).long().cuda()].contiguous()
            row_index = None
        y = torch.full((max_rows, d), 7.0, dtype=torch.float32, device="cuda")
        moe.moe_grouped_ffn(w, x_rows, torch.from_numpy(offs).cuda(), y, row_index=row_index,
                            max_rows=max_rows)
        torch.cuda.synchronize()
        got = to_np(y)
        assert rel_err(got[:R], ref) <= TOL_FP8, max_rows
        assert np.all(got[R:] == 7.0)
        outs.append(y[:R].clone())
    assert torch.equal(outs[0], outs[1])


def test_grouped_ffn_256_row_tiles_with_tails(moe):
    """Experts averaging over 512 rows take 256-row M tiles for their full
    tiles and 128-row tiles for the rest; counts cover a multiple of 256 (no
    tail), a 1-row tail, a tail of one and of two 128-row tiles, an expert
    smaller than one tile and an empty one."""
    cfg = W.REDUCED["c2"]
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    dev = to_device(inp)
    E = cfg.n_experts
    counts = np.array([0, 768, 513, 1100, 700, 520, 1, 600])
    assert len(counts) == E and counts.sum() >= 512 * E
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    rng = np.random.default_rng(5)
    tok = rng.integers(0, cfg.n_tokens, size=R)
    w, keep = moe.ffn_weights(dev["w1"], dev["w2"], dev["w3"], cfg.act, None, None)
    y = torch.full((R + 3, cfg.d_model), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(w, dev["x"], torch.from_numpy(offs).cuda(), y,
                        row_index=torch.from_numpy(tok.astype(np.int32)).cuda(), max_rows=R)
    torch.cuda.synchronize()
    X64 = oracle.decode_rows(host["x"][tok], cfg.x_dtype)
    experts = np.repeat(np.arange(E), counts)
    ref = oracle.ffn_for_assignments(np.arange(R), experts, X64, cfg.act, cfg.w_dtype,
                                     experts_of(host))
    got = to_np(y)
    assert rel_err(got[:R], ref) <= out_tol(cfg)
    assert np.all(got[R:] == 7.0)


def test_grouped_ffn_256_row_tiles_partial_blocks(moe):
    """Long-K experts averaging 256-511 rows run 256-row tiles without a
    tail launch; the last tile's unused 32-row blocks skip their MFMAs.
    Tails of 44, 1 and 254 rows, one expert of exactly 256, one empty."""
    cfg = W.REDUCED["c2"].with_(name="long_k_256", n_tokens=600, d_model=4096, d_ff=256,
                                n_experts=5)
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    dev = to_device(inp)
    E = cfg.n_experts
    counts = np.array([300, 257, 0, 510, 256])
    assert 256 <= counts.sum() // E < 512
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    rng = np.random.default_rng(9)
    tok = rng.integers(0, cfg.n_tokens, size=R)
    w, keep = moe.ffn_weights(dev["w1"], dev["w2"], dev["w3"], cfg.act, None, None)
    y = torch.full((R + 3, cfg.d_model), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(w, dev["x"], torch.from_numpy(offs).cuda(), y,
                        row_index=torch.from_numpy(tok.astype(np.int32)).cuda(), max_rows=R)
    torch.cuda.synchronize()
    X64 = oracle.decode_rows(host["x"][tok], cfg.x_dtype)
    experts = np.repeat(np.arange(E), counts)
    ref = oracle.ffn_for_assignments(np.arange(R), experts, X64, cfg.act, cfg.w_dtype,
                                     experts_of(host))
    got = to_np(y)
    assert rel_err(got[:R], ref) <= out_tol(cfg)
    assert np.all(got[R:] == 7.0)
