"""Degenerate batch sizes through the whole layer: one token and a few
tokens (ragged against every tile size), for every workload recipe, token
choice and expert choice, forward (routing bit-exact from the oracle's
logits, outputs within the dtype's bar) and, for the training shapes, the
backward's expert weight gradients against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import backward as OB
from parity_utils import (experts_of, host_inputs, out_tol, rel_err, require_gpu, to_device,
                          to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    require_gpu()
    import sparse_mixture_experts_47_amd as m
    return m


def _forward(moe, cfg, train=False):
    inp = W.make_inputs(cfg, "cpu")
    host = host_inputs(inp)
    shared = experts_of(host, "shared_") if cfg.shared_d_ff else None
    ref = oracle.layer_forward(cfg, host["x"], cfg.x_dtype, host["w_gate"], experts_of(host),
                               shared, host["logit_bias"], host["select_bias"], host["w_noise"])
    dev = to_device(inp)
    spec = moe.spec_from_config(cfg)
    if train:
        spec.h_fp32 = False
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    layer = moe.MoELayer(spec, dev, x_dtype=xdt, train=train)
    noise_in = None
    if train and host["w_noise"] is not None:
        X = oracle.decode_rows(host["x"], cfg.x_dtype)
        noise_in = torch.from_numpy((X @ host["w_noise"].astype(np.float64).T)
                                    .astype(np.float32)).cuda()
    y = layer.forward(dev["x"], logits_in=torch.from_numpy(ref["logits"]).cuda(),
                      noise_in=noise_in)
    torch.cuda.synchronize()
    return host, ref, dev, layer, y


@pytest.mark.parametrize("N", [1, 2, 3, 7])
@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5", "c6"])
def test_tiny_batches_forward(moe, key, N):
    cfg = W.REDUCED[key].with_(n_tokens=N)
    print("edge", key, N, flush=True)
    host, ref, dev, layer, y = _forward(moe, cfg)
    if cfg.expert_choice:
        ec = ref["ec"]
        assert np.array_equal(to_np(layer.row_of), ec["row_of"])
        assert np.array_equal(to_np(layer.perm_token), ec["perm_token"])
    else:
        d = ref["dispatch"]
        assert np.array_equal(to_np(layer.cand_ids), ref["route"]["cand_ids"])
        assert np.array_equal(to_np(layer.row_of), d["row_of"])
        assert np.array_equal(to_np(layer.counts_kept), d["counts_kept"])
        assert np.array_equal(to_np(layer.perm_token)[:d["R"]], d["perm_token"])
    err = rel_err(to_np(y), ref["y"])
    assert err <= out_tol(cfg), err
    sc = to_np(layer.scalars)
    for i, name in enumerate(("switch_aux", "importance_cv2", "z_loss", "drop_rate")):
        assert abs(sc[i] - ref["stats"][name]) <= 1e-5 * abs(ref["stats"][name]) + 1e-7, name


@pytest.mark.parametrize("N", [1, 3])
@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c6"])
def test_tiny_batches_backward(moe, key, N):
    """The backward of a one- or three-token batch (most experts get no rows:
    their weight gradients must be exactly zero), held to the element-wise
    derived bounds and the router-side statistical bounds of the full
    backward tests."""
    from test_gpu_backward import _check_bounds, _check_router_statistical, _ec_view
    cfg = W.REDUCED[key].with_(n_tokens=N)
    print("edge backward", key, N, flush=True)
    host, ref, dev, layer, y = _forward(moe, cfg, train=True)
    shared = experts_of(host, "shared_") if cfg.shared_d_ff else None
    dy = torch.randn((N, cfg.d_model), generator=torch.Generator().manual_seed(N))
    dy64 = dy.numpy().astype(np.float64)
    gref = OB.layer_backward(cfg, host["x"], cfg.x_dtype, host["w_gate"], experts_of(host), ref,
                             dy64, 0.1, 0.01, shared=shared, logit_bias=host["logit_bias"],
                             w_noise=host["w_noise"], keep_terms=True)
    g = moe.layer_backward(layer, dev["x"], dy.cuda(), 0.1, 0.01)
    torch.cuda.synchronize()
    counts = to_np(layer.counts_kept)
    for n in ("dw1", "dw2"):
        G = to_np(g[n])
        for e in np.nonzero(counts == 0)[0]:
            assert not G[e].any(), (n, e)
    cfg_v, ref_v = (_ec_view(cfg, ref) if cfg.expert_choice else (cfg, ref))
    _check_bounds(g, gref, ref_v, dy64, host, cfg_v)
    _check_router_statistical(g, gref, ref_v, dy64, host, cfg_v)
