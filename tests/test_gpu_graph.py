"""A whole layer forward captured as a HIP graph (MoELayer.capture) replays
to the eager result bit for bit: several replays, with eager forwards on
other inputs (which overwrite every buffer the graph uses) between them."""
import numpy as np
import pytest
import torch

import workloads as W
from parity_utils import require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    require_gpu()
    import sparse_mixture_experts_47_amd as m
    return m


@pytest.mark.parametrize("key", ["c1", "c3", "c4", "c5", "c6", "c2_tails"])
def test_graph_replay_equals_eager(moe, key):
    # c2_tails: 525 rows per expert on average, so the grouped FFN runs
    # 256-row tiles plus the tail launches of experts' last rows
    cfg = W.REDUCED["c2"].with_(n_tokens=2100) if key == "c2_tails" else W.REDUCED[key]
    print("graph", key, cfg.name, flush=True)
    inp = W.make_inputs(cfg, "cpu")
    dev = to_device(inp)
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    layer = moe.MoELayer(moe.spec_from_config(cfg), dev, x_dtype=xdt)
    x = dev["x"]
    x2 = torch.flip(x, dims=[0]).contiguous()
    y0 = layer.forward(x).clone()
    sc0 = layer.scalars.clone()
    torch.cuda.synchronize()
    g = layer.capture(x)
    for i in range(3):
        layer.forward(x2)  # eager work on other data between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, y0), (key, i)
        assert torch.equal(layer.scalars, sc0), (key, i)
    # and eager after the graph still matches too
    assert torch.equal(layer.forward(x), y0)
