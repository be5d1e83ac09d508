"""Seeded synthetic inputs for the sparse MoE FFN layer forward.

This module only draws and stores inputs: random activations, router and
expert weights, biases, and the fp8 storage format of weights. It holds none
of the layer's arithmetic (no routing, no softmax, no FFN), so that both the
CPU oracle and the GPU path can take their inputs from it without sharing any
computation.

Workload shapes follow the model families the pages name: Switch top-1,
Mixtral-style top-2, DeepSeek-style fine-grained experts plus a shared expert
("[CS336-04] Mixture of Experts", section 3 and section 5; "MoE" Q4 on
ld246.com). The sizes themselves are synthetic choices of this library.

Every tensor has its own torch generator seeded from (config seed, tensor id,
expert index), so a tensor can be drawn alone, on CPU or on a GPU device, and
experts can be drawn one at a time to bound memory. The same seed gives the
same numbers on the same device type; CPU and GPU draws differ, which is
fine because a test always hands one draw to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import torch

# Activation ids and overflow-policy ids, same numbering as the C ABI.
ACT_RELU, ACT_GELU, ACT_SWIGLU = 0, 1, 2
DROPLESS, DROP, REROUTE_THEN_DROP = 0, 1, 2
# dtype ids, same numbering as the C ABI.
F32, BF16, FP8_E4M3 = 0, 1, 2

E4M3_MAX = 448.0  # largest finite OCP E4M3FN magnitude


@dataclass(frozen=True)
class MoEConfig:
    """One MoE layer workload. Dimensions follow the usual names:
    N tokens, d = d_model, E routed experts, d_ff per expert, top-k."""
    name: str
    n_tokens: int
    d_model: int
    n_experts: int
    d_ff: int
    top_k: int
    act: int                       # ACT_*
    x_dtype: int                   # F32 or BF16 (activations)
    w_dtype: int                   # F32, BF16 or FP8_E4M3 (expert weights)
    renormalize: bool              # True: gates = top-k scores / their sum
    overflow: int = DROPLESS       # DROPLESS, DROP, REROUTE_THEN_DROP
    capacity_factor: Optional[float] = None  # None = dropless; read as the decimal it prints as
    ffn_bias: bool = False         # b1/b2 present (C1)
    shared_d_ff: int = 0           # 0 = no shared expert
    select_bias: bool = False      # per-expert selection bias (loss-free balancing)
    zipf_s: Optional[float] = None # per-expert logit offset -s*ln(e+1)
    noisy: bool = False            # noisy top-k gating
    seed: int = 0
    weight_seed: Optional[int] = None  # seed for expert weights (C5 reuses C3's)
    noise_seed: int = 0
    router_std: float = 0.02
    # keep the FFN intermediate h in fp32 (GEMM 2 as hi+lo bf16 passes); used
    # where the layer is bound by weight reads and MFMA time is spare
    h_fp32: bool = False
    # expert-choice routing: every expert takes a fixed number of its top
    # tokens (top_k then only sets the average load per expert)
    expert_choice: bool = False

    @property
    def n_cand(self) -> int:
        return self.top_k + 1 if self.overflow == REROUTE_THEN_DROP else self.top_k

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads. Sizes are synthetic, shaped like the model families the
# pages list (Switch top-1; Mixtral top-2; DeepSeek fine-grained + shared).
C1 = MoEConfig("switch_tiny_top1", 256, 64, 4, 256, 1, ACT_RELU, F32, F32, False,
               overflow=DROP, capacity_factor=1.25, ffn_bias=True, seed=1)
C2 = MoEConfig("mixtral_prefill_top2", 4096, 4096, 8, 14336, 2, ACT_SWIGLU, BF16, BF16,
               True, seed=2)
C3 = MoEConfig("deepseek_prefill_top8_shared", 8192, 7168, 256, 2048, 8, ACT_SWIGLU, BF16,
               BF16, True, shared_d_ff=2048, select_bias=True, seed=3)
C4 = MoEConfig("switch_skewed_top1_capacity", 16384, 1024, 64, 4096, 1, ACT_GELU, BF16, BF16,
               False, overflow=REROUTE_THEN_DROP, capacity_factor=1.0, zipf_s=1.1,
               noisy=True, seed=4, noise_seed=44, h_fp32=True)
C5 = MoEConfig("deepseek_decode_fp8", 64, 7168, 256, 2048, 8, ACT_SWIGLU, BF16, FP8_E4M3,
               True, shared_d_ff=2048, seed=5, weight_seed=3)

# Expert-choice variant of the Mixtral-shaped prefill: same shapes, every
# expert takes N * 2 / 8 = 1024 tokens.
C6 = C2.with_(name="mixtral_prefill_expert_choice", expert_choice=True, seed=6)

# One GPU's share of the DeepSeek-shaped layer under 8-way expert parallelism:
# 32 of the 256 experts live on the GPU, and the tokens of all eight GPUs that
# route there arrive packed, about 8192 * 8 / 32 = 2048 rows per expert. Here
# the GPU's own 8192 tokens route top-8 over its 32 experts, which gives the
# grouped FFN that same shape (the exchange itself is not modelled); the
# shared expert runs on the local tokens as in the full layer.
C7 = C3.with_(name="deepseek_ep8_local_share", n_experts=32, seed=7)

CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5, "c6": C6, "c7": C7}

# Reduced shapes of the same recipes: small enough for the fp64 oracle to run
# in seconds, large enough to span several GEMM tiles with ragged tails.
REDUCED = {
    "c1": C1,
    "c2": C2.with_(name="mixtral_reduced", n_tokens=600, d_model=512, d_ff=1024),
    "c3": C3.with_(name="deepseek_reduced", n_tokens=320, d_model=512, n_experts=64,
                   d_ff=256, shared_d_ff=256),
    "c4": C4.with_(name="switch_skewed_reduced", n_tokens=2000, d_model=256, n_experts=16,
                   d_ff=512),
    "c5": C5.with_(name="deepseek_decode_reduced", n_tokens=24, d_model=512, n_experts=64,
                   d_ff=256, shared_d_ff=256),
    "c6": C6.with_(name="expert_choice_reduced", n_tokens=600, d_model=512, d_ff=1024),
}

# tensor ids used to derive per-tensor seeds
_T_X, _T_WG, _T_W1, _T_W3, _T_W2, _T_B1, _T_B2, _T_SEL, _T_WN = range(9)
_T_SH1, _T_SH3, _T_SH2 = 20, 21, 22


def _gen(device, *key) -> torch.Generator:
    s = 0
    for k in key:
        s = (s * 1_000_003 + int(k) + 1) % (2**62)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, std, device, *key) -> torch.Tensor:
    g = _gen(device, *key)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_e4m3_rows(w: torch.Tensor):
    """Store a [rows][cols] fp32 weight as OCP E4M3FN codes with one fp32 scale
    per row (per output channel): scale = amax(row)/448, code = RNE(w/scale).
    Returns (uint8 codes, fp32 scales). Storage format of the workload only."""
    amax = w.abs().amax(dim=1).clamp_min(1e-30)
    scale = (amax / E4M3_MAX).to(torch.float32)
    q = (w / scale[:, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def _store(w32: torch.Tensor, dtype: int):
    if dtype == F32:
        return w32, None
    if dtype == BF16:
        return w32.to(torch.bfloat16), None
    if dtype == FP8_E4M3:
        return quantize_e4m3_rows(w32)
    raise ValueError(dtype)


def _expert_stack(cfg: MoEConfig, device, tid: int, rows: int, cols: int, fan_in: int,
                  n_experts: int, wseed: int):
    """Draw [n_experts][rows][cols] one expert at a time in the storage dtype."""
    std = 1.0 / math.sqrt(fan_in)
    out, scales = None, None
    for e in range(n_experts):
        w32 = _normal((rows, cols), std, device, wseed, tid, e)
        w, s = _store(w32, cfg.w_dtype)
        del w32
        if out is None:
            out = torch.empty((n_experts, rows, cols), dtype=w.dtype, device=device)
            if s is not None:
                scales = torch.empty((n_experts, rows), dtype=torch.float32, device=device)
        out[e].copy_(w)
        if s is not None:
            scales[e].copy_(s)
    return out, scales


def make_inputs(cfg: MoEConfig, device="cpu") -> dict:
    """All inputs of one layer forward for `cfg`, drawn on `device`.

    Keys: x [N][d]; w_gate [E][d] fp32; logit_bias [E] or None; select_bias [E]
    or None; w_noise [E][d] or None; w1, w3 (SwiGLU only), w2 expert weights
    [E][d_ff][d], [E][d_ff][d], [E][d][d_ff]; s1, s3, s2 per-output-channel fp8
    scales or None; b1 [E][d_ff], b2 [E][d] or None; shared_{w1,w3,w2,s1,s3,s2}
    for the always-on expert (one expert, same layout) or None.
    """
    N, d, E, F = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.d_ff
    seed = cfg.seed
    wseed = cfg.weight_seed if cfg.weight_seed is not None else seed
    inp = {}
    x = _normal((N, d), 1.0, device, seed, _T_X)
    inp["x"] = x.to(torch.bfloat16) if cfg.x_dtype == BF16 else x
    inp["w_gate"] = _normal((E, d), cfg.router_std, device, seed, _T_WG)
    if cfg.zipf_s is not None:
        e = torch.arange(E, dtype=torch.float64, device=device)
        inp["logit_bias"] = (-cfg.zipf_s * torch.log(e + 1.0)).to(torch.float32)
    else:
        inp["logit_bias"] = None
    if cfg.select_bias:
        g = _gen(device, seed, _T_SEL)
        inp["select_bias"] = (torch.rand((E,), generator=g, device=device) * 0.02 - 0.01)
    else:
        inp["select_bias"] = None
    inp["w_noise"] = (_normal((E, d), cfg.router_std, device, seed, _T_WN)
                      if cfg.noisy else None)

    inp["w1"], inp["s1"] = _expert_stack(cfg, device, _T_W1, F, d, d, E, wseed)
    if cfg.act == ACT_SWIGLU:
        inp["w3"], inp["s3"] = _expert_stack(cfg, device, _T_W3, F, d, d, E, wseed)
    else:
        inp["w3"], inp["s3"] = None, None
    inp["w2"], inp["s2"] = _expert_stack(cfg, device, _T_W2, d, F, F, E, wseed)
    if cfg.ffn_bias:
        inp["b1"] = _normal((E, F), 1.0 / math.sqrt(d), device, wseed, _T_B1)
        inp["b2"] = _normal((E, d), 1.0 / math.sqrt(F), device, wseed, _T_B2)
    else:
        inp["b1"], inp["b2"] = None, None

    Fs = cfg.shared_d_ff
    if Fs:
        scfg = cfg.with_(d_ff=Fs)
        w1, s1 = _expert_stack(scfg, device, _T_SH1, Fs, d, d, 1, wseed)
        w3, s3 = _expert_stack(scfg, device, _T_SH3, Fs, d, d, 1, wseed)
        w2, s2 = _expert_stack(scfg, device, _T_SH2, d, Fs, Fs, 1, wseed)
        inp.update(shared_w1=w1, shared_w3=w3, shared_w2=w2,
                   shared_s1=s1, shared_s3=s3, shared_s2=s2)
    else:
        inp.update(shared_w1=None, shared_w3=None, shared_w2=None,
                   shared_s1=None, shared_s3=None, shared_s2=None)
    return inp


def uniform_logits(n_tokens: int, n_experts: int, std: float, seed: int, device="cpu"):
    """Random fp32 router logits [N][E] ~ N(0, std^2), for routing-only cases."""
    return _normal((n_tokens, n_experts), std, device, seed, 99)


def bits_u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
