"""Benchmark: one MoE FFN layer forward per step on one MI355X, through libmoe.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c1|c3|c4|c5]

A step is one pass of the whole layer: router GEMM + fp32 softmax + top-k,
dispatch (capacity, packing, row gather), the grouped expert FFN (+ shared
expert), the gate-weighted combine, and the balance statistics. Inputs are
synthetic (seeded, drawn on the GPU) and resident in HBM before timing.
Prints one JSON line. The default workload is the Mixtral-shaped prefill
(4096 tokens, d_model 4096, 8 experts of d_ff 14336 SwiGLU, top-2, bf16).

roofline: the grouped expert FFN (moe_grouped_ffn: tile table + GEMM 1
gate/up with fused SwiGLU + GEMM 2 down) is the dominant kernel group; its
duration is measured with HIP events on the launch stream inside the timed
region. cpu_baseline: the CPU oracle (fp64 FFNs) timed on a bounded sample of
the same workload on this host's cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + grouped-GEMM % MFMA peak / decode % HBM peak, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: choose by workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def ffn_work(cfg, counts_kept, touched):
    """Algorithmic FLOPs and bytes of the grouped expert FFN for one forward.
    FLOPs: 2 d F per matrix per kept assignment (3 matrices for SwiGLU, 2
    otherwise), plus the shared expert on every token. Bytes: every touched
    expert's weights once (+ per-channel scales for fp8), the packed rows in
    and out, and h written and read once."""
    d, F = cfg.d_model, cfg.d_ff
    nmat = 3 if cfg.act == 2 else 2
    R = int(sum(counts_kept))
    flops = 2.0 * d * F * nmat * R
    wbytes_el = {0: 4, 1: 2, 2: 1}[cfg.w_dtype]
    xbytes = 4 if cfg.x_dtype == 0 else 2
    wbytes = touched * nmat * d * F * wbytes_el
    if cfg.w_dtype == 2:
        wbytes += touched * 4 * ((nmat - 1) * F + d)
    act_bytes = R * d * xbytes * 2 + R * F * xbytes * 2
    if cfg.shared_d_ff:
        Fs = cfg.shared_d_ff
        flops += 2.0 * d * Fs * 3 * cfg.n_tokens
        wbytes += 3 * d * Fs * wbytes_el + (4 * (2 * Fs + d) if cfg.w_dtype == 2 else 0)
        act_bytes += cfg.n_tokens * (d * xbytes * 2 + Fs * xbytes * 2)
    return flops, wbytes, act_bytes


def cpu_baseline(cfg, dev, sample_tokens):
    """Time the CPU oracle's layer forward on the first `sample_tokens` tokens
    of the workload, as their own batch (same shapes per token)."""
    import numpy as np
    import torch

    import oracle

    def host(t):
        if t is None:
            return None
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    S = min(sample_tokens, cfg.n_tokens)
    scfg = cfg.with_(n_tokens=S)
    h = {k: host(v) for k, v in dev.items() if k != "x"}
    hx = host(dev["x"][:S])
    shared = None
    if cfg.shared_d_ff:
        shared = oracle.ExpertSource({k[7:]: v for k, v in h.items() if k.startswith("shared_")})
    oracle.lib()
    t0 = time.perf_counter()
    oracle.layer_forward(scfg, hx, cfg.x_dtype, h["w_gate"], oracle.ExpertSource(h), shared,
                         h.get("logit_bias"), h.get("select_bias"), h.get("w_noise"))
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return {"value": S / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "oracle layer forward (fp32 routing, fp64 FFN/combine) on the first %d "
                      "tokens of the workload as one batch; %.1f s" % (S, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_mixture_experts_47_amd as moe
    import workloads as W

    cfg = W.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    dev = W.make_inputs(cfg, "cuda")
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    layer = moe.MoELayer(moe.spec_from_config(cfg), dev, x_dtype=xdt)
    x = dev["x"]
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    counts = layer.counts_kept.cpu().numpy()
    touched = int((counts > 0).sum())

    names = ["router", "dispatch", "grouped_ffn", "combine", "stats"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(stream)
        layer.route(x)
        e[1].record(stream)
        layer.dispatch(x)
        e[2].record(stream)
        layer.experts(x)
        e[3].record(stream)
        layer.combine()
        e[4].record(stream)
        layer.stats()
        e[5].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per = {n: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}
    ms_step = elapsed * 1e3 / args.steps
    flops, wbytes, act_bytes = ffn_work(cfg, counts, touched)
    ffn_ms = per["grouped_ffn"]
    tflops = flops / (ffn_ms * 1e-3) / 1e12
    gbs = (wbytes + act_bytes) / (ffn_ms * 1e-3) / 1e9
    if cfg.w_dtype == 2 or args.workload in ("c3", "c4"):
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None}
    roof["kernel"] = "moe_grouped_ffn (tile table + GEMM1 gate/up+act + GEMM2 down)"
    roof["per_launch"] = {"flops": flops, "weight_bytes": wbytes, "activation_bytes": act_bytes,
                          "avg_ms": round(ffn_ms, 4)}

    out = {
        "metric": METRIC,
        "value": round(cfg.n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "fp8e4m3-w/bf16-a"}[cfg.w_dtype],
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_tokens": cfg.n_tokens, "d_model": cfg.d_model,
                   "n_experts": cfg.n_experts, "d_ff": cfg.d_ff, "top_k": cfg.top_k,
                   "act": ["relu", "gelu", "swiglu"][cfg.act],
                   "shared_d_ff": cfg.shared_d_ff, "capacity": cfg.capacity,
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "per_call_ms": {k: round(v, 4) for k, v in per.items()},
        "grouped_ffn_tflops": round(tflops, 1),
        "layer_hbm_gbs_weights": round(wbytes / (ms_step * 1e-3) / 1e9, 1),
        "touched_experts": touched,
        "kept_assignments": int(counts.sum()),
    }
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        S = args.cpu_sample or {"c1": 256, "c2": 128, "c3": 16, "c4": 2048, "c5": 16}[args.workload]
        out["cpu_baseline"] = cpu_baseline(cfg, dev, S)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
