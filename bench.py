"""Benchmark: one MoE FFN layer forward per step on one MI355X, through libmoe.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c1|c3|c4|c5|c6|c7]
                [--backward]

A step is one pass of the whole layer: router GEMM + fp32 softmax + top-k,
dispatch (capacity, packing, row gather), the grouped expert FFN (+ shared
expert), the gate-weighted combine, and the balance statistics. Inputs are
synthetic (seeded, drawn on the GPU) and resident in HBM before timing.
Prints one JSON line. The default workload is the Mixtral-shaped prefill
(4096 tokens, d_model 4096, 8 experts of d_ff 14336 SwiGLU, top-2, bf16).

decode: with the default workload, a sub-record for the decode-shaped layer
(64 tokens against the DeepSeek-shaped layer, fp8 e4m3 expert weights):
whole-layer and grouped-FFN bandwidth on the touched experts' weights against
the HBM peak. per_call_gbs: algorithmic bytes and achieved GB/s (fraction of
the HBM peak) of the router, dispatch and combine calls, and beside them
x_read_reference: torch.sum over x timed the same way (warm and cold), the
rate a plain read of the router's main input reaches at this size.

roofline: the grouped expert FFN (moe_grouped_ffn: tile table + GEMM 1
gate/up with fused SwiGLU + GEMM 2 down) is the dominant kernel group; its
duration is measured with HIP events on the launch stream inside the timed
region. graph_replay: the same step replayed as one HIP graph (reported
beside the eager figure, which stays the metric). cpu_baseline: the CPU
oracle (fp64 FFNs) timed on a bounded sample of
the same workload on this host's cores (for the tiny Switch layer also on one
pinned core, in a child process). clocks: GFX and memory clocks and socket
power read with amd-smi while the same step runs back to back, after the
timed region.

--backward: a step is one training pass of the layer instead: the training
forward (which keeps the experts' pre-activations) and the backward pass of
L = <dy, y> + 0.01 Switch aux + 0.001 z-loss (combine backward, grouped FFN
backward, router backward). The dominant kernel group is the grouped FFN
backward (four bf16 MFMA GEMMs: data and weight gradients of both expert
GEMMs, 4 d d_ff FLOPs per weight matrix per kept assignment).
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
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector (published, with packed fp32 FMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5", "c6", "c7"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="with the default Mixtral workload: skip the decode-shaped sub-record")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens in the oracle's timed sample (0: choose by workload)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps timed one by one after writing a 512 MiB buffer "
                         "(evicts the 256 MB Infinity Cache); reported beside the warm run")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step (forward + backward) instead of the forward")
    ap.add_argument("--dw-bf16", action="store_true",
                    help="with --backward: expert weight gradients in bf16 instead of fp32")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step after the timed region")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the amd-smi clock and power sample after the timed region")
    ap.add_argument("--oracle-single-core", action="store_true",
                    help=argparse.SUPPRESS)  # child process: time the oracle on one core
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB read + 1 GiB write streaming kernel (torch.neg) "
                         "to calibrate the HBM byte counters")
    return ap.parse_args()


def ffn_work(cfg, counts_kept, touched, fused_combine=False):
    """Algorithmic work of one routed moe_grouped_ffn launch (the dominant
    kernel pair): FLOPs = 2 d F per weight matrix per kept assignment (3
    matrices for SwiGLU, 2 otherwise); weight bytes = every touched expert's
    weights once (+ fp32 per-channel scales for fp8); activation bytes = the
    packed rows read (bf16) and expert outputs written (fp32), h written and
    read once (bf16, or a bf16 pair with h_fp32). With the top-1 combine in
    GEMM 2's epilogue the outputs go to all N token rows instead (dropped
    tokens' rows zeroed)."""
    d, F = cfg.d_model, cfg.d_ff
    nmat = 3 if cfg.act == 2 else 2
    R = int(sum(counts_kept))
    flops = 2.0 * d * F * nmat * R
    wbytes_el = {0: 4, 1: 2, 2: 1}[cfg.w_dtype]
    xbytes = 4 if cfg.x_dtype == 0 else 2
    hbytes = 4 if (cfg.x_dtype == 0 or cfg.h_fp32) else 2
    wbytes = touched * nmat * d * F * wbytes_el
    if cfg.w_dtype == 2:
        wbytes += touched * 4 * ((nmat - 1) * F + d)
    out_rows = cfg.n_tokens if fused_combine else R
    act_bytes = R * d * xbytes + out_rows * d * 4 + R * F * hbytes * 2
    return flops, wbytes, act_bytes


def layer_weight_bytes(cfg, touched):
    """Weight bytes one whole layer forward must read: router weights, the
    touched routed experts, and the shared expert."""
    d, F = cfg.d_model, cfg.d_ff
    nmat = 3 if cfg.act == 2 else 2
    wb = {0: 4, 1: 2, 2: 1}[cfg.w_dtype]
    total = cfg.n_experts * d * 4 * (2 if cfg.noisy else 1)
    total += touched * nmat * d * F * wb + (touched * 4 * ((nmat - 1) * F + d) if wb == 1 else 0)
    if cfg.shared_d_ff:
        Fs = cfg.shared_d_ff
        total += 3 * d * Fs * wb + (4 * (2 * Fs + d) if wb == 1 else 0)
    return total


KERNEL_SOURCES = ["sparse_mixture_experts_47_amd/csrc/gemm_bf16.h",
                  "sparse_mixture_experts_47_amd/csrc/grouped_ffn.hip",
                  "sparse_mixture_experts_47_amd/csrc/moe_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_ffn_traffic.json")


def kernel_sources_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per grouped-FFN launch from the committed PMC record
    (FETCH_SIZE + WRITE_SIZE of its kernels, each scaled by the same
    counter's reading for a 1 GiB device copy), or None when there is no
    record for this workload or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sources_sha256") != kernel_sources_hash():
        return None
    return rec.get("traffic_bytes")


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
                      "tokens of the workload as one batch; %.1f s; CPU: %s" % (S, dt, cpu_model())}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_single_core_child(args):
    """Child-process entry (no GPU use): pin this process to one core, draw the
    workload's inputs by the same recipe with the CPU generator, and time the
    oracle's layer forward on them; prints one JSON object."""
    import workloads as W
    core = sorted(os.sched_getaffinity(0))[0]
    os.sched_setaffinity(0, {core})
    cfg = W.CONFIGS[args.workload]
    host = W.make_inputs(cfg, "cpu")
    S = args.cpu_sample or cfg.n_tokens
    runs, t0 = [], time.perf_counter()
    while len(runs) < 3 or (time.perf_counter() - t0 < 2.0 and len(runs) < 200):
        runs.append(cpu_baseline(cfg, host, S))
    vals = sorted(r["value"] for r in runs)
    r = runs[0]
    r["value"] = vals[len(vals) // 2]
    r["cores"] = 1
    r["sample"] = ("oracle layer forward (fp32 routing, fp64 FFN/combine) on the first %d "
                   "tokens of the workload as one batch, median of %d runs; one pinned core; "
                   "inputs drawn by the same recipe with the CPU generator; CPU: %s"
                   % (S, len(runs), cpu_model()))
    print(json.dumps(r), flush=True)


def cpu_baseline_single_core(workload, sample_tokens):
    """The oracle on one core: a child process with every thread pool at one
    thread (OpenMP, BLAS) and its affinity pinned to one core."""
    import subprocess
    env = dict(os.environ)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        env[k] = "1"
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", workload,
           "--oracle-single-core", "--cpu-sample", str(sample_tokens)]
    try:
        r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            return {"error": "child exited with %d: %s" % (r.returncode, r.stderr[-300:])}
        return json.loads(lines[-1])
    except (OSError, subprocess.SubprocessError, ValueError) as e:
        return {"error": repr(e)}


def sample_clocks(run_step, cap_s=20.0):
    """GFX and memory clocks and socket power while `run_step` (one step of
    the workload) runs back to back: `amd-smi metric -c -p` is read from a
    side thread while the main thread keeps the GPU busy. Returns the
    per-domain clocks in MHz, or an error string if amd-smi is unavailable."""
    import shutil
    import subprocess
    import threading

    import torch

    exe = shutil.which("amd-smi")
    if exe is None:
        return {"error": "amd-smi not found"}
    res = {}

    def probe():
        # let the clock settle under the load first; the second of two reads
        # is the one reported (the first can return the idle values of the
        # firmware's previous metrics update)
        time.sleep(1.0)
        try:
            for _ in range(2):
                r = subprocess.run([exe, "metric", "-c", "-p"], capture_output=True, text=True,
                                   timeout=60)
                res["text"], res["rc"] = r.stdout, r.returncode
        except (OSError, subprocess.SubprocessError) as e:
            res["error"] = repr(e)

    th = threading.Thread(target=probe)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while th.is_alive() and time.perf_counter() - t0 < cap_s:
        for _ in range(4):
            run_step()
        torch.cuda.synchronize()
        n += 4
    th.join()
    if "text" not in res:
        return {"error": res.get("error", "amd-smi did not finish")}
    out = parse_amd_smi_clocks(res["text"])
    if "error" in out:
        out["error"] += " (rc %s)" % res.get("rc")
        return out
    out.update(steps_during_sample=n,
               source="amd-smi metric -c -p, second of two reads taken while the step ran "
                      "back to back (after 1 s of it) following the timed region")
    return out


def parse_amd_smi_clocks(text):
    """Clocks from amd-smi's text report: each domain is a header line
    ("GFX_0:", "MEM_0:", ...) followed by its "CLK: <n> MHz" line; the socket
    power is a "SOCKET_POWER: <w> W" line."""
    clocks, power, header = {}, None, None
    for line in text.splitlines():
        t = line.strip()
        if t.endswith(":") and " " not in t:
            header = t[:-1]
        elif t.startswith("CLK:") and header and header not in clocks:
            v = t[4:].split()
            if v and v[0].isdigit():
                clocks[header] = int(v[0])
        elif t.startswith("SOCKET_POWER:"):
            v = t.split(":", 1)[1].split()
            if v and v[0].replace(".", "", 1).isdigit():
                power = float(v[0])
    gfx = [v for k, v in clocks.items() if k.upper().startswith("GFX")]
    mem = [v for k, v in clocks.items() if k.upper().startswith("MEM")]
    if not gfx:
        return {"error": "no GFX clock in amd-smi output"}
    return {"sclk_mhz_min": min(gfx), "sclk_mhz_max": max(gfx),
            "mclk_mhz": max(mem) if mem else None, "socket_power_w": power,
            "clocks_mhz": clocks}


def cpu_baseline_backward(cfg, dev, sample_tokens, alpha, beta):
    """Time the CPU oracle's layer forward + backward on the first
    `sample_tokens` tokens of the workload as their own batch."""
    import numpy as np
    import torch

    import oracle
    from oracle import backward as OB

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
    experts = oracle.ExpertSource(h)
    dy = np.random.default_rng(0).standard_normal((S, cfg.d_model))
    oracle.lib()
    t0 = time.perf_counter()
    fwd = oracle.layer_forward(scfg, hx, cfg.x_dtype, h["w_gate"], experts, None,
                               h.get("logit_bias"), h.get("select_bias"), h.get("w_noise"))
    OB.layer_backward(scfg, hx, cfg.x_dtype, h["w_gate"], experts, fwd, dy, alpha, beta,
                      logit_bias=h.get("logit_bias"))
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return {"value": S / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "oracle layer forward + backward (fp32 routing, fp64 FFNs and gradients) "
                      "on the first %d tokens of the workload as one batch; %.1f s; CPU: %s"
                      % (S, dt, cpu_model())}


def bench_backward(args):
    import numpy as np
    import torch

    import sparse_mixture_experts_47_amd as moe
    import workloads as W

    alpha, beta = 0.01, 0.001
    cfg = W.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    dev = W.make_inputs(cfg, "cuda")
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    spec = moe.spec_from_config(cfg)
    spec.h_fp32 = False  # training keeps h in bf16
    layer = moe.MoELayer(spec, dev, x_dtype=xdt, train=True)
    x = dev["x"]
    g = torch.Generator(device="cuda").manual_seed(1234)
    dy = torch.randn((cfg.n_tokens, cfg.d_model), generator=g, device="cuda")
    stream = torch.cuda.current_stream()

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        layer.forward(x, stats=False)
        if e is not None:
            e[1].record(stream)
        b = layer._bwd
        sh = layer.shared is not None
        gates, cand, expert_of, routed, k, renorm = moe._routing_for_backward(layer)
        moe.moe_combine_backward(dy, layer.y_rows, layer.row_of, gates, b[0]["d_rows"],
                                 b[0]["dgates"], d_shared=b[0]["d_shared"] if sh else None)
        if e is not None:
            e[2].record(stream)
        rows, index = layer._packed_rows(x)
        moe.moe_grouped_ffn_backward(layer.ffn, rows, layer.offsets, layer.preact, layer.h,
                                     b[0]["d_rows"], b[0]["dx_rows"], b[0]["dw1"], b[0]["dw3"],
                                     b[0]["dw2"], row_index=index, max_rows=layer.R, ws=b[1])
        if sh:
            moe.moe_grouped_ffn_backward(layer.shared, x, layer.sh_offsets, layer.preact_sh,
                                         layer.h_sh, b[0]["d_shared"], b[0]["dx_shared"],
                                         b[0]["shared_dw1"], b[0]["shared_dw3"],
                                         b[0]["shared_dw2"], max_rows=cfg.n_tokens, ws=b[1])
        if e is not None:
            e[3].record(stream)
        moe.moe_router_backward(x, dev["w_gate"], layer.logits, cand, expert_of,
                                layer.row_of, b[0]["dgates"], routed,
                                b[0]["dlogits"], b[0]["dw_gate"], b[0]["dx"],
                                top_k=k, renormalize=renorm, alpha=alpha,
                                beta=beta, dx_rows=b[0]["dx_rows"],
                                dx_shared=b[0]["dx_shared"] if sh else None,
                                dlogit_bias=b[0]["dlogit_bias"], w_noise=dev.get("w_noise"),
                                noise_seed=cfg.noise_seed, noise_v=layer.noise_v,
                                dw_noise=b[0]["dw_noise"], ws=b[2])
        if e is not None:
            e[4].record(stream)

    dw_dtype = torch.bfloat16 if args.dw_bf16 else torch.float32
    # one full step allocates the backward buffers (the forward first: the
    # backward reads its routing and saved activations)
    layer.forward(x, stats=False)
    moe.layer_backward(layer, x, dy, alpha, beta, dw_dtype)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    names = ["forward_train", "combine_backward", "grouped_ffn_backward", "router_backward"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(ev[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    samples = {n: [ev[s_][i].elapsed_time(ev[s_][i + 1]) for s_ in range(args.steps)]
               for i, n in enumerate(names)}
    counts = layer.counts_kept.cpu().numpy()
    touched = int((counts > 0).sum())
    R = int(counts.sum())
    d, F = cfg.d_model, cfg.d_ff
    nmat = 3 if cfg.act == 2 else 2  # weight matrices per expert
    flops = 4.0 * nmat * d * (F * R + cfg.shared_d_ff * cfg.n_tokens)
    ms_bwd_ffn = float(np.median(samples["grouped_ffn_backward"]))
    tflops = flops / (ms_bwd_ffn * 1e-3) / 1e12
    # algorithmic bytes of the expert backward: the data gradients read every
    # touched weight once (bf16); every expert's weight gradients are written
    # once; activations at their minimum (dO read twice, the saved pre-
    # activations and h once, dpre written once and read twice, x rows read
    # once, dX rows written once in fp32)
    gb = 2 if args.dw_bf16 else 4
    P = (2 if nmat == 3 else 1) * F
    wbytes = nmat * d * F * 2 * touched + nmat * d * F * gb * cfg.n_experts
    abytes = R * (2 * d * 2 + P * 2 + F * 2 + 3 * P * 2 + d * 2 + d * 4)
    if cfg.shared_d_ff:
        Fs, Ps = cfg.shared_d_ff, (2 if nmat == 3 else 1) * cfg.shared_d_ff
        wbytes += nmat * d * Fs * (2 + gb)
        abytes += cfg.n_tokens * (2 * d * 2 + Ps * 2 + Fs * 2 + 3 * Ps * 2 + d * 2 + d * 4)
    gbs = (wbytes + abytes) / (ms_bwd_ffn * 1e-3) / 1e9
    if args.workload in ("c3", "c4"):  # weight-bound shapes, as for the forward
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    roof.update(traffic=None,
                kernel="moe_grouped_ffn_backward (data and weight gradients of both expert "
                       "GEMMs, activation backward fused; routed + shared experts)",
                per_launch={"flops": flops, "weight_bytes": wbytes, "activation_bytes": abytes,
                            "avg_ms": round(ms_bwd_ffn, 4), "kept_assignments": R,
                            "touched_experts": touched})
    ms_step = elapsed * 1e3 / args.steps
    out = {
        "metric": "MoE-layer training-step tokens/sec (forward + backward) + grouped-GEMM "
                  "backward % MFMA peak, 1 MI355X",
        "value": round(cfg.n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + "_training_step", "n_tokens": cfg.n_tokens,
                   "d_model": d, "n_experts": cfg.n_experts, "d_ff": F, "top_k": cfg.top_k,
                   "act": ["relu", "gelu", "swiglu"][cfg.act], "loss": "<dy,y> + 0.01 aux + "
                   "0.001 z", "weight_grad_dtype": "bf16" if args.dw_bf16 else "f32",
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "grouped_ffn_backward_tflops": round(tflops, 1),
        "grouped_ffn_backward_gbs": round(gbs, 1),
        "per_call_ms_median": {k: round(float(np.median(v)), 4) for k, v in samples.items()},
        "per_call_ms_min": {k: round(float(np.min(v)), 4) for k, v in samples.items()},
    }
    if not args.no_clocks:
        out["clocks"] = sample_clocks(step)
    if not args.no_cpu_baseline:
        S = args.cpu_sample or 256
        out["cpu_baseline"] = cpu_baseline_backward(cfg, dev, S, alpha, beta)
    print(json.dumps(out), flush=True)


def call_bytes(cfg, layer, counts):
    """Algorithmic bytes of the memory-bound calls of one forward, in the
    formats this library moves: router (x and router weights read once,
    candidates, gates and logits written), dispatch (candidates and gates
    read, per-assignment rows and counts written), combine (each kept fp32
    expert row and the shared expert's row read once, the output written)."""
    N, d, E = cfg.n_tokens, cfg.d_model, cfg.n_experts
    k, C = layer.gates.shape[1], layer.C
    xb = 4 if cfg.x_dtype == 0 else 2
    R = int(sum(counts))
    router = N * d * xb + E * d * 4 * (2 if cfg.noisy else 1) + N * E * 4 + N * (2 * C + k) * 4
    if layer.scores is not None:
        router += N * E * 4
    if layer.ec:
        dispatch = N * E * 4 + E * 4 + layer.R * 4 + N * E * 8
    else:
        dispatch = N * C * 8 + N * k * 4 * 5 + E * 12
    slots = layer.row_of.shape[1]
    combine = R * d * 4 + N * slots * 8 + N * d * layer.y.element_size()
    if layer.shared is not None:
        combine += N * d * 4
    return {"router": router, "dispatch": dispatch, "combine": combine}


def time_forward(cfg, steps, warmup, cold_steps):
    """Build the layer for `cfg` on resident synthetic inputs, run `warmup`
    forwards, then time `steps` back-to-back forwards (wall clock between
    two synchronisations; HIP events on the launch stream around the grouped
    FFN), then as many more with events around every call for the per-call
    breakdown (and `cold_steps` more, each after a 512 MiB write that evicts
    the 256 MB Infinity Cache)."""
    import numpy as np
    import torch

    import sparse_mixture_experts_47_amd as moe
    import workloads as W

    dev = W.make_inputs(cfg, "cuda")
    xdt = torch.float32 if cfg.x_dtype == W.F32 else torch.bfloat16
    layer = moe.MoELayer(moe.spec_from_config(cfg), dev, x_dtype=xdt)
    x = dev["x"]
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    counts = layer.counts_kept.cpu().numpy()
    names = ["router", "dispatch", "grouped_ffn", "combine", "stats"]

    def one_step(e):
        e[0].record(stream)
        layer.start_shared(x)
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

    def timed_step(e):
        # the timed steps carry events around the grouped FFN only: an event
        # record between two calls costs the stream 1.5-5 us, which every
        # per-call event would add to the step
        layer.start_shared(x)
        layer.route(x)
        layer.dispatch(x)
        e[0].record(stream)
        layer.experts(x)
        e[1].record(stream)
        layer.combine()
        layer.stats()

    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(steps):
        timed_step(fev[st])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-call breakdown: as many steps again, with events around every call
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(steps)]
    for st in range(steps):
        one_step(ev[st])
    torch.cuda.synchronize()
    samples = {n: [ev[st][i].elapsed_time(ev[st][i + 1]) for st in range(steps)]
               for i, n in enumerate(names)}
    samples["grouped_ffn"] = [fev[st][0].elapsed_time(fev[st][1]) for st in range(steps)]
    layer_ev = [ev[st][0].elapsed_time(ev[st][len(names)]) for st in range(steps)]
    # yardstick for the router: torch's own reduction over x (a plain read of
    # the router's main input), timed with the same events, warm and cold
    xev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for st in range(steps):
        xev[st][0].record(stream)
        torch.sum(x, dtype=torch.float32)
        xev[st][1].record(stream)
    torch.cuda.synchronize()
    x_read = {"warm": [xev[st][0].elapsed_time(xev[st][1]) for st in range(steps)], "cold": []}
    cold = None
    if cold_steps > 0:
        evict = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(cold_steps)]
        for st in range(cold_steps):
            evict.fill_(float(st))
            one_step(cev[st])
            torch.cuda.synchronize()
        csamp = {n: [cev[st][i].elapsed_time(cev[st][i + 1]) for st in range(cold_steps)]
                 for i, n in enumerate(names)}
        clayer = [cev[st][0].elapsed_time(cev[st][len(names)]) for st in range(cold_steps)]
        xc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(cold_steps)]
        for st in range(cold_steps):
            evict.fill_(float(st))
            xc[st][0].record(stream)
            torch.sum(x, dtype=torch.float32)
            xc[st][1].record(stream)
            torch.cuda.synchronize()
        x_read["cold"] = [xc[st][0].elapsed_time(xc[st][1]) for st in range(cold_steps)]
        cold = {"steps": cold_steps, "evict_bytes": 4 << 27,
                "ms_per_step_median": round(float(np.median(clayer)), 4),
                "ms_per_step_min": round(float(np.min(clayer)), 4),
                "per_call_ms_median": {kk: round(float(np.median(v)), 4)
                                       for kk, v in csamp.items()}}
        del evict
    return dict(dev=dev, layer=layer, x=x, counts=counts, samples=samples, layer_ev=layer_ev,
                ms_step=elapsed * 1e3 / steps, cold=cold, x_read=x_read)


def per_call_gbs(cfg, layer, counts, samples, x_read=None):
    """Achieved algorithmic GB/s and fraction of HBM peak of the router,
    dispatch and combine calls (median call time); with x_read, the same
    figures for torch.sum over x timed alike (warm, and cold after the
    cache-evicting write), the rate a plain read of the router's main input
    reaches at this size."""
    import numpy as np
    out = {}
    if x_read:
        xb = cfg.n_tokens * cfg.d_model * (4 if cfg.x_dtype == 0 else 2)
        ref = {"bytes": int(xb), "what": "torch.sum over x, HIP events around the call"}
        for kk, v in x_read.items():
            if v:
                ms = float(np.median(v))
                ref[kk] = {"ms_median": round(ms, 4), "gbs": round(xb / (ms * 1e-3) / 1e9, 1),
                           "frac_hbm": round(xb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        out["x_read_reference"] = ref
    for name, nbytes in call_bytes(cfg, layer, counts).items():
        ms = float(np.median(samples[name]))
        if name == "combine" and layer.fused_combine:
            out[name] = {"fused_into": "grouped_ffn", "ms_median": round(ms, 4)}
            continue
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"bytes": int(nbytes), "ms_median": round(ms, 4), "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def decode_record(steps, warmup):
    """The decode-shaped layer (64 tokens against the DeepSeek-shaped layer,
    fp8 e4m3 expert weights): whole-layer and grouped-FFN bandwidth against
    the HBM peak, on the touched experts' weights."""
    import numpy as np
    import workloads as W
    cfg = W.CONFIGS["c5"]
    r = time_forward(cfg, steps, warmup, 0)
    layer, counts = r["layer"], r["counts"]
    touched = int((counts > 0).sum())
    flops, wbytes, act_bytes = ffn_work(cfg, counts, touched, layer.fused_combine)
    ffn_ms = float(np.median(r["samples"]["grouped_ffn"]))
    lw = layer_weight_bytes(cfg, touched)
    lay_ms = float(np.median(r["layer_ev"]))
    rec = {"workload": cfg.name, "n_tokens": cfg.n_tokens, "steps": steps,
           "ms_per_step": round(r["ms_step"], 4),
           "layer_ms_events_median": round(lay_ms, 4),
           "touched_experts": touched, "layer_weight_bytes": int(lw),
           "layer_weight_gbs": round(lw / (r["ms_step"] * 1e-3) / 1e9, 1),
           "layer_weight_frac_hbm": round(lw / (r["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "grouped_ffn_ms_median": round(ffn_ms, 4),
           "grouped_ffn_bytes": int(wbytes + act_bytes),
           "grouped_ffn_gbs": round((wbytes + act_bytes) / (ffn_ms * 1e-3) / 1e9, 1),
           "grouped_ffn_frac_hbm": round((wbytes + act_bytes) / (ffn_ms * 1e-3) / 1e9
                                         / PEAK_HBM_GBS, 4),
           "per_call_ms_median": {kk: round(float(np.median(v)), 4)
                                  for kk, v in r["samples"].items()},
           "per_call_gbs": per_call_gbs(cfg, layer, counts, r["samples"], r.get("x_read")),
           "tokens_per_s": round(cfg.n_tokens / (r["ms_step"] * 1e-3), 1)}
    del r
    return rec


def main():
    args = parse()
    if args.oracle_single_core:
        return oracle_single_core_child(args)
    if args.gpus != 1:
        print("bench.py measures one GPU: libmoe has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.backward:
        return bench_backward(args)
    import numpy as np
    import torch

    import sparse_mixture_experts_47_amd as moe
    import workloads as W

    cfg = W.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    r = time_forward(cfg, args.steps, args.warmup, args.cold_steps)
    dev, layer, x, counts = r["dev"], r["layer"], r["x"], r["counts"]
    touched = int((counts > 0).sum())
    samples, layer_ev, cold = r["samples"], r["layer_ev"], r["cold"]
    per = {n: float(np.mean(v)) for n, v in samples.items()}
    ms_step = r["ms_step"]
    flops, wbytes, act_bytes = ffn_work(cfg, counts, touched, layer.fused_combine)
    ffn_ms = per["grouped_ffn"]
    tflops = flops / (ffn_ms * 1e-3) / 1e12
    gbs = (wbytes + act_bytes) / (ffn_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload)
    if cfg.w_dtype == 2 or args.workload in ("c3", "c4"):
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    elif cfg.x_dtype == W.F32:
        # fp32 experts run on the vector ALU (fp32 FMA), not on MFMA
        roof = {"bound": "alu", "achieved": round(tflops, 3), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_TFLOPS, 6),
                "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic}
    roof["kernel"] = ("moe_grouped_ffn, routed experts (tile table + GEMM 1 gate/up with "
                      "fused activation + GEMM 2 down" +
                      (" with the top-1 combine in its epilogue)" if layer.fused_combine else ")"))
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
                   "shared_d_ff": cfg.shared_d_ff, "capacity": layer.spec.capacity,
                   "routing": "expert_choice" if cfg.expert_choice else "token_choice",
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "per_call_ms": {k: round(v, 4) for k, v in per.items()},
        "per_call_ms_median": {k: round(float(np.median(v)), 4) for k, v in samples.items()},
        "per_call_ms_min": {k: round(float(np.min(v)), 4) for k, v in samples.items()},
        "layer_ms_events_median": round(float(np.median(layer_ev)), 4),
        "layer_ms_events_min": round(float(np.min(layer_ev)), 4),
        "cold_cache": cold,
        "grouped_ffn_tflops": round(tflops, 1),
        "layer_weight_gbs": round(layer_weight_bytes(cfg, touched) / (ms_step * 1e-3) / 1e9, 1),
        "layer_weight_frac_hbm": round(layer_weight_bytes(cfg, touched) / (ms_step * 1e-3) / 1e9
                                       / PEAK_HBM_GBS, 4),
        "touched_experts": touched,
        "kept_assignments": int(counts.sum()),
        "per_call_gbs": per_call_gbs(cfg, layer, counts, samples, r.get("x_read")),
        "library": os.path.relpath(moe.LIB_PATH, ROOT),
    }
    if args.copy_calibration:
        # a plain streaming kernel of known size for HBM counter calibration:
        # torch.neg over 2^28 fp32 values reads 1 GiB and writes 1 GiB
        n = 1 << 28
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 4 * n
        del a, b
    # the same step as one HIP graph replay (every kernel of the layer in one
    # launch): reported beside the eager figure, which stays the metric
    try:
        if args.no_graph:
            raise RuntimeError("skipped (--no-graph)")
        g = layer.capture(x)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        out["graph_replay"] = {"ms_per_step": round(gms, 4),
                               "tokens_per_s": round(cfg.n_tokens / (gms * 1e-3), 1),
                               "steps": args.steps}
        del g
    except Exception as e:  # reported, never fatal to the measurement
        out["graph_replay"] = {"error": repr(e)[:300]}
    if not args.no_clocks:
        out["clocks"] = sample_clocks(lambda: layer.forward(x))

    if not args.no_cpu_baseline:
        S = args.cpu_sample or {"c1": 256, "c2": 1024, "c3": 64, "c4": 4096, "c5": 64,
                                  "c6": 1024, "c7": 64}[args.workload]
        out["cpu_baseline"] = cpu_baseline(cfg, dev, S)
        if args.workload == "c1":
            out["cpu_baseline"]["single_core"] = cpu_baseline_single_core("c1", S)
    if args.workload == "c2" and not args.no_decode:
        # the second target: the decode-shaped layer against the HBM peak
        del layer, dev, r
        torch.cuda.empty_cache()
        out["decode"] = decode_record(args.steps, args.warmup)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
