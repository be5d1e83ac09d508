"""Helpers for GPU-vs-oracle parity tests (no test functions here)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

# Output tolerances: max |y - y_ref| / RMS(y_ref).
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2
TOL_F32 = 1e-5
# scores, losses and statistics: relative
TOL_REL = 1e-5
# id comparison skips tokens whose k-th / (k+1)-th key margin is below this
MARGIN = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def out_tol(cfg):
    if cfg.w_dtype == W.FP8_E4M3:
        return TOL_FP8
    if cfg.x_dtype == W.F32:
        return TOL_F32
    return TOL_BF16


def host_view(t):
    """torch tensor -> numpy in the oracle's storage form."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def host_inputs(inp):
    return {k: host_view(v) for k, v in inp.items()}


def to_device(inp, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(y)))
    return float(np.max(np.abs(y - ref)) / rms)


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


class DeviceExperts(oracle.ExpertSource):
    """Fetch one expert's weights from device tensors on demand."""

    def __init__(self, dev_inputs, prefix=""):
        self.d = dev_inputs
        self.prefix = prefix
        self.cache = {}

    def get(self, e):
        # only the latest expert stays on the host: the oracle walks experts
        # one at a time, and a full-size layer's weights run to 22 GB
        if e not in self.cache:
            out = {}
            for k in ("w1", "w3", "w2", "b1", "b2", "s1", "s3", "s2"):
                v = self.d.get(self.prefix + k)
                out[k] = None if v is None else host_view(v[e])
            self.cache = {e: out}
        return self.cache[e]


def experts_of(host, prefix=""):
    return oracle.ExpertSource({k[len(prefix):]: v for k, v in host.items()
                                if k.startswith(prefix) and v is not None})


def margins(keys, k):
    """k-th minus (k+1)-th largest key per token (inf when E == k)."""
    s = -np.sort(-keys.astype(np.float64), axis=1)
    if s.shape[1] <= k:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def oracle_keys(route, select_bias):
    s = route["s"]
    return s + select_bias[None, :] if select_bias is not None else s


def tile_cover_sample(row_of, offsets, block=128, max_tokens=None):
    """Tokens whose packed rows touch every `block`-row slice of every
    expert's rows (slices start at the expert's first row, so every tile of
    any row tiling in multiples of `block` -- full tiles, the ragged last
    tile, a separate tail launch -- holds a sampled row) and every expert's
    last row. Greedy set cover: repeatedly take the token that covers the most
    targets not yet covered (ties to the lower token). row_of [N][slots]
    (-1 = not kept), offsets [E+1] from the oracle's dispatch. Returns
    (sorted token array, coverage dict)."""
    row_of = np.asarray(row_of)
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    M = np.diff(off)
    nblk = (M + block - 1) // block
    blk_base = np.concatenate([[0], np.cumsum(nblk)])
    n_targets = int(blk_base[-1]) + E
    N, S = row_of.shape
    rows = row_of.astype(np.int64)
    kept = rows >= 0
    e_of = np.clip(np.searchsorted(off, np.maximum(rows, 0), side="right") - 1, 0, E - 1)
    t_blk = np.where(kept, blk_base[e_of] + (rows - off[e_of]) // block, -1)
    t_last = np.where(kept & (rows == off[e_of + 1] - 1), blk_base[-1] + e_of, -1)
    targets = np.concatenate([t_blk, t_last], axis=1)  # [N][2*slots], -1 = none
    covered = np.zeros(n_targets + 1, bool)
    covered[-1] = True  # the -1 slot
    exists = np.zeros(n_targets, bool)
    exists[targets[targets >= 0]] = True
    covered[:-1] = ~exists
    chosen = []
    while not covered[:-1].all():
        gain = np.zeros(N, np.int64)
        for c in range(targets.shape[1]):
            gain += ~covered[targets[:, c]]
        t = int(np.argmax(gain))
        if gain[t] == 0:
            break
        chosen.append(t)
        covered[targets[t]] = True
        if max_tokens is not None and len(chosen) >= max_tokens:
            break
    cov = dict(tokens=len(chosen), blocks=int(covered[:int(blk_base[-1])].sum()),
               blocks_total=int(blk_base[-1]), last_rows=int(covered[int(blk_base[-1]):-1].sum()),
               experts_with_rows=int((M > 0).sum()))
    return np.array(sorted(chosen), np.int64), cov
