"""Python binding of libmoe: the sparse MoE FFN layer forward on MI355X.

Argument marshalling only. Each function takes torch tensors that already
live on the GPU, checks dtype, shape and contiguity, and passes raw device
pointers plus the current HIP stream to the C ABI in include/libmoe.h; every
step of the layer runs in libmoe's HIP kernels. torch supplies device memory
and streams, nothing else. There is no CPU fallback: if libmoe.so is not
built, importing the binding raises.

Calls (same names as the C ABI): moe_router_topk, moe_dispatch,
moe_grouped_ffn, moe_combine, moe_balance_stats; MoELayer strings them
together for one layer forward.
"""
from __future__ import annotations

import ctypes
import os
from fractions import Fraction
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, always (no environment override)
LIB_PATH = os.path.join(_HERE, "libmoe.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
RELU, GELU, SWIGLU = 0, 1, 2
DROPLESS, DROP, REROUTE_THEN_DROP = 0, 1, 2
_STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE",
           4: "MOE_EHIP"}


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status


class RouterParams(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_cand", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("logit_bias", ctypes.c_void_p), ("select_bias", ctypes.c_void_p),
                ("w_noise", ctypes.c_void_p), ("noise_seed", ctypes.c_uint64),
                ("scores_out", ctypes.c_void_p), ("noise_out", ctypes.c_void_p),
                ("w_planes", ctypes.c_void_p)]


class FFNWeights(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("act", ctypes.c_int32), ("w_dt", ctypes.c_int32),
                ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b1", ctypes.c_void_p), ("b2", ctypes.c_void_p), ("s1", ctypes.c_void_p),
                ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p), ("h_fp32", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe.so is not built at %s; run "
                          "`python __graft_entry__.py` (build())" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.moe_router_topk.argtypes = [ctypes.POINTER(RouterParams), P, i32, P, P, P, P, P, P, P, P,
                                  sz, P]
    L.moe_router_topk.restype = i32
    L.moe_router_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.moe_router_workspace_bytes.restype = sz
    L.moe_router_planes_bytes.argtypes = [i32, i32, i32]
    L.moe_router_planes_bytes.restype = sz
    L.moe_router_prepare.argtypes = [P, P, i32, i32, P, sz, P]
    L.moe_router_prepare.restype = i32
    L.moe_dispatch.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, i32, i32, P, P, P, P,
                               P, P, P, P, sz, P]
    L.moe_dispatch.restype = i32
    L.moe_dispatch_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, i32, i32, P, P,
                                       P, P, P, P, P, P]
    L.moe_dispatch_noalloc.restype = i32
    L.moe_dispatch_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_dispatch_workspace_bytes.restype = sz
    L.moe_capacity.argtypes = [i32, i32, i32, i32]
    L.moe_capacity.restype = i32
    L.moe_grouped_ffn.argtypes = [ctypes.POINTER(FFNWeights), P, i32, P, P, i32, P, i32, P, sz,
                                  P]
    L.moe_grouped_ffn.restype = i32
    L.moe_grouped_ffn_combine_top1.argtypes = [ctypes.POINTER(FFNWeights), P, i32, P, P, i32,
                                               i32, P, P, P, P, P, sz, P]
    L.moe_grouped_ffn_combine_top1.restype = i32
    L.moe_grouped_ffn_workspace_bytes.argtypes = [ctypes.POINTER(FFNWeights), i32, i32]
    L.moe_grouped_ffn_workspace_bytes.restype = sz
    L.moe_combine.argtypes = [i32, i32, i32, P, i32, P, P, P, i32, P, i32, P]
    L.moe_combine.restype = i32
    L.moe_expert_choice.argtypes = [i32, i32, i32, P, P, P, P, P, P, P]
    L.moe_expert_choice.restype = i32
    L.moe_grouped_ffn_train.argtypes = [ctypes.POINTER(FFNWeights), P, P, P, i32, P, i32, P, P,
                                        P, sz, P]
    L.moe_grouped_ffn_train.restype = i32
    L.moe_grouped_ffn_backward_workspace_bytes.argtypes = [ctypes.POINTER(FFNWeights), i32, i32]
    L.moe_grouped_ffn_backward_workspace_bytes.restype = sz
    L.moe_grouped_ffn_backward.argtypes = [ctypes.POINTER(FFNWeights), P, P, P, i32, P, P, P, P,
                                           P, P, P, i32, P, sz, P]
    L.moe_grouped_ffn_backward.restype = i32
    L.moe_combine_backward.argtypes = [i32, i32, i32, P, P, i32, P, P, P, P, P, P]
    L.moe_combine_backward.restype = i32
    L.moe_router_backward_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_router_backward_workspace_bytes.restype = sz
    L.moe_router_backward.argtypes = [ctypes.POINTER(RouterParams), P, i32, P, P, P, P, P, P, P,
                                      ctypes.c_float, ctypes.c_float, P, P, P, P, P, P, P, P, P,
                                      sz, P]
    L.moe_router_backward.restype = i32
    L.moe_balance_stats.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, ctypes.c_float, P]
    L.moe_balance_stats.restype = i32
    L.moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_version.argtypes = []
    L.moe_version.restype = ctypes.c_char_p
    return L


lib = _load()


def _check(status):
    if status != 0:
        raise MoEError(status, lib.moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libmoe needs contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError("unsupported dtype %s" % t.dtype)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libmoe tensors must live on the GPU")


def capacity(n_tokens: int, n_experts: int, capacity_factor) -> int:
    """moe_capacity: ceil(n_tokens / n_experts * capacity_factor). A float
    factor is passed as the decimal it prints as (1.1 -> 11/10); an int or a
    fractions.Fraction as itself."""
    f = Fraction(repr(capacity_factor)) if isinstance(capacity_factor, float) else \
        Fraction(capacity_factor)
    if f.numerator > 2**31 - 1 or f.denominator > 2**31 - 1:
        raise ValueError("capacity factor %r needs a fraction of 31-bit integers" %
                         (capacity_factor,))
    c = int(lib.moe_capacity(n_tokens, n_experts, f.numerator, f.denominator))
    if c < 0:
        raise MoEError(1, "moe_capacity(%d, %d, %s) out of range" % (n_tokens, n_experts, f))
    return c


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- calls
def moe_router_prepare(w_gate, w_noise=None, planes=None, stream=None):
    """The router weights as three exact bf16 planes for later router calls
    (w_planes=); returns the (new or given) uint8 device buffer."""
    E, d = w_gate.shape
    nb = lib.moe_router_planes_bytes(E, d, int(w_noise is not None))
    if planes is None:
        planes = workspace(nb, w_gate.device)
    _dev_check(w_gate, w_noise, planes)
    _check(lib.moe_router_prepare(_ptr(w_gate), _ptr(w_noise), E, d, _ptr(planes), planes.numel(),
                                  _stream(stream)))
    return planes


def moe_router_topk(x, w_gate, *, top_k, n_cand=None, renormalize=True, logit_bias=None,
                    select_bias=None, w_noise=None, noise_seed=0, logits_in=None, cand_ids,
                    cand_scores, gates, logits_out=None, score_sums=None, scores_out=None,
                    noise_out=None, w_planes=None, ws=None, stream=None):
    """Router GEMM + fp32 softmax + top-k. Outputs are written in place;
    scores_out [N][E] fp32 (optional) receives every softmax score; w_planes
    (from moe_router_prepare) skips the per-call weight split."""
    N, E = cand_ids.shape[0], (w_gate.shape[0] if logits_in is None else logits_in.shape[1])
    d = x.shape[1] if x is not None else 0
    n_cand = n_cand or top_k
    _dev_check(x, w_gate, logits_in, cand_ids, cand_scores, gates, logits_out, score_sums,
               scores_out, noise_out)
    p = RouterParams(N, d, E, top_k, n_cand, int(bool(renormalize)),
                     _ptr(logit_bias), _ptr(select_bias), _ptr(w_noise), int(noise_seed),
                     _ptr(scores_out), _ptr(noise_out), _ptr(w_planes))
    if ws is None:
        ws = workspace(lib.moe_router_workspace_bytes(N, d, E, int(w_noise is not None)),
                       cand_ids.device)
    _check(lib.moe_router_topk(ctypes.byref(p), _ptr(x), _dt(x) if x is not None else F32,
                               _ptr(w_gate), _ptr(logits_in), _ptr(cand_ids), _ptr(cand_scores),
                               _ptr(gates), _ptr(logits_out), _ptr(score_sums), _ptr(ws),
                               ws.numel(), _stream(stream)))


def moe_dispatch(cand_ids, cand_scores, gates, *, n_experts, top_k, policy=DROPLESS,
                 capacity=-1, x=None, counts_routed, counts_kept, offsets, row_of, expert_of,
                 perm_token, x_perm=None, ws=None, stream=None):
    N, C = cand_ids.shape
    _dev_check(cand_ids, cand_scores, gates, x, counts_routed, counts_kept, offsets, row_of,
               expert_of, perm_token, x_perm)
    if ws is None:
        ws = workspace(lib.moe_dispatch_workspace_bytes(N, n_experts, top_k), cand_ids.device)
    d = x.shape[1] if x is not None else 0
    _check(lib.moe_dispatch(N, n_experts, top_k, C, policy, capacity, _ptr(cand_ids),
                            _ptr(cand_scores), _ptr(gates), _ptr(x),
                            _dt(x) if x is not None else F32, d, _ptr(counts_routed),
                            _ptr(counts_kept), _ptr(offsets), _ptr(row_of), _ptr(expert_of),
                            _ptr(perm_token), _ptr(x_perm), _ptr(ws), ws.numel(),
                            _stream(stream)))


def moe_dispatch_noalloc(cand_ids, cand_scores, gates, *, n_experts, top_k, policy=DROPLESS,
                         capacity=-1, x=None, counts_routed, counts_kept, offsets, row_of,
                         expert_of, perm_token, x_perm=None, stream=None):
    """moe_dispatch with the library's fixed scratch instead of a workspace
    (no device allocation anywhere in the call)."""
    N, C = cand_ids.shape
    _dev_check(cand_ids, cand_scores, gates, x, counts_routed, counts_kept, offsets, row_of,
               expert_of, perm_token, x_perm)
    d = x.shape[1] if x is not None else 0
    _check(lib.moe_dispatch_noalloc(N, n_experts, top_k, C, policy, capacity, _ptr(cand_ids),
                                    _ptr(cand_scores), _ptr(gates), _ptr(x),
                                    _dt(x) if x is not None else F32, d, _ptr(counts_routed),
                                    _ptr(counts_kept), _ptr(offsets), _ptr(row_of),
                                    _ptr(expert_of), _ptr(perm_token), _ptr(x_perm),
                                    _stream(stream)))


def moe_expert_choice(scores, capacity, *, offsets, perm_token, row_of, gates, counts=None,
                      stream=None):
    """Expert-choice selection: every expert takes its min(capacity, N)
    top-scoring tokens, listed in token order."""
    N, E = scores.shape
    _dev_check(scores, offsets, perm_token, row_of, gates, counts)
    _check(lib.moe_expert_choice(N, E, int(capacity), _ptr(scores), _ptr(offsets),
                                 _ptr(perm_token), _ptr(row_of), _ptr(gates), _ptr(counts),
                                 _stream(stream)))


def ffn_weights(w1, w2, w3=None, act=SWIGLU, b1=None, b2=None, s1=None, s3=None, s2=None,
                h_fp32=False):
    E, F, d = w1.shape
    return FFNWeights(E, d, F, act, _dt(w1), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(b1), _ptr(b2),
                      _ptr(s1), _ptr(s3), _ptr(s2), int(bool(h_fp32))), \
        (w1, w2, w3, b1, b2, s1, s3, s2)


def moe_grouped_ffn(weights: FFNWeights, x_rows, offsets, y_rows, *, row_index=None,
                    max_rows=None, ws=None, stream=None):
    """Grouped expert FFN. row_index (e.g. perm_token) makes packed row r read
    x_rows[row_index[r]], so x_rows can be the unpermuted token rows."""
    _dev_check(x_rows, offsets, y_rows, row_index)
    max_rows = max_rows or (row_index.shape[0] if row_index is not None else x_rows.shape[0])
    if ws is None:
        ws = workspace(lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(weights), _dt(x_rows),
                                                           max_rows), x_rows.device)
    _check(lib.moe_grouped_ffn(ctypes.byref(weights), _ptr(x_rows), _dt(x_rows),
                               _ptr(row_index), _ptr(offsets), max_rows, _ptr(y_rows),
                               _dt(y_rows), _ptr(ws), ws.numel(), _stream(stream)))


def moe_grouped_ffn_combine_top1(weights: FFNWeights, x_rows, offsets, perm_token, row_of, gates,
                                 y, *, row_index=None, max_rows=None, ws=None, stream=None):
    """Grouped expert FFN with the top-1 gate-weighted combine in GEMM 2's
    epilogue: writes y [N][d] (fp32) in token order directly."""
    _dev_check(x_rows, offsets, perm_token, row_of, gates, y, row_index)
    N = row_of.shape[0]
    max_rows = max_rows or perm_token.shape[0]
    if ws is None:
        ws = workspace(lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(weights), _dt(x_rows),
                                                           max_rows), x_rows.device)
    _check(lib.moe_grouped_ffn_combine_top1(ctypes.byref(weights), _ptr(x_rows), _dt(x_rows),
                                            _ptr(row_index), _ptr(offsets), max_rows, N,
                                            _ptr(perm_token), _ptr(row_of), _ptr(gates), _ptr(y),
                                            _ptr(ws), ws.numel(), _stream(stream)))


def moe_combine(y_rows, row_of, gates, y, *, y_shared=None, stream=None):
    N, k = row_of.shape
    _dev_check(y_rows, row_of, gates, y, y_shared)
    _check(lib.moe_combine(N, y.shape[1], k, _ptr(y_rows), _dt(y_rows), _ptr(row_of),
                           _ptr(gates), _ptr(y_shared),
                           _dt(y_shared) if y_shared is not None else F32, _ptr(y), _dt(y),
                           _stream(stream)))


def moe_balance_stats(n_tokens, top_k, counts_routed, counts_kept, score_sums, f, P, scalars,
                      *, select_bias=None, bias_rate=0.0, stream=None):
    E = counts_routed.shape[0]
    _dev_check(counts_routed, counts_kept, score_sums, f, P, scalars, select_bias)
    _check(lib.moe_balance_stats(n_tokens, E, top_k, _ptr(counts_routed), _ptr(counts_kept),
                                 _ptr(score_sums), _ptr(f), _ptr(P), _ptr(scalars),
                                 _ptr(select_bias), float(bias_rate), _stream(stream)))


# ------------------------------------------------------------------ training
def moe_grouped_ffn_train(weights: FFNWeights, x_rows, offsets, y_rows, preact, h, *,
                          row_index=None, max_rows=None, ws=None, stream=None):
    """Grouped FFN forward that also saves the pre-activations [R][2 d_ff]
    and h [R][d_ff] (bf16) for the backward pass."""
    _dev_check(x_rows, offsets, y_rows, preact, h, row_index)
    max_rows = max_rows or (row_index.shape[0] if row_index is not None else x_rows.shape[0])
    if ws is None:
        ws = workspace(lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(weights), BF16,
                                                           max_rows), x_rows.device)
    _check(lib.moe_grouped_ffn_train(ctypes.byref(weights), _ptr(x_rows), _ptr(row_index),
                                     _ptr(offsets), max_rows, _ptr(y_rows), _dt(y_rows),
                                     _ptr(preact), _ptr(h), _ptr(ws), ws.numel(),
                                     _stream(stream)))


def moe_combine_backward(dy, y_rows, row_of, gates, d_rows, dgates, *, d_shared=None,
                         stream=None):
    N, k = row_of.shape
    _dev_check(dy, y_rows, row_of, gates, d_rows, dgates, d_shared)
    _check(lib.moe_combine_backward(N, dy.shape[1], k, _ptr(dy), _ptr(y_rows), _dt(y_rows),
                                    _ptr(row_of), _ptr(gates), _ptr(d_rows), _ptr(dgates),
                                    _ptr(d_shared), _stream(stream)))


def moe_grouped_ffn_backward(weights: FFNWeights, x_rows, offsets, preact, h, d_rows, dx_rows,
                             dw1, dw3, dw2, *, row_index=None, max_rows=None, ws=None,
                             stream=None):
    _dev_check(x_rows, offsets, preact, h, d_rows, dx_rows, dw1, dw3, dw2, row_index)
    max_rows = max_rows or d_rows.shape[0]
    if ws is None:
        ws = workspace(lib.moe_grouped_ffn_backward_workspace_bytes(
            ctypes.byref(weights), max_rows, int(row_index is not None)), x_rows.device)
    _check(lib.moe_grouped_ffn_backward(ctypes.byref(weights), _ptr(x_rows), _ptr(row_index),
                                        _ptr(offsets), max_rows, _ptr(preact), _ptr(h),
                                        _ptr(d_rows), _ptr(dx_rows), _ptr(dw1), _ptr(dw3),
                                        _ptr(dw2), _dt(dw1), _ptr(ws), ws.numel(),
                                        _stream(stream)))


def moe_router_backward(x, w_gate, logits, cand_ids, expert_of, row_of, dgates, counts_routed,
                        dlogits, dw_gate, dx, *, top_k, renormalize, alpha=0.0, beta=0.0,
                        dx_rows=None, dx_shared=None, dlogit_bias=None, w_noise=None,
                        noise_seed=0, noise_v=None, dw_noise=None, ws=None, stream=None):
    N, E = logits.shape
    d = x.shape[1]
    _dev_check(x, w_gate, logits, cand_ids, expert_of, row_of, dgates, counts_routed, dlogits,
               dw_gate, dx, dx_rows, dx_shared, dlogit_bias, w_noise, noise_v, dw_noise)
    p = RouterParams(N, d, E, top_k, cand_ids.shape[1], int(bool(renormalize)), None, None,
                     _ptr(w_noise), int(noise_seed), None, None)
    if ws is None:
        ws = workspace(lib.moe_router_backward_workspace_bytes(N, d, E), x.device)
    _check(lib.moe_router_backward(ctypes.byref(p), _ptr(x), _dt(x), _ptr(w_gate), _ptr(logits),
                                   _ptr(cand_ids), _ptr(expert_of), _ptr(row_of), _ptr(dgates),
                                   _ptr(counts_routed), float(alpha), float(beta),
                                   _ptr(dx_rows), _ptr(dx_shared), _ptr(noise_v), _ptr(dlogits),
                                   _ptr(dw_gate), _ptr(dlogit_bias), _ptr(dw_noise), _ptr(dx),
                                   _ptr(ws), ws.numel(), _stream(stream)))


# --------------------------------------------------------------------- layer
@dataclass
class LayerSpec:
    n_tokens: int
    d_model: int
    n_experts: int
    d_ff: int
    top_k: int
    act: int
    renormalize: bool
    overflow: int = DROPLESS
    capacity: int = -1
    n_cand: int = 0
    noise_seed: int = 0
    bias_rate: float = 1e-3
    shared_d_ff: int = 0
    h_fp32: bool = False
    expert_choice: bool = False  # experts pick their ec_capacity top tokens
    ec_capacity: int = 0


class MoELayer:
    """One MoE FFN layer forward through libmoe. Holds device weights and
    preallocated outputs/workspaces so repeated forwards allocate nothing.

    weights: dict with w_gate, logit_bias, select_bias, w_noise, w1, w3, w2,
    b1, b2, s1, s3, s2 and shared_{w1,w3,w2,s1,s3,s2} (device tensors/None).

    With spec.expert_choice the router's full score matrix feeds
    moe_expert_choice instead of moe_dispatch: every expert gets exactly
    cap = min(ec_capacity, N) rows and a token sums over the experts that
    chose it (combine with k = E).
    """

    def __init__(self, spec: LayerSpec, weights: dict, x_dtype=torch.bfloat16, device="cuda",
                 out_dtype=None, fused_gather=True, train=False, fuse_combine=True):
        self.spec = s = spec
        self.w = weights
        self.dev = torch.device(device)
        N, E, k = s.n_tokens, s.n_experts, s.top_k
        self.ec = bool(s.expert_choice)
        if self.ec:
            if s.ec_capacity < 1:
                raise ValueError("expert choice needs ec_capacity >= 1")
            k = 1  # the router's own top-k is unused; its scores_out feeds the selection
            self.cap = min(s.ec_capacity, N)
        C = 1 if self.ec else (s.n_cand or k)
        self.C = C
        # packed rows: N*k assignments (token choice) or E*cap (expert choice)
        R = E * self.cap if self.ec else N * k
        self.R = R
        dev = self.dev
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.cand_ids = torch.empty((N, C), **i32)
        self.cand_scores = torch.empty((N, C), **f32)
        self.gates = torch.empty((N, k), **f32)
        self.logits = torch.empty((N, E), **f32)
        self.score_sums = torch.empty(E + 1, dtype=torch.float64, device=dev)
        self.counts_routed = torch.empty(E, **i32)
        self.counts_kept = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.row_of = torch.empty((N, E if self.ec else k), **i32)
        self.expert_of = None if self.ec else torch.empty((N, k), **i32)
        self.perm_token = torch.empty(R, **i32)
        self.scores = torch.empty((N, E), **f32) if self.ec else None
        self.ec_gates = torch.empty((N, E), **f32) if self.ec else None
        # fused_gather: GEMM 1 reads token rows through perm_token, so no
        # packed copy of x is made; otherwise dispatch gathers x_perm first
        # (expert choice always reads through perm_token)
        self.fused_gather = fused_gather or self.ec
        self.x_perm = (None if self.fused_gather else
                       torch.empty((R, s.d_model), dtype=x_dtype, device=dev))
        # Expert outputs and the layer output stay fp32: the only bf16
        # rounding on the path is the intermediate h inside the grouped FFN.
        ydt = torch.float32
        self.y_rows = torch.empty((R, s.d_model), dtype=ydt, device=dev)
        self.out_dtype = out_dtype or torch.float32
        self.y = torch.empty((N, s.d_model), dtype=self.out_dtype, device=dev)
        self.f = torch.empty(E, **f32)
        self.P = torch.empty(E, **f32)
        self.scalars = torch.empty(4, **f32)
        self.ffn, self._keep = ffn_weights(weights["w1"], weights["w2"], weights.get("w3"),
                                           s.act, weights.get("b1"), weights.get("b2"),
                                           weights.get("s1"), weights.get("s3"),
                                           weights.get("s2"), s.h_fp32)
        self.shared = None
        if weights.get("shared_w1") is not None:
            self.shared, self._keep_sh = ffn_weights(
                weights["shared_w1"], weights["shared_w2"], weights.get("shared_w3"), s.act,
                None, None, weights.get("shared_s1"), weights.get("shared_s3"),
                weights.get("shared_s2"), s.h_fp32)
            self.sh_offsets = torch.tensor([0, N], **i32)
            self.y_shared = torch.empty((N, s.d_model), dtype=ydt, device=dev)
            # the always-on expert depends only on x: it runs on a side stream
            # (default priority) next to routing, dispatch and the routed FFN
            self.side = torch.cuda.Stream(device=dev)
            self.ev_x = torch.cuda.Event()
            self.ev_shared = torch.cuda.Event()
            self._shared_pending = False
        xdt = _dt(torch.empty(0, dtype=x_dtype))
        noise = int(weights.get("w_noise") is not None)
        # router weights as exact bf16 planes, split once (bf16 x, matrix-
        # core router); prepare_router() redoes it after the weights change
        self.router_planes = None
        if xdt == BF16 and s.d_model % 64 == 0:
            self.prepare_router()
        self.ws_router = workspace(lib.moe_router_workspace_bytes(N, s.d_model, E, noise), dev)
        self.ws_dispatch = workspace(lib.moe_dispatch_workspace_bytes(N, E, k), dev)
        self.ws_ffn = workspace(lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(self.ffn), xdt,
                                                                    R), dev)
        if self.shared is not None:
            self.ws_shared = workspace(lib.moe_grouped_ffn_workspace_bytes(
                ctypes.byref(self.shared), xdt, N), dev)
        # training: the experts' forward keeps its pre-activations and h
        self.train = bool(train)
        if self.train:
            if s.h_fp32:
                raise ValueError("training keeps h in bf16 (build the spec with h_fp32=False)")
            bf = dict(dtype=torch.bfloat16, device=dev)
            glu = s.act == SWIGLU
            self.preact = torch.empty((R, (2 if glu else 1) * s.d_ff), **bf)
            self.noise_v = (torch.empty((N, E), **f32) if weights.get("w_noise") is not None
                            else None)
            self.h = torch.empty((R, s.d_ff), **bf)
            # expert choice: slot j of a token is expert j in the backward's router step
            self.ec_expert_of = (torch.arange(E, **i32).repeat(N, 1).contiguous()
                                 if self.ec else None)
            if self.shared is not None:
                self.preact_sh = torch.empty((N, (2 if glu else 1) * s.shared_d_ff), **bf)
                self.h_sh = torch.empty((N, s.shared_d_ff), **bf)
            self._bwd = None
        # top-1 routing without a shared expert: the combine runs in GEMM 2's
        # epilogue (moe_grouped_ffn_combine_top1), y_rows is not written
        self.fused_combine = bool(fuse_combine and not self.ec and k == 1 and
                                  self.shared is None and not self.train and
                                  weights["w1"].dtype != torch.uint8 and
                                  self.out_dtype == torch.float32 and s.d_model % 4 == 0)
        self._forward_done = False

    def prepare_router(self, stream=None):
        """(Re)split w_gate / w_noise into the router's bf16 weight planes."""
        self.router_planes = moe_router_prepare(self.w["w_gate"], self.w.get("w_noise"),
                                                planes=self.router_planes, stream=stream)

    def route(self, x, logits_in=None, stream=None, noise_in=None):
        """noise_in (training with noisy gating and logits_in only): the noise
        pre-activations v = x W_noise^T that produced logits_in, kept for the
        backward pass (the router computes none when given logits)."""
        s, w = self.spec, self.w
        if self.train and self.noise_v is not None:
            if logits_in is not None:
                if noise_in is None:
                    raise ValueError("noisy gating with logits_in needs noise_in for training")
                self.noise_v.copy_(noise_in)
        moe_router_topk(x, w["w_gate"], top_k=1 if self.ec else s.top_k, n_cand=self.C,
                        renormalize=s.renormalize and not self.ec,
                        logit_bias=w.get("logit_bias"),
                        select_bias=None if self.ec else w.get("select_bias"),
                        w_noise=w.get("w_noise"), noise_seed=s.noise_seed, logits_in=logits_in,
                        cand_ids=self.cand_ids, cand_scores=self.cand_scores, gates=self.gates,
                        logits_out=self.logits, score_sums=self.score_sums,
                        scores_out=self.scores,
                        noise_out=self.noise_v if self.train else None,
                        w_planes=self.router_planes, ws=self.ws_router, stream=stream)

    def dispatch(self, x, stream=None):
        s = self.spec
        if self.ec:
            moe_expert_choice(self.scores, self.cap, offsets=self.offsets,
                              perm_token=self.perm_token, row_of=self.row_of,
                              gates=self.ec_gates, counts=self.counts_kept, stream=stream)
            return
        moe_dispatch(self.cand_ids, self.cand_scores, self.gates, n_experts=s.n_experts,
                     top_k=s.top_k, policy=s.overflow, capacity=s.capacity, x=x,
                     counts_routed=self.counts_routed, counts_kept=self.counts_kept,
                     offsets=self.offsets, row_of=self.row_of, expert_of=self.expert_of,
                     perm_token=self.perm_token, x_perm=self.x_perm, ws=self.ws_dispatch,
                     stream=stream)

    def _packed_rows(self, x):
        return (x, self.perm_token) if self.fused_gather else (self.x_perm, None)

    def start_shared(self, x, stream=None):
        """Launch the shared expert's FFN on the side stream once x is ready
        on `stream`; combine() waits for it."""
        if self.shared is None or self._shared_pending:
            return
        main = stream or torch.cuda.current_stream()
        self.ev_x.record(main)
        self.side.wait_event(self.ev_x)
        if self.train:
            moe_grouped_ffn_train(self.shared, x, self.sh_offsets, self.y_shared, self.preact_sh,
                                  self.h_sh, max_rows=self.spec.n_tokens, ws=self.ws_shared,
                                  stream=self.side)
        else:
            moe_grouped_ffn(self.shared, x, self.sh_offsets, self.y_shared,
                            max_rows=self.spec.n_tokens, ws=self.ws_shared, stream=self.side)
        self.ev_shared.record(self.side)
        self._shared_pending = True

    def experts(self, x, stream=None):
        rows, index = self._packed_rows(x)
        if self.train:
            moe_grouped_ffn_train(self.ffn, rows, self.offsets, self.y_rows, self.preact, self.h,
                                  row_index=index, max_rows=self.R, ws=self.ws_ffn,
                                  stream=stream)
        elif self.fused_combine:
            moe_grouped_ffn_combine_top1(self.ffn, rows, self.offsets, self.perm_token,
                                         self.row_of, self.gates, self.y, row_index=index,
                                         max_rows=self.R, ws=self.ws_ffn, stream=stream)
        else:
            moe_grouped_ffn(self.ffn, rows, self.offsets, self.y_rows, row_index=index,
                            max_rows=self.R, ws=self.ws_ffn, stream=stream)
        self.start_shared(x, stream)

    def combine(self, stream=None):
        if self.fused_combine:
            return  # done in the experts' GEMM 2 epilogue
        if self.shared is not None:
            (stream or torch.cuda.current_stream()).wait_event(self.ev_shared)
            self._shared_pending = False
        moe_combine(self.y_rows, self.row_of, self.ec_gates if self.ec else self.gates, self.y,
                    y_shared=self.y_shared if self.shared is not None else None, stream=stream)

    def stats(self, update_bias=False, stream=None):
        s = self.spec
        # expert choice: every expert is routed and keeps exactly cap rows
        routed = self.counts_kept if self.ec else self.counts_routed
        moe_balance_stats(s.n_tokens, s.top_k, routed, self.counts_kept,
                          self.score_sums, self.f, self.P, self.scalars,
                          select_bias=self.w.get("select_bias") if update_bias else None,
                          bias_rate=s.bias_rate, stream=stream)

    def capture(self, x, stats=True):
        """A HIP graph of one whole forward on x (torch.cuda.CUDAGraph): one
        replay relaunches every kernel of the layer (router, dispatch,
        grouped FFN, shared expert on its side stream, combine, statistics)
        with a single call, for launch-bound small batches. The graph reads x
        and writes self.y (and the other buffers) in place; the library
        makes no allocation, memset or host synchronisation inside a forward,
        so the captured work is exactly the eager one."""
        warm = torch.cuda.Stream(device=self.dev)
        warm.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(warm):
            self.forward(x, stats=stats)  # first launches set kernel attributes
        torch.cuda.current_stream(self.dev).wait_stream(warm)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, stats=stats)
        return g

    def forward(self, x, logits_in=None, stats=True, update_bias=False, stream=None,
                noise_in=None):
        self.start_shared(x, stream)
        self.route(x, logits_in, stream, noise_in)
        self.dispatch(x, stream)
        self.experts(x, stream)
        self.combine(stream)
        if stats:
            self.stats(update_bias, stream)
        self._forward_done = True
        return self.y


def _backward_buffers(layer, dw_dtype=torch.float32):
    s, dev = layer.spec, layer.dev
    E, d, F, N, R = s.n_experts, s.d_model, s.d_ff, s.n_tokens, layer.R
    f32 = dict(dtype=torch.float32, device=dev)
    wdt = dict(dtype=dw_dtype, device=dev)
    b = dict(d_rows=torch.empty((R, d), dtype=torch.bfloat16, device=dev),
             dgates=torch.empty((N, E if layer.ec else s.top_k), **f32),
             dx_rows=torch.empty((R, d), **f32),
             dw1=torch.empty((E, F, d), **wdt),
             dw3=torch.empty((E, F, d), **wdt) if s.act == SWIGLU else None,
             dw2=torch.empty((E, d, F), **wdt), dlogits=torch.empty((N, E), **f32),
             dw_gate=torch.empty((E, d), **f32), dx=torch.empty((N, d), **f32),
             dw_noise=torch.empty((E, d), **f32) if layer.noise_v is not None else None,
             dlogit_bias=torch.empty(E, **f32) if layer.w.get("logit_bias") is not None else None)
    ws_f = workspace(lib.moe_grouped_ffn_backward_workspace_bytes(
        ctypes.byref(layer.ffn), R, int(layer.fused_gather)), dev)
    if layer.shared is not None:
        Fs = s.shared_d_ff
        b.update(d_shared=torch.empty((N, d), dtype=torch.bfloat16, device=dev),
                 dx_shared=torch.empty((N, d), **f32), shared_dw1=torch.empty((1, Fs, d), **wdt),
                 shared_dw3=torch.empty((1, Fs, d), **wdt) if s.act == SWIGLU else None,
                 shared_dw2=torch.empty((1, d, Fs), **wdt))
        ws_s = workspace(lib.moe_grouped_ffn_backward_workspace_bytes(
            ctypes.byref(layer.shared), N, 0), dev)
        ws_f = workspace(max(ws_f.numel(), ws_s.numel()), dev)
    ws_r = workspace(lib.moe_router_backward_workspace_bytes(N, d, E), dev)
    return b, ws_f, ws_r


def _routing_for_backward(layer):
    """(gates, candidate ids, expert of each slot, routed counts, slots per
    token, renormalised) as the backward's combine and router steps see the
    forward's routing. Expert choice: a token's slots are all E experts
    (slot j = expert j, kept where expert j chose the token), its gates the
    chosen scores, not renormalised, and every expert routed its capacity."""
    s = layer.spec
    if layer.ec:
        return (layer.ec_gates, layer.ec_expert_of, layer.ec_expert_of, layer.counts_kept,
                s.n_experts, False)
    return (layer.gates, layer.cand_ids, layer.expert_of, layer.counts_routed, s.top_k,
            s.renormalize)


def layer_backward(layer, x, dy, alpha=0.0, beta=0.0, dw_dtype=torch.float32, stream=None):
    """Backward of the last `layer.forward` (the layer built with train=True):
    L = <dy, y> + alpha * Switch aux + beta * z-loss. Returns a dict of fp32
    device tensors: dx, dw_gate, dlogit_bias (or None), dw_noise (or None),
    dw1, dw3 (None unless SwiGLU), dw2,
    dlogits, dgates ([N][top_k], or [N][E] with expert choice: the gradient
    of each chosen pair's gate, 0 elsewhere), and with a shared expert
    shared_dw1/3/2 [1][...] (buffers reused by the next call). dw_dtype:
    float32, or bfloat16 for the expert weight gradients."""
    if not layer.train:
        raise ValueError("build the layer with train=True to run its backward pass")
    if not layer._forward_done:
        # the backward reads the forward's routing and saved activations
        raise ValueError("run the layer's forward before its backward pass")
    if layer._bwd is None or layer._bwd[0]["dw1"].dtype != dw_dtype:
        layer._bwd = _backward_buffers(layer, dw_dtype)
    b, ws_f, ws_r = layer._bwd
    s, w = layer.spec, layer.w
    sh = layer.shared is not None
    gates, cand, expert_of, routed, k, renorm = _routing_for_backward(layer)
    moe_combine_backward(dy, layer.y_rows, layer.row_of, gates, b["d_rows"], b["dgates"],
                         d_shared=b["d_shared"] if sh else None, stream=stream)
    rows, index = layer._packed_rows(x)
    moe_grouped_ffn_backward(layer.ffn, rows, layer.offsets, layer.preact, layer.h, b["d_rows"],
                             b["dx_rows"], b["dw1"], b["dw3"], b["dw2"], row_index=index,
                             max_rows=layer.R, ws=ws_f, stream=stream)
    if sh:
        # one expert over every token with gate 1 (the workspace is reused in stream order)
        moe_grouped_ffn_backward(layer.shared, x, layer.sh_offsets, layer.preact_sh, layer.h_sh,
                                 b["d_shared"], b["dx_shared"], b["shared_dw1"],
                                 b["shared_dw3"], b["shared_dw2"], max_rows=s.n_tokens, ws=ws_f,
                                 stream=stream)
    moe_router_backward(x, w["w_gate"], layer.logits, cand, expert_of, layer.row_of,
                        b["dgates"], routed, b["dlogits"], b["dw_gate"], b["dx"], top_k=k,
                        renormalize=renorm, alpha=alpha, beta=beta, dx_rows=b["dx_rows"],
                        dx_shared=b["dx_shared"] if sh else None,
                        dlogit_bias=b["dlogit_bias"], w_noise=w.get("w_noise"),
                        noise_seed=s.noise_seed, noise_v=layer.noise_v, dw_noise=b["dw_noise"],
                        ws=ws_r, stream=stream)
    return b


def spec_from_config(cfg) -> LayerSpec:
    """LayerSpec from a workload config object (duck-typed). Capacities come
    from moe_capacity: ceil(N * capacity_factor / E) under a dropping policy,
    ceil(N * top_k / E) tokens per expert under expert choice."""
    N, E = cfg.n_tokens, cfg.n_experts
    ec = bool(getattr(cfg, "expert_choice", False))
    cap = -1
    if cfg.overflow != DROPLESS:
        if cfg.capacity_factor is None:
            raise ValueError("a dropping policy needs a capacity factor")
        cap = capacity(N, E, cfg.capacity_factor)
    return LayerSpec(N, cfg.d_model, E, cfg.d_ff, cfg.top_k, cfg.act,
                     cfg.renormalize, cfg.overflow, cap, cfg.n_cand, cfg.noise_seed,
                     1e-3, cfg.shared_d_ff, bool(getattr(cfg, "h_fp32", False)), ec,
                     capacity(N, E, cfg.top_k) if ec else 0)
