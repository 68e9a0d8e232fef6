"""MI355X (gfx950) DeepSeekMoE layer forward: Python binding of libmoe.so.

The functions below mirror the C ABI in include/moe.h one to one
(moe_router, moe_permute, moe_expert_ffn, moe_combine, moe_forward).  They
check shapes, take device pointers and the current HIP stream from torch
tensors, and call the library; all arithmetic runs in its HIP kernels.
There is no fallback: without the built library importing this package
raises ImportError, and the library itself needs a GPU to run.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (MoeConfig, MoeError, config_from, make_config, status_string, last_error,
                   version, workspace_size, EXPORTS, LIB_PATH, NOALLOC_SCRATCH_BYTES)

__all__ = ["MoeConfig", "MoeError", "config_from", "make_config", "status_string", "last_error",
           "version", "workspace_size", "Workspace", "router", "permute", "expert_ffn",
           "combine", "forward", "forward_noalloc", "EXPORTS", "LIB_PATH",
           "NOALLOC_SCRATCH_BYTES"]

_ACT = {0: (torch.float32,), 1: (torch.bfloat16, torch.int16, torch.uint16)}
_W = {0: (torch.float32,), 1: (torch.bfloat16, torch.int16, torch.uint16),
      2: (torch.uint8, torch.float8_e4m3fn)}
_OUT = {0: torch.float32, 1: torch.bfloat16}


def _p(t, name, dtypes=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(s=None):
    return (s if s is not None else torch.cuda.current_stream()).cuda_stream


class Workspace:
    """Device workspace grown on demand (one per device); never shrinks.

    One cached workspace serves every call on its device that does not pass
    its own, so such calls must be ordered (one stream, or streams the caller
    synchronises); calls that may overlap pass separate workspaces.  Before a
    smaller cached buffer is dropped for a larger one the device is
    synchronised: the old buffer may still be in use by work queued on any
    stream, and torch's caching allocator only tracks the stream that
    allocated it."""

    _cache: dict = {}

    @classmethod
    def get(cls, cfg: MoeConfig, device) -> torch.Tensor:
        need = max(workspace_size(cfg), 256)
        dev = torch.device(device)
        ws = cls._cache.get(dev)
        if ws is None or ws.numel() < need:
            if ws is not None:
                torch.cuda.synchronize(dev)
                cls._cache.pop(dev)
                del ws
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            cls._cache[dev] = ws
        return ws


def _ws(cfg, ws, device):
    if ws is None:
        ws = Workspace.get(cfg, device)
    return ws.data_ptr(), ws.numel()


def router(cfg: MoeConfig, x, W_r, b=None, topk_idx=None, topk_gate=None, scores=None,
           want_scores=False, ws=None, stream=None):
    """moe_router: returns (topk_idx [T,k] int32, topk_gate [T,k] f32[, scores [T,N] f32])."""
    T, d, N, k = cfg.T, cfg.d, cfg.n_routed, cfg.k
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    if want_scores and scores is None:
        scores = torch.empty((T, N), dtype=torch.float32, device=dev)
    wsp, wsn = _ws(cfg, ws, dev)
    st = _lib.LIB.moe_router(
        cfg, _p(x, "x", _ACT[cfg.act_dtype], T * d), _p(W_r, "W_r", (torch.float32,), N * d),
        _p(b, "b", (torch.float32,), N, optional=True),
        _p(topk_idx, "topk_idx", (torch.int32,), T * k), _p(topk_gate, "topk_gate", (torch.float32,), T * k),
        _p(scores, "scores", (torch.float32,), T * N, optional=True), wsp, wsn, _stream(stream))
    _lib.check("moe_router", st)
    return (topk_idx, topk_gate, scores) if want_scores else (topk_idx, topk_gate)


def router_masked(cfg: MoeConfig, x, W_r, b=None, allow=None, mask_top=0, want_scores=False,
                  ws=None, stream=None):
    """moe_router_masked: the router with experts out of the selection.  ``allow``
    is a host sequence of N truthy values (None = all allowed); ``mask_top``
    removes each token's best remaining experts.  Returns (topk_idx, topk_gate[,
    scores])."""
    T, d, N, k = cfg.T, cfg.d, cfg.n_routed, cfg.k
    dev = x.device
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    scores = torch.empty((T, N), dtype=torch.float32, device=dev) if want_scores else None
    allow_buf = None
    if allow is not None:
        allow = [1 if a else 0 for a in allow]
        if len(allow) != N:
            raise ValueError(f"allow has {len(allow)} entries, expected {N}")
        allow_buf = (ctypes.c_uint8 * N)(*allow)
    wsp, wsn = _ws(cfg, ws, dev)
    st = _lib.LIB.moe_router_masked(
        cfg, _p(x, "x", _ACT[cfg.act_dtype], T * d), _p(W_r, "W_r", (torch.float32,), N * d),
        _p(b, "b", (torch.float32,), N, optional=True),
        ctypes.cast(allow_buf, ctypes.c_void_p) if allow_buf is not None else None, int(mask_top),
        _p(topk_idx, "topk_idx", (torch.int32,), T * k), _p(topk_gate, "topk_gate", (torch.float32,), T * k),
        _p(scores, "scores", (torch.float32,), T * N, optional=True), wsp, wsn, _stream(stream))
    _lib.check("moe_router_masked", st)
    return (topk_idx, topk_gate, scores) if want_scores else (topk_idx, topk_gate)


def bias_update(cfg: MoeConfig, b, counts, gamma: float, stream=None):
    """moe_bias_update: b [N] fp32 (device, in place) moves by gamma towards
    balance given the batch's counts [N] int32."""
    N = cfg.n_routed
    st = _lib.LIB.moe_bias_update(cfg, _p(b, "b", (torch.float32,), N),
                                  _p(counts, "counts", (torch.int32,), N), float(gamma),
                                  _stream(stream))
    _lib.check("moe_bias_update", st)
    return b


def permute(cfg: MoeConfig, topk_idx, x=None, want_x_perm=False, ws=None, stream=None):
    """moe_permute: returns dict(counts, offsets, row_token, slot_row[, x_perm])."""
    T, k, N, d = cfg.T, cfg.k, cfg.n_routed, cfg.d
    dev = topk_idx.device
    res = dict(counts=torch.empty(N, dtype=torch.int32, device=dev),
               offsets=torch.empty(N + 1, dtype=torch.int32, device=dev),
               row_token=torch.empty(T * k, dtype=torch.int32, device=dev),
               slot_row=torch.empty(T * k, dtype=torch.int32, device=dev))
    x_perm = None
    if want_x_perm:
        x_perm = torch.empty((T * k, d), dtype=x.dtype, device=dev)
        res["x_perm"] = x_perm
    wsp, wsn = _ws(cfg, ws, dev)
    st = _lib.LIB.moe_permute(
        cfg, _p(topk_idx, "topk_idx", (torch.int32,), T * k),
        _p(x, "x", _ACT[cfg.act_dtype], T * d, optional=True),
        res["counts"].data_ptr(), res["offsets"].data_ptr(), res["row_token"].data_ptr(),
        res["slot_row"].data_ptr(), _p(x_perm, "x_perm", optional=True), wsp, wsn, _stream(stream))
    _lib.check("moe_permute", st)
    return res


def expert_ffn(cfg: MoeConfig, n_experts: int, offsets, max_rows: int, x_rows, W1, W3, W2,
               s1=None, s3=None, s2=None, row_index=None, inter: int = 0, y_rows=None, ws=None,
               stream=None):
    """moe_expert_ffn: grouped SwiGLU experts; returns y_rows [max_rows, d]."""
    d = cfg.d
    I = inter if inter > 0 else cfg.inter
    dev = x_rows.device
    if y_rows is None:
        y_rows = torch.empty((max_rows, d), dtype=x_rows.dtype, device=dev)
    wsp, wsn = _ws(cfg, ws, dev)
    wd = _W[cfg.w_dtype]
    st = _lib.LIB.moe_expert_ffn(
        cfg, n_experts, _p(offsets, "offsets", (torch.int32,), n_experts + 1), max_rows, inter,
        _p(x_rows, "x_rows", _ACT[cfg.act_dtype]),
        _p(row_index, "row_index", (torch.int32,), optional=True),
        _p(W1, "W1", wd, n_experts * I * d), _p(W3, "W3", wd, n_experts * I * d),
        _p(W2, "W2", wd, n_experts * d * I),
        _p(s1, "s1", (torch.float32,), optional=True), _p(s3, "s3", (torch.float32,), optional=True),
        _p(s2, "s2", (torch.float32,), optional=True),
        _p(y_rows, "y_rows", _ACT[cfg.act_dtype]), wsp, wsn, _stream(stream))
    _lib.check("moe_expert_ffn", st)
    return y_rows


def combine(cfg: MoeConfig, y_perm, slot_row, topk_gate, y_shared=None, residual=None, out=None,
            stream=None):
    """moe_combine: out = residual + y_shared + sum_j gate_j * y_perm[slot_row]."""
    T, d, k = cfg.T, cfg.d, cfg.k
    if out is None:
        out = torch.empty((T, d), dtype=_OUT[cfg.out_dtype], device=y_perm.device)
    st = _lib.LIB.moe_combine(
        cfg, _p(y_perm, "y_perm", _ACT[cfg.act_dtype], T * k * d),
        _p(slot_row, "slot_row", (torch.int32,), T * k),
        _p(topk_gate, "topk_gate", (torch.float32,), T * k),
        _p(y_shared, "y_shared", _ACT[cfg.act_dtype], T * d, optional=True),
        _p(residual, "residual", _ACT[cfg.act_dtype], T * d, optional=True),
        _p(out, "out", (_OUT[cfg.out_dtype],), T * d), _stream(stream))
    _lib.check("moe_combine", st)
    return out


def _forward_args(cfg: MoeConfig, x, W_r, b, experts: dict, shared, out, want_routing):
    """The moe_forward arguments from cfg through counts_out, and the returned tensors."""
    T, d, N, k, I, S = cfg.T, cfg.d, cfg.n_routed, cfg.k, cfg.inter, cfg.n_shared
    dev = x.device
    if out is None:
        out = torch.empty((T, d), dtype=_OUT[cfg.out_dtype], device=dev)
    idx = gate = counts = None
    if want_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty(N, dtype=torch.int32, device=dev)
    wd = _W[cfg.w_dtype]
    f32 = (torch.float32,)
    sh = shared or {}
    args = (
        cfg, _p(x, "x", _ACT[cfg.act_dtype], T * d), _p(W_r, "W_r", f32, N * d),
        _p(b, "b", f32, N, optional=True),
        _p(experts["w1"], "W1", wd, N * I * d), _p(experts["w3"], "W3", wd, N * I * d),
        _p(experts["w2"], "W2", wd, N * d * I),
        _p(experts.get("s1"), "s1", f32, optional=True), _p(experts.get("s3"), "s3", f32, optional=True),
        _p(experts.get("s2"), "s2", f32, optional=True),
        _p(sh.get("w1"), "W1s", wd, S * I * d, optional=True),
        _p(sh.get("w3"), "W3s", wd, S * I * d, optional=True),
        _p(sh.get("w2"), "W2s", wd, S * d * I, optional=True),
        _p(sh.get("s1"), "s1s", f32, optional=True), _p(sh.get("s3"), "s3s", f32, optional=True),
        _p(sh.get("s2"), "s2s", f32, optional=True),
        _p(out, "out", (_OUT[cfg.out_dtype],), T * d),
        _p(idx, "topk_idx_out", optional=True), _p(gate, "topk_gate_out", optional=True),
        _p(counts, "counts_out", optional=True))
    return args, ((out, idx, gate, counts) if want_routing else out)


def forward(cfg: MoeConfig, x, W_r, b, experts: dict, shared=None, out=None, want_routing=False,
            ws=None, stream=None, side_stream=None):
    """moe_forward: the whole layer.  ``experts`` / ``shared`` are dicts with
    w1, w3, w2 (and s1, s3, s2 for fp8).  Returns out [T, d], plus
    (topk_idx, topk_gate, counts) when want_routing is set."""
    args, res = _forward_args(cfg, x, W_r, b, experts, shared, out, want_routing)
    wsp, wsn = _ws(cfg, ws, x.device)
    st = _lib.LIB.moe_forward(*args, wsp, wsn, _stream(stream),
                              _stream(side_stream) if side_stream is not None else None)
    _lib.check("moe_forward", st)
    return res


def forward_noalloc(cfg: MoeConfig, x, W_r, b, experts: dict, shared=None, out=None,
                    want_routing=False, stream=None, side_stream=None):
    """moe_forward_noalloc: moe_forward on the library's static per-GPU scratch
    array (no workspace argument; configs whose workspace exceeds
    NOALLOC_SCRATCH_BYTES are rejected).  Calls that overlap on one GPU race on
    that array.  Returns what forward() returns."""
    args, res = _forward_args(cfg, x, W_r, b, experts, shared, out, want_routing)
    st = _lib.LIB.moe_forward_noalloc(*args, _stream(stream),
                                      _stream(side_stream) if side_stream is not None else None)
    _lib.check("moe_forward_noalloc", st)
    return res
