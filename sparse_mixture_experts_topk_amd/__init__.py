"""Sparse top-k Mixture-of-Experts feed-forward layer for AMD MI355X (gfx950).

Thin Python binding of libmoe.so (C ABI in include/moe.h).  The functions
below carry the C names and only marshal arguments: torch tensors supply
device pointers and the current HIP stream, every step of the layer runs in
the library's HIP kernels.  There is no CPU or fallback path: if libmoe.so
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_CALL_DOWN, MOE_CALL_FORWARD, MOE_CALL_GATE_UP,
                   MOE_CALL_PERMUTE, MOE_CALL_ROUTE, MOE_DROPLESS, MOE_F32, MOE_FP8_E4M3, MOE_MXFP4,
                   MOE_NOALLOC_SCRATCH_BYTES, MOE_OVERFLOW_DROP, MOE_OVERFLOW_NEXT_BEST, MoeShape)

__all__ = ["MoEError", "MoeShape", "make_shape", "moe_status_string", "moe_version",
           "moe_workspace_bytes", "moe_route_topk", "moe_permute", "moe_expert_gemm_gate_up",
           "moe_expert_gemm_down", "moe_combine", "moe_forward", "moe_forward_noalloc",
           "MOE_NOALLOC_SCRATCH_BYTES", "MOE_F32", "MOE_BF16",
           "MOE_FP8_E4M3", "MOE_MXFP4", "MOE_DROPLESS", "MOE_CALL_PERMUTE", "MOE_CALL_GATE_UP",
           "MOE_CALL_DOWN", "MOE_CALL_FORWARD", "MOE_CALL_ROUTE", "MOE_OVERFLOW_DROP", "MOE_OVERFLOW_NEXT_BEST"]

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8_e4m3": MOE_FP8_E4M3, "mxfp4": MOE_MXFP4}
_OVF = {"drop": MOE_OVERFLOW_DROP, "next_best": MOE_OVERFLOW_NEXT_BEST}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {moe_status_string(status)} ({status})")


def make_shape(T: int, d_model: int, d_ff: int, n_experts: int = 8, top_k: int = 2,
               capacity: int = MOE_DROPLESS, act_dtype="bf16", w_dtype="bf16",
               overflow="drop", n_shared: int = 0) -> MoeShape:
    a = _DT.get(act_dtype, act_dtype)
    w = _DT.get(w_dtype, w_dtype)
    return MoeShape(T, d_model, d_ff, n_experts, top_k, capacity, a, w, _OVF.get(overflow, overflow),
                    n_shared)


def shape_of(cfg) -> MoeShape:
    """Shape of a synthetic.MoEConfig."""
    return make_shape(cfg.T, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, cfg.capacity,
                      cfg.act_dtype, cfg.w_dtype, cfg.overflow, cfg.n_shared)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)
    if t.device.type != "cuda":
        raise ValueError("MoE tensors must live in device memory")
    if not t.is_contiguous():
        raise ValueError("MoE tensors must be contiguous (row-major)")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MoEError(fn, status)


def moe_status_string(status: int) -> str:
    return _lib.load().moe_status_string(status).decode()


def moe_version() -> str:
    return _lib.load().moe_version().decode()


def moe_workspace_bytes(shape: MoeShape, call: int = MOE_CALL_FORWARD) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", _lib.load().moe_workspace_bytes(ctypes.byref(shape), call,
                                                                  ctypes.byref(n)))
    return n.value


def moe_route_topk(shape, x, w_gate, router_bias, topk_ids, topk_weights, logits=None,
                   next_ids=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_route_topk", _lib.load().moe_route_topk(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(router_bias), _p(topk_ids), _p(topk_weights),
        _p(logits), _p(next_ids), _p(workspace), ws_bytes, _stream(stream)))


def moe_permute(shape, topk_ids, topk_weights, next_ids, x, expert_counts, expert_offsets,
                perm_src, slot_to_row, drop_mask, x_perm, x_perm_scale=None, workspace=None,
                stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_permute", _lib.load().moe_permute(
        ctypes.byref(shape), _p(topk_ids), _p(topk_weights), _p(next_ids), _p(x), _p(expert_counts),
        _p(expert_offsets), _p(perm_src), _p(slot_to_row), _p(drop_mask), _p(x_perm),
        _p(x_perm_scale), _p(workspace), ws_bytes, _stream(stream)))


def moe_expert_gemm_gate_up(shape, x_perm, x_perm_scale, expert_offsets, w1, w3, w1_scale,
                            w3_scale, h, h_scale=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_expert_gemm_gate_up", _lib.load().moe_expert_gemm_gate_up(
        ctypes.byref(shape), _p(x_perm), _p(x_perm_scale), _p(expert_offsets), _p(w1), _p(w3),
        _p(w1_scale), _p(w3_scale), _p(h), _p(h_scale), _p(workspace), ws_bytes,
        _stream(stream)))


def moe_expert_gemm_down(shape, h, h_scale, expert_offsets, w2, w2_scale, y_perm,
                         workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_expert_gemm_down", _lib.load().moe_expert_gemm_down(
        ctypes.byref(shape), _p(h), _p(h_scale), _p(expert_offsets), _p(w2), _p(w2_scale),
        _p(y_perm), _p(workspace), ws_bytes, _stream(stream)))


def moe_combine(shape, y_perm, slot_to_row, topk_weights, y, stream=None):
    _check("moe_combine", _lib.load().moe_combine(
        ctypes.byref(shape), _p(y_perm), _p(slot_to_row), _p(topk_weights), _p(y),
        _stream(stream)))


def moe_forward(shape, x, w_gate, router_bias, w1, w3, w2, w1_scale, w3_scale, w2_scale, y,
                topk_ids_out=None, topk_weights_out=None, expert_counts_out=None,
                drop_mask_out=None, logits_out=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_forward", _lib.load().moe_forward(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(router_bias), _p(w1), _p(w3), _p(w2),
        _p(w1_scale), _p(w3_scale), _p(w2_scale), _p(y), _p(topk_ids_out),
        _p(topk_weights_out), _p(expert_counts_out), _p(drop_mask_out), _p(logits_out),
        _p(workspace), ws_bytes, _stream(stream)))


def moe_forward_noalloc(shape, x, w_gate, router_bias, w1, w3, w2, w1_scale, w3_scale, w2_scale, y,
                        topk_ids_out=None, topk_weights_out=None, expert_counts_out=None,
                        drop_mask_out=None, logits_out=None, stream=None):
    _check("moe_forward_noalloc", _lib.load().moe_forward_noalloc(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(router_bias), _p(w1), _p(w3), _p(w2),
        _p(w1_scale), _p(w3_scale), _p(w2_scale), _p(y), _p(topk_ids_out),
        _p(topk_weights_out), _p(expert_counts_out), _p(drop_mask_out), _p(logits_out),
        _stream(stream)))
