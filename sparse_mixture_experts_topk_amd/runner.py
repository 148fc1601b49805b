"""Device buffers and call sequences around the C ABI (allocation and marshalling only).

``DeviceInputs`` moves a synthetic.MoEInputs to the GPU; ``forward`` runs the
fused ``moe_forward``; ``staged`` runs the five boundary calls one after the
other and returns every intermediate, so each step can be checked on its own.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import (moe_combine, moe_expert_gemm_down, moe_expert_gemm_gate_up, moe_forward,
               moe_permute, moe_route_topk, moe_workspace_bytes, shape_of, MOE_CALL_DOWN,
               MOE_CALL_FORWARD, MOE_CALL_ROUTE)


def _dev(t: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.to(device).contiguous()


@dataclasses.dataclass
class DeviceInputs:
    cfg: object
    x: torch.Tensor
    w_gate: torch.Tensor
    router_bias: Optional[torch.Tensor]
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    w1_scale: Optional[torch.Tensor]
    w3_scale: Optional[torch.Tensor]
    w2_scale: Optional[torch.Tensor]

    @classmethod
    def from_host(cls, inp, device="cuda"):
        return cls(inp.cfg, *(_dev(getattr(inp, f), device) for f in
                              ("x", "w_gate", "router_bias", "w1", "w3", "w2", "w1_scale",
                               "w3_scale", "w2_scale")))

    def with_weights(self, w1, w3, w2):
        return dataclasses.replace(self, w1=w1, w3=w3, w2=w2)


def _act_dtype(cfg):
    return torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16


def _perm_dtype(cfg):
    if cfg.w_dtype == "fp8_e4m3":
        return torch.uint8
    return _act_dtype(cfg)


@dataclasses.dataclass
class ForwardBuffers:
    y: torch.Tensor
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    expert_counts: torch.Tensor
    drop_mask: torch.Tensor
    logits: torch.Tensor
    workspace: torch.Tensor


def alloc_forward(cfg, device="cuda", with_outputs=True) -> ForwardBuffers:
    T, d, E, k = cfg.T, cfg.d_model, cfg.n_experts, cfg.top_k
    shape = shape_of(cfg)
    ws = torch.empty(max(1, moe_workspace_bytes(shape, MOE_CALL_FORWARD)), dtype=torch.uint8,
                     device=device)
    y = torch.empty(T, d, dtype=_act_dtype(cfg), device=device)
    if not with_outputs:
        return ForwardBuffers(y, None, None, None, None, None, ws)
    return ForwardBuffers(y, torch.empty(T, k, dtype=torch.int32, device=device),
                          torch.empty(T, k, dtype=torch.float32, device=device),
                          torch.empty(E + cfg.n_shared, dtype=torch.int32, device=device),
                          torch.empty(T * k, dtype=torch.uint8, device=device),
                          torch.empty(T, E, dtype=torch.float32, device=device), ws)


def forward(di: DeviceInputs, buf: Optional[ForwardBuffers] = None, stream=None) -> ForwardBuffers:
    cfg = di.cfg
    if buf is None:
        buf = alloc_forward(cfg, di.x.device)
    moe_forward(shape_of(cfg), di.x, di.w_gate, di.router_bias, di.w1, di.w3, di.w2, di.w1_scale,
                di.w3_scale, di.w2_scale, buf.y, buf.topk_ids, buf.topk_weights,
                buf.expert_counts, buf.drop_mask, buf.logits, buf.workspace, stream)
    return buf


def staged(di: DeviceInputs, stream=None) -> dict:
    """The five boundary calls in sequence; returns every intermediate buffer."""
    cfg = di.cfg
    dev = di.x.device
    T, d, F, E, k, S = cfg.T, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, cfg.n_shared
    A = T * k                  # routed slots
    R = T * (k + S)            # slots incl. the shared expert = most rows
    shape = shape_of(cfg)
    fp8 = cfg.w_dtype == "fp8_e4m3"
    o = {}
    o["topk_ids"] = torch.empty(T, k, dtype=torch.int32, device=dev)
    o["topk_weights"] = torch.empty(T, k, dtype=torch.float32, device=dev)
    o["logits"] = torch.empty(T, E, dtype=torch.float32, device=dev)
    o["next_ids"] = torch.empty(T, 2, dtype=torch.int32, device=dev)
    route_ws = moe_workspace_bytes(shape, MOE_CALL_ROUTE)   # used when no logits buffer is passed
    o["route_ws"] = torch.empty(route_ws, dtype=torch.uint8, device=dev) if route_ws else None
    moe_route_topk(shape, di.x, di.w_gate, di.router_bias, o["topk_ids"], o["topk_weights"],
                   o["logits"], o["next_ids"], None, stream)
    o["expert_counts"] = torch.empty(E + S, dtype=torch.int32, device=dev)
    o["expert_offsets"] = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
    o["perm_src"] = torch.full((R,), -7, dtype=torch.int32, device=dev)
    o["slot_to_row"] = torch.empty(R, dtype=torch.int32, device=dev)
    o["drop_mask"] = torch.empty(A, dtype=torch.uint8, device=dev)
    o["x_perm"] = torch.empty(R, d, dtype=_perm_dtype(cfg), device=dev)
    o["x_perm_scale"] = torch.empty(R, d // 32, dtype=torch.uint8, device=dev) if fp8 else None
    moe_permute(shape, o["topk_ids"], o["topk_weights"], o["next_ids"], di.x, o["expert_counts"],
                o["expert_offsets"], o["perm_src"], o["slot_to_row"], o["drop_mask"], o["x_perm"],
                o["x_perm_scale"], None, stream)
    o["h"] = torch.empty(R, F, dtype=_perm_dtype(cfg), device=dev)
    o["h_scale"] = torch.empty(R, F // 32, dtype=torch.uint8, device=dev) if fp8 else None
    moe_expert_gemm_gate_up(shape, o["x_perm"], o["x_perm_scale"], o["expert_offsets"], di.w1,
                            di.w3, di.w1_scale, di.w3_scale, o["h"], o["h_scale"], None, stream)
    o["y_perm"] = torch.empty(R, d, dtype=torch.float32, device=dev)
    down_ws = moe_workspace_bytes(shape, MOE_CALL_DOWN)
    o["down_ws"] = torch.empty(down_ws, dtype=torch.uint8, device=dev) if down_ws else None
    moe_expert_gemm_down(shape, o["h"], o["h_scale"], o["expert_offsets"], di.w2, di.w2_scale,
                         o["y_perm"], o["down_ws"], stream)
    o["y"] = torch.empty(T, d, dtype=_act_dtype(cfg), device=dev)
    moe_combine(shape, o["y_perm"], o["slot_to_row"], o["topk_weights"], o["y"], stream)
    return o
