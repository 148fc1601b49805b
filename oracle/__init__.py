"""fp64 CPU oracle of the sparse top-k MoE layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It shares no code with the HIP path
(sparse_mixture_experts_topk_amd/csrc) and neither imports the other; the
seeded input generator (sparse_mixture_experts_topk_amd.synthetic) is the only
module both use, and it holds none of the layer's arithmetic.
"""
from .moe_oracle import (NEAR_TIE, OracleResult, Permutation, Routing, capacity_select,
                         dequant_weight, fallback_select, fallback_targets, forward,
                         near_tie_next_tokens, near_tie_ranking_ok, near_tie_tokens, permutation, router_logits,
                         silu, swiglu, swiglu_act_quant, to_f64, topk_gate)
from . import fp8, brute, mxfp4

__all__ = ["NEAR_TIE", "OracleResult", "Permutation", "Routing", "capacity_select",
           "dequant_weight", "fallback_select", "fallback_targets", "forward",
           "near_tie_next_tokens", "near_tie_ranking_ok", "near_tie_tokens", "permutation", "router_logits", "silu",
           "swiglu", "swiglu_act_quant", "to_f64", "topk_gate", "fp8", "brute", "mxfp4"]
