"""ctypes declarations of libmoe.so (include/moe.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
MOE_DROPLESS = -1
MOE_OVERFLOW_DROP, MOE_OVERFLOW_NEXT_BEST = 0, 1
MOE_CALL_PERMUTE, MOE_CALL_GATE_UP, MOE_CALL_DOWN, MOE_CALL_FORWARD, MOE_CALL_ROUTE = range(5)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol include/moe.h declares.
EXPORTS = ("moe_status_string", "moe_version", "moe_workspace_bytes", "moe_route_topk",
           "moe_permute", "moe_expert_gemm_gate_up", "moe_expert_gemm_down", "moe_combine",
           "moe_forward", "moe_forward_noalloc")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("overflow", ctypes.c_int32),
                ("n_shared", ctypes.c_int32)]


P = ctypes.c_void_p
I32 = ctypes.c_int32
SZ = ctypes.c_size_t
SHAPE = ctypes.POINTER(MoeShape)

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [I32]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (I32, [SHAPE, I32, ctypes.POINTER(SZ)]),
    "moe_route_topk": (I32, [SHAPE, P, P, P, P, P, P, P, P, SZ, P]),
    "moe_permute": (I32, [SHAPE, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
    "moe_expert_gemm_gate_up": (I32, [SHAPE, P, P, P, P, P, P, P, P, P, P, SZ, P]),
    "moe_expert_gemm_down": (I32, [SHAPE, P, P, P, P, P, P, P, SZ, P]),
    "moe_combine": (I32, [SHAPE, P, P, P, P, P]),
    "moe_forward": (I32, [SHAPE, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
    "moe_forward_noalloc": (I32, [SHAPE, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_topk_amd.build_lib` "
                               "(the MoE layer has no CPU or fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
