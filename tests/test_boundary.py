"""C ABI boundary checks that need no GPU: the library loads, exports every
symbol include/moe.h declares, and rejects bad arguments on the host before
enqueueing any device work."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_topk_amd as moe
from sparse_mixture_experts_topk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_permute", "moe_expert_gemm_gate_up", "moe_expert_gemm_down",
              "moe_combine", "moe_forward"):
        assert n in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    # symbols are C (unmangled) exports
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_status_strings():
    assert "gfx950" in moe.moe_version()
    assert moe.moe_status_string(0) == "MOE_OK"
    assert moe.moe_status_string(3) == "MOE_ERR_WORKSPACE"
    assert moe.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def _status(fn, *args):
    return getattr(_lib.load(), fn)(*args)


def S(**kw):
    base = dict(T=16, d_model=4096, d_ff=14336, n_experts=8, top_k=2, capacity=-1,
                act_dtype="bf16", w_dtype="bf16")
    base.update(kw)
    return moe.make_shape(**base)


@pytest.mark.parametrize("kw,expected", [
    (dict(), 0),
    (dict(T=-1), 1), (dict(T=(1 << 24) + 1), 1), (dict(n_experts=1), 1), (dict(top_k=0), 1),
    (dict(d_model=0), 1), (dict(capacity=-2), 1), (dict(act_dtype=7), 1), (dict(w_dtype=9), 1),
    (dict(d_model=100), 2), (dict(d_ff=4000), 2),
    # general top-k, many experts, a shared expert
    (dict(top_k=1), 0), (dict(top_k=3), 0), (dict(n_experts=256, top_k=8), 0),
    (dict(n_experts=256, top_k=8, n_shared=1), 0), (dict(n_experts=65), 0),
    (dict(n_experts=257), 2), (dict(n_experts=16, top_k=9), 2), (dict(top_k=9), 1),
    (dict(n_shared=2), 2), (dict(n_shared=-1), 1),
    (dict(act_dtype="f32", w_dtype="f32", n_experts=64, top_k=5), 0),
    (dict(act_dtype="f32", w_dtype="f32", n_experts=65), 2),
    (dict(top_k=3, capacity=10, overflow="next_best"), 2), (dict(top_k=3, overflow="next_best"), 0),
    (dict(w_dtype="mxfp4", T=64, n_shared=1, capacity=8), 0),
    (dict(w_dtype="mxfp4", T=65, n_shared=1, capacity=8), 2),
    (dict(act_dtype="f32", w_dtype="bf16"), 2), (dict(act_dtype="bf16", w_dtype="f32"), 2),
    (dict(act_dtype="f32", w_dtype="f32"), 0), (dict(capacity=0), 0), (dict(T=0), 0),
    (dict(w_dtype="fp8_e4m3"), 0), (dict(w_dtype="fp8_e4m3", d_model=4160), 2),
    (dict(w_dtype="fp8_e4m3", d_ff=14400), 2), (dict(act_dtype="f32", w_dtype="fp8_e4m3"), 2),
    (dict(overflow=2), 1), (dict(overflow=-1), 1), (dict(overflow="next_best"), 0),
    (dict(overflow="next_best", capacity=3), 0),
    # MXFP4 experts: bf16 activations, <= 64 rows per expert, d and F multiples of 256
    (dict(w_dtype="mxfp4"), 0), (dict(w_dtype="mxfp4", T=64), 0), (dict(w_dtype="mxfp4", T=65), 2),
    (dict(w_dtype="mxfp4", T=5000, capacity=64), 0), (dict(w_dtype="mxfp4", T=5000, capacity=65), 2),
    (dict(w_dtype="mxfp4", d_model=4160), 2), (dict(w_dtype="mxfp4", d_ff=14400), 2),
    (dict(act_dtype="f32", w_dtype="mxfp4"), 2), (dict(w_dtype=4), 1),
])
def test_workspace_query_validates_shape(kw, expected):
    n = ctypes.c_size_t(0)
    st = _status("moe_workspace_bytes", ctypes.byref(S(**kw)), moe.MOE_CALL_FORWARD, ctypes.byref(n))
    assert st == expected


def test_workspace_sizes():
    s = S(T=8192)
    ws = moe.moe_workspace_bytes(s, moe.MOE_CALL_FORWARD)
    A = 8192 * 2
    assert ws >= A * 4096 * 2 + A * 14336 * 2 + A * 4096 * 4
    assert moe.moe_workspace_bytes(s, moe.MOE_CALL_PERMUTE) == 0
    # the fallback round keeps the 3rd/4th-ranked experts of every token
    fb = moe.moe_workspace_bytes(S(T=8192, capacity=2560, overflow="next_best"))
    assert fb - moe.moe_workspace_bytes(S(T=8192, capacity=2560)) == A * 4
    assert moe.moe_workspace_bytes(S(T=8192, overflow="next_best")) == ws   # dropless: no round
    with pytest.raises(moe.MoEError):
        moe.moe_workspace_bytes(S(T=-5))
    assert _status("moe_workspace_bytes", ctypes.byref(s), 0, None) == 1


def test_workspace_covers_every_slot_with_a_shared_expert():
    # 8192 tokens x (8 routed + 1 shared) slots: x_perm, h (bf16) and y_perm (fp32) rows
    s = S(T=8192, d_model=4096, d_ff=2048, n_experts=256, top_k=8, n_shared=1)
    R = 8192 * 9
    assert moe.moe_workspace_bytes(s) >= R * (4096 * 2 + 2048 * 2 + 4096 * 4)
    s0 = S(T=8192, d_model=4096, d_ff=2048, n_experts=256, top_k=8)
    diff = moe.moe_workspace_bytes(s) - moe.moe_workspace_bytes(s0)
    assert diff >= 8192 * (4096 * 2 + 2048 * 2 + 4096 * 4)
    # the shared expert takes every token: > 64 rows per expert means the tiled bf16 path
    assert moe.moe_workspace_bytes(S(T=100, capacity=8, n_shared=1), moe.MOE_CALL_DOWN) > 0
    assert moe.moe_workspace_bytes(S(T=100, capacity=8), moe.MOE_CALL_DOWN) == 0


def test_route_workspace_for_many_experts():
    # bf16 with more than 64 experts: an fp32 [T, E] logit buffer unless `logits` is passed
    s = S(T=16, n_experts=256, top_k=8, n_shared=1)
    assert moe.moe_workspace_bytes(s, moe.MOE_CALL_ROUTE) == 16 * 256 * 4
    assert moe.moe_workspace_bytes(S(T=16), moe.MOE_CALL_ROUTE) == 0
    assert moe.moe_workspace_bytes(S(T=16, n_experts=64), moe.MOE_CALL_ROUTE) == 0
    assert moe.moe_workspace_bytes(s) >= moe.moe_workspace_bytes(S(T=16, n_experts=256, top_k=8)) + 16 * 4096 * 2
    dummy = 1 << 20
    b = ctypes.byref(s)
    assert _status("moe_route_topk", b, dummy, dummy, None, dummy, dummy, None, None, None, 0, None) == 3
    assert _status("moe_route_topk", b, dummy, dummy, None, dummy, dummy, None, None, dummy,
                   16 * 256 * 4 - 1, None) == 3
    assert _status("moe_route_topk", b, dummy, dummy, None, dummy, dummy, None, None, dummy + 8,
                   16 * 256 * 4, None) == 3


def test_forward_workspace_holds_the_decode_router_partials():
    # decode batches (T <= 16, E <= 16, top-2, dropless, no shared expert): moe_forward's router
    # writes eight partial 16 x 16 fp32 tiles (8 x 64 lanes x 16 B) before selecting; the same
    # shape with a capacity takes the staged router and needs none of it
    part = 8 * 64 * 16
    for w in ("bf16", "mxfp4"):
        fused = moe.moe_workspace_bytes(S(T=16, w_dtype=w))
        staged = moe.moe_workspace_bytes(S(T=16, w_dtype=w, capacity=16))
        assert fused - staged == part
    assert moe.moe_workspace_bytes(S(T=16, n_experts=17)) == moe.moe_workspace_bytes(
        S(T=16, n_experts=17, capacity=16))


def test_down_workspace_size_and_requirement():
    # many rows per expert (bf16): fp32 partial tiles for the split tail work
    big = S(T=8192)
    need = moe.moe_workspace_bytes(big, moe.MOE_CALL_DOWN)
    assert need == 256 * 2 * 256 * 384 * 4          # two 256 x 384 fp32 tiles per workgroup
    assert moe.moe_workspace_bytes(big, moe.MOE_CALL_FORWARD) >= need
    # the weight-streaming path (<= 64 rows per expert), fp8 and fp32 need none
    assert moe.moe_workspace_bytes(S(T=16), moe.MOE_CALL_DOWN) == 0
    assert moe.moe_workspace_bytes(S(T=30, capacity=64), moe.MOE_CALL_DOWN) == 0
    assert moe.moe_workspace_bytes(S(T=8192, w_dtype="fp8_e4m3"), moe.MOE_CALL_DOWN) == 0
    assert moe.moe_workspace_bytes(S(T=8192, d_model=128, d_ff=256, act_dtype="f32",
                                     w_dtype="f32"), moe.MOE_CALL_DOWN) == 0
    # missing, too small or misaligned workspace is rejected on the host
    dummy = 1 << 20
    b = ctypes.byref(big)
    assert _status("moe_expert_gemm_down", b, dummy, None, dummy, dummy, None, dummy, None, 0,
                   None) == 3
    assert _status("moe_expert_gemm_down", b, dummy, None, dummy, dummy, None, dummy, dummy,
                   need - 1, None) == 3
    assert _status("moe_expert_gemm_down", b, dummy, None, dummy, dummy, None, dummy, dummy + 8,
                   need, None) == 3


def test_calls_reject_null_and_misaligned_pointers_without_device_work():
    s = ctypes.byref(S())
    dummy = 1 << 20  # never dereferenced: validation fails first
    assert _status("moe_route_topk", s, None, dummy, None, dummy, dummy, None, None, None, 0, None) == 1
    assert _status("moe_route_topk", s, dummy + 2, dummy, None, dummy, dummy, None, None, None, 0, None) == 1
    assert _status("moe_route_topk", s, dummy, dummy, None, dummy, dummy, None, dummy + 4, None, 0, None) == 1
    assert _status("moe_combine", s, None, dummy, dummy, dummy, None) == 1
    assert _status("moe_expert_gemm_gate_up", s, dummy, None, None, dummy, dummy, None, None,
                   dummy, None, None, 0, None) == 1
    assert _status("moe_expert_gemm_down", s, dummy, None, dummy, None, None, None, None, 0, None) == 1
    # capacity mode needs a drop mask buffer
    sc = ctypes.byref(S(capacity=4))
    assert _status("moe_permute", sc, dummy, dummy, None, dummy, dummy, dummy, dummy, dummy, None,
                   dummy, None, None, 0, None) == 1
    # the overflow fallback needs the 3rd/4th-ranked experts
    sf = ctypes.byref(S(capacity=4, overflow="next_best"))
    assert _status("moe_permute", sf, dummy, dummy, None, dummy, dummy, dummy, dummy, dummy, dummy,
                   dummy, None, None, 0, None) == 1
    assert _status("moe_permute", ctypes.byref(S(overflow=7)), dummy, dummy, None, dummy, dummy,
                   dummy, dummy, dummy, dummy, dummy, None, None, 0, None) == 1
    # MXFP4 experts need their block scales
    s4 = ctypes.byref(S(w_dtype="mxfp4"))
    assert _status("moe_expert_gemm_gate_up", s4, dummy, None, dummy, dummy, dummy, None, dummy,
                   dummy, None, None, 0, None) == 1
    assert _status("moe_expert_gemm_down", s4, dummy, None, dummy, dummy, None, dummy, None, 0,
                   None) == 1
    # moe_forward: too small / missing workspace
    args = [dummy] * 6
    assert _status("moe_forward", s, dummy, dummy, None, dummy, dummy, dummy, None, None, None,
                   dummy, None, None, None, None, None, None, 0, None) == 3
    assert _status("moe_forward", s, dummy, dummy, None, dummy, dummy, dummy, None, None, None,
                   dummy, None, None, None, None, None, dummy, 1024, None) == 3
    del args


def test_unsupported_shapes_rejected_by_every_call():
    bad = ctypes.byref(S(n_experts=300, top_k=4))
    dummy = 1 << 20
    assert _status("moe_route_topk", bad, dummy, dummy, None, dummy, dummy, None, None, None, 0, None) == 2
    assert _status("moe_combine", bad, dummy, dummy, dummy, dummy, None) == 2


def test_empty_input_is_a_no_op():
    s = ctypes.byref(S(T=0))
    # all pointers NULL: T == 0 returns before any pointer check or launch
    assert _status("moe_route_topk", s, None, None, None, None, None, None, None, None, 0, None) == 0
    assert _status("moe_forward", s, *([None] * 15), None, 0, None) == 0
    assert _status("moe_combine", s, None, None, None, None, None) == 0


def test_python_binding_requires_device_tensors():
    import torch
    x = torch.zeros(16, 4096, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_route_topk(S(), x, x, None, x, x)


def test_noalloc_forward_rejects_shapes_beyond_its_scratch_on_the_host():
    """moe_forward_noalloc checks the shape against its fixed scratch before any device call."""
    lib = _lib.load()
    fake = 1 << 20                       # aligned non-NULL; never dereferenced on this path
    for cfg, expect in ((S(T=8192), 3), (S(T=0), 0), (S(T=16, top_k=9, n_experts=16), 2), (S(T=16, d_model=100), 2)):
        args = [ctypes.byref(cfg)] + [fake] * 15 + [None]
        args[3] = None                   # router bias
        assert lib.moe_forward_noalloc(*args) == expect
    big = ctypes.c_size_t(0)
    lib.moe_workspace_bytes(ctypes.byref(S(T=8192)), moe.MOE_CALL_FORWARD, ctypes.byref(big))
    assert big.value > moe.MOE_NOALLOC_SCRATCH_BYTES
    small = ctypes.c_size_t(0)
    lib.moe_workspace_bytes(ctypes.byref(S(T=64)), moe.MOE_CALL_FORWARD, ctypes.byref(small))
    assert small.value <= moe.MOE_NOALLOC_SCRATCH_BYTES
