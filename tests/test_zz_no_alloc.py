"""moe_forward_noalloc, the entry point for callers that cannot allocate device memory,
against moe_forward (the same kernels with a caller workspace): outputs must agree bit for
bit, on two calls in a row with the second on a smaller input, for each weight format."""
import dataclasses
import sys

import pytest
import torch

import sparse_mixture_experts_topk_amd as moe
from sparse_mixture_experts_topk_amd import runner, synthetic

from parity import cached_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def shrink(di, T):
    """The same weights with only the first T tokens."""
    return dataclasses.replace(di, cfg=di.cfg.replace(T=T), x=di.x[:T].contiguous())


def noalloc_forward(di):
    cfg = di.cfg
    buf = runner.alloc_forward(cfg)          # the caller's output buffers
    moe.moe_forward_noalloc(moe.shape_of(cfg), di.x, di.w_gate, di.router_bias, di.w1, di.w3,
                            di.w2, di.w1_scale, di.w3_scale, di.w2_scale, buf.y, buf.topk_ids,
                            buf.topk_weights, buf.expert_counts, buf.drop_mask, buf.logits)
    return buf


def assert_same(got, ref, what):
    for f in ("y", "topk_ids", "topk_weights", "expert_counts", "logits"):
        assert torch.equal(getattr(got, f), getattr(ref, f)), f"{what}: {f} differs from moe_forward"
    if ref.drop_mask is not None and di_capacity(got):
        assert torch.equal(got.drop_mask, ref.drop_mask), f"{what}: drop mask differs"


def di_capacity(buf):
    return buf.drop_mask is not None


def mid(name, **kw):
    base = dict(name=name, T=48, d_model=512, d_ff=768, n_experts=8, act_dtype="bf16",
                w_dtype="bf16", x_std=1.0, wg_std=512 ** -0.5, w13_std=0.05, w2_std=0.05, seed=71)
    base.update(kw)
    return synthetic.MoEConfig(**base)


CASES = {
    "decode_bf16": lambda: runner.DeviceInputs.from_host(cached_inputs("decode_bf16")),
    "capacity_fallback": lambda: runner.DeviceInputs.from_host(synthetic.make_inputs(
        mid("na_cap", T=64, capacity=12, overflow="next_best", router_bias="zipf1.2"))),
    "fp8": lambda: runner.DeviceInputs.from_host(synthetic.make_inputs(
        mid("na_fp8", T=40, w_dtype="fp8_e4m3", seed=72))),
    "mxfp4": lambda: runner.DeviceInputs.from_host(synthetic.make_inputs(
        mid("na_mx4", T=40, w_dtype="mxfp4", seed=73))),
    "topk8_shared_e256": lambda: runner.DeviceInputs.from_host(synthetic.make_inputs(
        mid("na_fg", T=24, n_experts=256, top_k=8, n_shared=1, d_ff=256, seed=74))),
}


@pytest.mark.parametrize("case,small_T", [("decode_bf16", 5), ("capacity_fallback", 9), ("fp8", 3),
                                          ("mxfp4", 1), ("topk8_shared_e256", 2)])
def test_noalloc_matches_moe_forward_on_two_calls(case, small_T):
    di = CASES[case]()
    small = shrink(di, small_T)
    say(f"moe_forward_noalloc vs moe_forward: {case} T={di.cfg.T} then T={small_T}")
    ref_big = runner.forward(di)
    ref_small = runner.forward(small)
    torch.cuda.synchronize()
    got_big = noalloc_forward(di)
    torch.cuda.synchronize()
    assert_same(got_big, ref_big, f"{case} T={di.cfg.T}")
    got_small = noalloc_forward(small)        # second call, smaller input, same scratch
    torch.cuda.synchronize()
    assert_same(got_small, ref_small, f"{case} T={small_T}")
    # the reference again after the scratch holds the smaller call's contents
    again = runner.forward(di)
    got_again = noalloc_forward(di)
    torch.cuda.synchronize()
    assert_same(got_again, again, f"{case} T={di.cfg.T}, third call")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    say("moe_forward_noalloc: prefill shape beyond the scratch array")
    cfg = synthetic.CONFIGS["prefill_bf16"]
    shape = moe.shape_of(cfg)
    assert moe.moe_workspace_bytes(shape) > moe.MOE_NOALLOC_SCRATCH_BYTES
    t = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.moe_forward_noalloc(shape, t, t, None, t, t, t, None, None, None, t)
    assert e.value.status == 3          # MOE_ERR_WORKSPACE, nothing enqueued
