"""GPU parity: every boundary call and the fused layer against the fp64 oracle.

All calls go through the C ABI (libmoe.so) via the thin Python binding.  Each
test prints its case before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_topk_amd as moe
from sparse_mixture_experts_topk_amd import runner, synthetic
from parity import (adjusted_oracle, assert_close, cached_inputs, check_next, check_permutation,
                    check_routing, rel_errors, sample_tokens, tile_coverage, to_np, token_of_slot,
                    tol_key)

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def record(case, **metrics):
    """Append measured error figures, one JSON line per case, to the file that the environment
    variable MOE_PARITY_METRICS names (nothing is written when it is unset)."""
    import json
    import os
    path = os.environ.get("MOE_PARITY_METRICS")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": case, **{k: float(v) for k, v in metrics.items()}}) + "\n")


def mid_cfg(name, **kw):
    base = dict(name=name, T=1536, d_model=512, d_ff=448, n_experts=4, act_dtype="bf16",
                w_dtype="bf16", x_std=1.0, wg_std=512 ** -0.5, w13_std=0.05, w2_std=0.05, seed=1)
    base.update(kw)
    return synthetic.MoEConfig(**base)


def run_staged_and_check(cfg, inputs=None, tokens=None, check_h=True, tile_rows=256):
    inputs = inputs if inputs is not None else synthetic.make_inputs(cfg)
    say(f"staged {cfg.name} T={cfg.T} d={cfg.d_model} F={cfg.d_ff} E={cfg.n_experts} "
        f"k={cfg.top_k} shared={cfg.n_shared} cap={cfg.capacity} overflow={cfg.overflow} "
        f"{cfg.act_dtype}/{cfg.w_dtype}")
    di = runner.DeviceInputs.from_host(inputs)
    st = runner.staged(di)
    torch.cuda.synchronize()
    gpu_ids = to_np(st["topk_ids"])
    marks = to_np(st["drop_mask"]).reshape(-1, cfg.top_k)
    fallback = cfg.capacity >= 0 and cfg.overflow == "next_best"
    gpu_next = to_np(st["next_ids"]) if fallback else None
    gpu_keep = (marks == 0) if fallback else ~marks.astype(bool)
    base, res = adjusted_oracle(inputs, gpu_ids, gpu_keep, tokens=tokens, want_h=check_h,
                                gpu_next=gpu_next, gpu_status=marks if fallback else None)
    key = tol_key(cfg)
    logit_atol = 1e-5 if cfg.act_dtype == "f32" else 3e-4
    check_routing(base, gpu_ids, to_np(st["topk_weights"]), to_np(st["logits"]), logit_atol)
    # the router writes the 3rd/4th-ranked experts whenever asked (runner.staged always asks)
    check_next(base, to_np(st["next_ids"]), gpu_ids)
    check_permutation(res, st)
    n = int(res.perm.offsets[-1])
    row_tok = token_of_slot(res.perm.perm_src, cfg.T, cfg.top_k)
    rows = np.arange(n) if tokens is None else np.flatnonzero(np.isin(row_tok, np.asarray(tokens)))
    # x_perm is a copy of the token rows (bit-exact)
    if cfg.w_dtype != "fp8_e4m3":
        xs = st["x_perm"][torch.from_numpy(rows).cuda()].cpu()
        src = inputs.x[torch.from_numpy(row_tok[rows])]
        assert torch.equal(xs, src), "x_perm is not an exact copy of x"
    else:
        # fp8: x_perm holds block-quantised codes; they must equal the oracle's exactly
        codes, ex, _ = oracle.fp8.block_quantize(oracle.to_f64(inputs.x)[row_tok[rows]])
        idx = torch.from_numpy(rows).cuda()
        assert np.array_equal(to_np(st["x_perm"][idx]), codes), "fp8 x codes differ"
        assert np.array_equal(to_np(st["x_perm_scale"][idx]).astype(np.int64) - 127, ex), "x scales differ"
    h_fro = np.nan
    if check_h:
        idx = torch.from_numpy(rows).cuda()
        if cfg.w_dtype == "fp8_e4m3":
            q = oracle.fp8.e4m3_decode(to_np(st["h"][idx]))
            sc = np.repeat(to_np(st["h_scale"][idx]).astype(np.int64) - 127, 32, axis=1)
            h_gpu = q * np.exp2(sc)
        else:
            h_gpu = to_np(st["h"][idx].float())
        h_fro, _ = assert_close(h_gpu, res.h[rows], key, "h (gate/up + SwiGLU)")
    yp = to_np(st["y_perm"][torch.from_numpy(rows).cuda()])
    yp_fro, _ = assert_close(yp, res.y_perm[rows], key, "y_perm (down)")
    want = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    y = to_np(st["y"].float())[want]
    fro, mx = assert_close(y, res.y[want], key, "y (layer output)")
    say(f"  y rel_frob={fro:.3e} rel_max={mx:.3e}")
    hit, tot = tile_coverage(res, want, tile_rows)
    record(cfg.name, h_rel_frob=h_fro, y_perm_rel_frob=yp_fro, y_rel_frob=fro, y_rel_max=mx,
           tokens_checked=len(want), token_tiles_checked=hit, token_tiles=tot,
           dropped=int((~res.keep).sum()))
    return st, res, inputs


# ---------------------------------------------------------------- routing ---

def test_worked_example_through_route_kernel():
    """Interview article worked example: W_g = I makes the logits the printed scores."""
    say("worked example via moe_route_topk (fp32, d=64, W_g = I)")
    scores = [2.1, 0.3, 1.4, -0.5, 0.0, 0.9, -1.2, 0.2]
    d = 64
    x = torch.zeros(1, d, dtype=torch.float32)
    x[0, :8] = torch.tensor(scores)
    wg = torch.zeros(8, d, dtype=torch.float32)
    wg[:, :8] = torch.eye(8)
    shape = moe.make_shape(1, d, 64, 8, act_dtype="f32", w_dtype="f32")
    ids = torch.empty(1, 2, dtype=torch.int32, device="cuda")
    w = torch.empty(1, 2, dtype=torch.float32, device="cuda")
    lg = torch.empty(1, 8, dtype=torch.float32, device="cuda")
    moe.moe_route_topk(shape, x.cuda(), wg.cuda(), None, ids, w, lg)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [[0, 2]]
    assert np.round(w.cpu().numpy()[0].astype(np.float64), 4).tolist() == [0.6682, 0.3318]
    assert abs(float(w[0, 0]) - 0.6681877722) < 1e-6
    assert torch.equal(lg.cpu(), x[:, :8])


@pytest.mark.parametrize("E", [2, 8, 16, 33, 64])
def test_route_expert_counts(E):
    cfg = synthetic.MoEConfig(name=f"route_E{E}", T=301, d_model=192, d_ff=64, n_experts=E,
                              wg_std=192 ** -0.5, seed=4)
    inp = synthetic.make_inputs(cfg, with_weights=False)
    say(f"route E={E} T=301 d=192 bf16")
    shape = moe.shape_of(cfg)
    ids = torch.empty(cfg.T, 2, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, 2, dtype=torch.float32, device="cuda")
    lg = torch.empty(cfg.T, E, dtype=torch.float32, device="cuda")
    moe.moe_route_topk(shape, inp.x.cuda(), inp.w_gate.cuda(), None, ids, w, lg)
    torch.cuda.synchronize()
    res = oracle.forward(inp, tokens=[])
    check_routing(res, to_np(ids), to_np(w), to_np(lg), 3e-4)


def test_route_ties_go_to_lower_index():
    say("route with duplicated router rows (exact ties)")
    cfg = synthetic.MoEConfig(name="ties", T=200, d_model=128, d_ff=64, wg_std=128 ** -0.5, seed=5)
    inp = synthetic.make_inputs(cfg, with_weights=False)
    wg = inp.w_gate.clone()
    wg[5] = wg[2]
    wg[7] = wg[2]
    inp.w_gate = wg
    shape = moe.shape_of(cfg)
    ids = torch.empty(cfg.T, 2, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, 2, dtype=torch.float32, device="cuda")
    moe.moe_route_topk(shape, inp.x.cuda(), wg.cuda(), None, ids, w, None)
    torch.cuda.synchronize()
    g = to_np(ids)
    # rows 2, 5, 7 give bit-identical logits: 7 can never be picked, and 5 only
    # as the second slot right after 2 (their shared logit is the largest).
    assert not np.any(g == 7)
    has5 = np.any(g == 5, axis=1)
    assert has5.any() and np.all(g[has5] == [2, 5])
    res = oracle.forward(inp, tokens=[])
    assert np.array_equal(g, res.routing.ids)
    # all rows equal: every token picks (0, 1) with weights 1/2
    wg_all = wg.clone()
    wg_all[:] = wg[0]
    moe.moe_route_topk(shape, inp.x.cuda(), wg_all.cuda(), None, ids, w, None)
    torch.cuda.synchronize()
    assert np.all(to_np(ids) == [0, 1]) and np.all(to_np(w) == 0.5)


# ------------------------------------------------------------ full steps ---

def test_tiny_fp32_config_full():
    run_staged_and_check(synthetic.CONFIGS["tiny_fp32"])


def test_mid_bf16_prefill_path_ragged_tiles():
    # ~384 rows per expert -> 2 token tiles of 256 (ragged); F = 448 -> 3.5 channel tiles
    run_staged_and_check(mid_cfg("mid_prefill"))


def test_mid_bf16_prefill_many_tiles():
    run_staged_and_check(mid_cfg("mid_prefill_e2", T=1300, n_experts=2, d_ff=320, seed=2))


def test_mid_bf16_decode_path():
    # T <= 64: the weight-streaming kernels; up to 40 rows per expert -> 3 token tiles of 16
    run_staged_and_check(mid_cfg("mid_decode", T=40, n_experts=8, seed=3))


@pytest.mark.parametrize("T,seed,most_rows", [(2, 41, 1), (8, 40, 4), (10, 40, 5), (14, 54, 8),
                                              (16, 42, 9)])
def test_bf16_decode_token_tile_heights(T, seed, most_rows):
    """The bf16 weight-streaming kernels pack 4, 2 or 1 token operands per load instruction for a
    token tile of at most 4, 8 or 16 rows (gate/up at d = 512: 128-element stages, up to 4; down
    and the fused down + combine at F = 448: 64-element stages, up to 2); each band and its edges
    against the oracle (staged calls) and the fused call bitwise against the staged one."""
    cfg = mid_cfg(f"bf16_rows{most_rows}", T=T, n_experts=8, seed=seed)
    st, res, inputs = run_staged_and_check(cfg)
    assert int(res.perm.counts.max()) == most_rows
    b = runner.forward(runner.DeviceInputs.from_host(inputs))
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y)


def test_mid_bf16_single_token():
    run_staged_and_check(mid_cfg("mid_t1", T=1, n_experts=8, seed=6))


def test_mid_capacity_zipf():
    T = 1000
    cfg = mid_cfg("mid_capacity", T=T, n_experts=8, capacity=synthetic.capacity_from_factor(T, 2, 8),
                  router_bias="zipf1.2", seed=7)
    st, res, _ = run_staged_and_check(cfg)
    assert (~res.keep).sum() > 0, "the skewed case must drop assignments"


def test_capacity_zero_drops_everything():
    cfg = mid_cfg("cap0", T=300, n_experts=8, capacity=0, seed=8)
    st, res, _ = run_staged_and_check(cfg, check_h=False)
    assert torch.count_nonzero(st["y"]).item() == 0
    assert to_np(st["drop_mask"]).all()


def test_capacity_one_and_large():
    run_staged_and_check(mid_cfg("cap1", T=200, n_experts=8, capacity=1, seed=9))
    run_staged_and_check(mid_cfg("cap_big", T=200, n_experts=8, capacity=10_000, seed=9))


def test_capacity_expert_beyond_lds_key_buffer():
    # one expert receives more than 8192 assignments: its cutoff comes from the
    # radix select over global memory instead of the in-LDS sort
    T = 12000
    cfg = mid_cfg("cap_many", T=T, d_model=64, d_ff=64, n_experts=8, router_bias="zipf1.2",
                  capacity=9000, wg_std=64 ** -0.5, seed=12)
    st, res, _ = run_staged_and_check(cfg, check_h=False)
    loads = np.bincount(to_np(st["topk_ids"]).ravel(), minlength=8)
    assert loads.max() > 9000 > 8192, loads
    assert (~res.keep).sum() > 0


def test_fallback_worked_example_through_gpu():
    """Hand-worked overflow fallback case (oracle pin): E = 4, capacity 1, W_g = I."""
    say("overflow fallback worked example (fp32, d=64, E=4, capacity 1)")
    logits = [[4, 3, 2, 1], [3, 4, 1, 2], [3.5, 0, 0.5, 0.25]]
    cfg = synthetic.MoEConfig(name="fb_worked", T=3, d_model=64, d_ff=64, n_experts=4, capacity=1,
                              overflow="next_best", act_dtype="f32", w_dtype="f32",
                              wg_std=64 ** -0.5, w13_std=0.1, w2_std=0.1, seed=13)
    inp = synthetic.make_inputs(cfg)
    x = torch.zeros(3, 64, dtype=torch.float32)
    x[:, :4] = torch.tensor(logits, dtype=torch.float32)
    wg = torch.zeros(4, 64, dtype=torch.float32)
    wg[:, :4] = torch.eye(4)
    inp.x, inp.w_gate = x, wg
    st, res, _ = run_staged_and_check(cfg, inputs=inp)
    assert to_np(st["topk_ids"]).tolist() == [[0, 1], [1, 0], [0, 2]]
    assert to_np(st["next_ids"]).tolist() == [[2, 3], [3, 2], [3, 1]]
    assert to_np(st["drop_mask"]).tolist() == [1, 2, 0, 1, 0, 0]
    assert to_np(st["expert_counts"]).tolist() == [1, 1, 1, 1]
    assert to_np(st["perm_src"])[:4].tolist() == [4, 2, 5, 1]


def test_mid_capacity_fallback_zipf():
    T = 1000
    cfg = mid_cfg("mid_fallback", T=T, n_experts=8, capacity=synthetic.capacity_from_factor(T, 2, 8),
                  router_bias="zipf1.2", overflow="next_best", seed=7)
    st, res, _ = run_staged_and_check(cfg)
    assert (res.status == 2).sum() > 0 and (res.status == 1).sum() > 0
    assert res.perm.counts.max() <= cfg.capacity


def test_fallback_small_expert_counts_and_both_slots():
    # E = 3: no 4th-ranked expert; a tight capacity drops both slots of many tokens
    run_staged_and_check(mid_cfg("fb_e3", T=400, n_experts=3, capacity=150, overflow="next_best",
                                 router_bias=None, seed=14))
    # E = 2: nothing to fall back to; the round changes nothing
    st, res, _ = run_staged_and_check(mid_cfg("fb_e2", T=300, n_experts=2, capacity=200,
                                              overflow="next_best", seed=15))
    assert np.all(to_np(st["next_ids"]) == -1) and not np.any(res.status == 2)
    # capacity 0: every offer finds no free slot
    st, res, _ = run_staged_and_check(mid_cfg("fb_cap0", T=200, n_experts=8, capacity=0,
                                              overflow="next_best", seed=16), check_h=False)
    assert np.all(to_np(st["drop_mask"]) == 1)


def test_dense_reduction_all_experts_equal():
    """All experts equal: the layer must equal one dense SwiGLU FFN (oracle, E=1 form)."""
    cfg = mid_cfg("dense", T=700, n_experts=8, seed=10)
    inp = synthetic.make_inputs(cfg)
    for name in ("w1", "w3", "w2"):
        w = getattr(inp, name)
        setattr(inp, name, w[:1].expand_as(w).contiguous())
    say("dense reduction (all experts equal)")
    di = runner.DeviceInputs.from_host(inp)
    buf = runner.forward(di)
    torch.cuda.synchronize()
    x = oracle.to_f64(inp.x)
    dense, _ = oracle.swiglu(x, oracle.to_f64(inp.w1[0]), oracle.to_f64(inp.w3[0]),
                             oracle.to_f64(inp.w2[0]))
    assert_close(to_np(buf.y.float()), dense, "bf16", "dense reduction")


@pytest.mark.parametrize("T,cap", [(900, 250), (60, 12)])
@pytest.mark.parametrize("overflow", ["drop", "next_best"])
def test_forward_matches_staged_bitwise_and_is_deterministic(overflow, T, cap):
    """T=900: the tiled path (256 x 320 tiles, token rows gathered through perm_src in moe_forward);
    T=60: weight streaming with a capacity (the gate/up gathers there too)."""
    cfg = mid_cfg("fwd_vs_staged", T=T, n_experts=8, capacity=cap, router_bias="zipf1.2", seed=11,
                  overflow=overflow)
    inp = synthetic.make_inputs(cfg)
    say(f"moe_forward vs the five staged calls ({overflow}); run twice")
    di = runner.DeviceInputs.from_host(inp)
    st = runner.staged(di)
    b1 = runner.forward(di)
    torch.cuda.synchronize()
    y1 = b1.y.clone()
    ids1, cnt1, drop1 = b1.topk_ids.clone(), b1.expert_counts.clone(), b1.drop_mask.clone()
    b2 = runner.forward(di, b1)
    torch.cuda.synchronize()
    assert torch.equal(y1, b2.y) and torch.equal(ids1, b2.topk_ids)
    assert torch.equal(cnt1, b2.expert_counts) and torch.equal(drop1, b2.drop_mask)
    assert torch.equal(st["y"], y1)
    assert torch.equal(st["topk_ids"], ids1) and torch.equal(st["drop_mask"], drop1)


@pytest.mark.parametrize("T,E,w,F", [(16, 8, "bf16", 448), (1, 8, "bf16", 448), (16, 16, "bf16", 384),
                                     (7, 2, "bf16", 448), (13, 3, "bf16", 384), (16, 8, "mxfp4", 768),
                                     (5, 16, "mxfp4", 768), (1, 2, "mxfp4", 768)])
def test_decode_forward_fused_router_matches_staged(T, E, w, F):
    """At decode shapes moe_forward groups tokens in the router's workgroup, the gate/up weight
    streamer reads x through perm_src and (bf16) one launch does the down projection and the
    combine (load rows of 128 B when F is not a multiple of 128, else 256 B); every output must
    equal the staged calls'."""
    cfg = mid_cfg(f"dec_fused_T{T}_E{E}_{w}", T=T, n_experts=E, w_dtype=w, seed=60 + T + E, d_ff=F)
    inp = synthetic.make_inputs(cfg)
    say(f"decode moe_forward (fused router + grouping) vs staged: T={T} E={E}")
    di = runner.DeviceInputs.from_host(inp)
    st = runner.staged(di)
    b = runner.forward(di)
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y) and torch.equal(st["topk_ids"], b.topk_ids)
    assert torch.equal(st["topk_weights"], b.topk_weights) and torch.equal(st["logits"], b.logits)
    assert torch.equal(st["expert_counts"], b.expert_counts)
    assert not b.drop_mask.any()
    base, res = adjusted_oracle(inp, to_np(b.topk_ids))
    assert_close(to_np(b.y.float()), res.y, "bf16", "decode y")


def test_decode_mxfp4_config_fused_forward_full():
    inp = cached_inputs("decode_mxfp4")
    say("MXFP4 decode config via moe_forward (fused router + grouping, gathered rows)")
    di = runner.DeviceInputs.from_host(inp)
    st = runner.staged(di)
    b = runner.forward(di)
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y) and torch.equal(st["expert_counts"], b.expert_counts)
    _, res = adjusted_oracle(inp, to_np(b.topk_ids))
    assert_close(to_np(b.y.float()), res.y, "bf16", "MXFP4 decode y (fused call)")


def test_decode_config_fused_forward_full():
    cfg = synthetic.CONFIGS["decode_bf16"]
    inp = cached_inputs("decode_bf16")
    say("decode config via moe_forward (the benchmarked call)")
    di = runner.DeviceInputs.from_host(inp)
    st = runner.staged(di)
    b = runner.forward(di)
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y) and torch.equal(st["expert_counts"], b.expert_counts)
    _, res = adjusted_oracle(inp, to_np(b.topk_ids))
    fro, mx = assert_close(to_np(b.y.float()), res.y, "bf16", "decode y (fused call)")
    say(f"  y rel_frob={fro:.3e} rel_max={mx:.3e}")


def test_combine_isolated():
    cfg = mid_cfg("combine", T=500, n_experts=8, capacity=120, seed=12)
    inp = synthetic.make_inputs(cfg)
    say("combine in isolation")
    st = runner.staged(runner.DeviceInputs.from_host(inp))
    torch.cuda.synchronize()
    yp = to_np(st["y_perm"])
    s2r = to_np(st["slot_to_row"]).reshape(-1, 2)
    g = to_np(st["topk_weights"]).astype(np.float64)
    ref = np.zeros((cfg.T, cfg.d_model))
    for s in range(2):
        ok = s2r[:, s] >= 0
        ref[ok] += g[ok, s, None] * yp[s2r[ok, s]]
    got = to_np(st["y"].float())
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


# ------------------------------------------------------ full-size configs ---

def test_decode_config_full():
    run_staged_and_check(synthetic.CONFIGS["decode_bf16"], inputs=cached_inputs("decode_bf16"))


def test_prefill_config_sampled():
    cfg = synthetic.CONFIGS["prefill_bf16"]
    inp = cached_inputs("prefill_bf16")
    base = oracle.forward(inp, tokens=[])
    toks = sample_tokens(base)
    run_staged_and_check(cfg, inputs=inp, tokens=toks, check_h=True)


def test_skewed_capacity_config_sampled():
    cfg = synthetic.CONFIGS["skewed_capacity_bf16"]
    inp = cached_inputs("skewed_capacity_bf16")
    base = oracle.forward(inp, tokens=[])
    toks = sample_tokens(base)
    st, res, _ = run_staged_and_check(cfg, inputs=inp, tokens=toks, check_h=True)
    counts = res.perm.counts
    assert counts.max() == cfg.capacity and (~res.keep).sum() > 1000


def test_skewed_fallback_config_sampled():
    cfg = synthetic.CONFIGS["skewed_fallback_bf16"]
    inp = cached_inputs("skewed_fallback_bf16")
    base = oracle.forward(inp, tokens=[])
    toks = sample_tokens(base)
    st, res, _ = run_staged_and_check(cfg, inputs=inp, tokens=toks, check_h=True)
    assert res.perm.counts.max() == cfg.capacity
    assert (res.status == 2).sum() > 500 and (res.status == 1).sum() > 0


def test_prefill_config_fused_forward_sampled():
    cfg = synthetic.CONFIGS["prefill_bf16"]
    inp = cached_inputs("prefill_bf16")
    say("prefill config via moe_forward (the benchmarked call)")
    di = runner.DeviceInputs.from_host(inp)
    buf = runner.forward(di)
    torch.cuda.synchronize()
    gpu_ids = to_np(buf.topk_ids)
    base = oracle.forward(inp, tokens=[])
    toks = sample_tokens(base, seed=3)
    _, res = adjusted_oracle(inp, gpu_ids, tokens=toks)
    check_routing(base, gpu_ids, to_np(buf.topk_weights), to_np(buf.logits), 3e-4)
    assert np.array_equal(to_np(buf.expert_counts), res.perm.counts)
    y = to_np(buf.y.float())[toks]
    fro, mx = assert_close(y, res.y[toks], "bf16", "prefill y")
    say(f"  y rel_frob={fro:.3e} rel_max={mx:.3e}")


# -------------------------------------------------------------- fp8 path ---

def fp8_mid_cfg(name, **kw):
    base = dict(name=name, T=700, d_model=512, d_ff=384, n_experts=8, act_dtype="bf16",
                w_dtype="fp8_e4m3", x_std=1.0, wg_std=512 ** -0.5, w13_std=0.05, w2_std=0.05,
                seed=21)
    base.update(kw)
    return synthetic.MoEConfig(**base)


def test_fp8_mid_staged():
    # 8 experts x ~175 rows: one ragged token tile per expert; F = 384 -> 3 channel tiles
    run_staged_and_check(fp8_mid_cfg("fp8_mid"))


def test_fp8_mid_many_tiles_and_capacity():
    run_staged_and_check(fp8_mid_cfg("fp8_e2", T=900, n_experts=2, d_ff=640, seed=22))
    run_staged_and_check(fp8_mid_cfg("fp8_cap", T=800, capacity=150, router_bias="zipf1.2", seed=23))


def test_fp8_small_batch():
    run_staged_and_check(fp8_mid_cfg("fp8_t16", T=16, seed=24))


# ------------------------------------------------------------ MXFP4 path ---

def mx4_mid_cfg(name, **kw):
    base = dict(name=name, T=40, d_model=512, d_ff=768, n_experts=8, act_dtype="bf16",
                w_dtype="mxfp4", x_std=1.0, wg_std=512 ** -0.5, w13_std=0.05, w2_std=0.05,
                seed=31)
    base.update(kw)
    return synthetic.MoEConfig(**base)


def test_mxfp4_mid_decode():
    # up to 40 rows per expert -> 3 token tiles of 16; 768 channels -> 24 groups of 32
    run_staged_and_check(mx4_mid_cfg("mx4_mid"))


def test_mxfp4_edge_cases():
    run_staged_and_check(mx4_mid_cfg("mx4_t1", T=1, seed=32))
    run_staged_and_check(mx4_mid_cfg("mx4_e2", T=64, n_experts=2, d_ff=512, seed=33))
    # capacity bounds the rows per expert (the decode path at a larger T), with the fallback
    cfg = mx4_mid_cfg("mx4_cap", T=300, capacity=48, overflow="next_best", router_bias="zipf1.2",
                      seed=34)
    st, res, _ = run_staged_and_check(cfg)
    assert res.perm.counts.max() <= 48 and (res.status == 2).sum() > 0


@pytest.mark.parametrize("T,seed,most_rows", [(2, 37, 1), (4, 36, 2), (6, 36, 3), (8, 36, 4),
                                              (10, 36, 5), (16, 37, 8), (24, 36, 9)])
def test_mxfp4_token_tile_heights(T, seed, most_rows):
    """The MXFP4 kernel packs 8, 4, 2 or 1 token operands per load instruction when the launch's
    fullest token tile has at most 2, 4, 8 or 16 rows; each band and its edges against the
    oracle (staged calls, token rows from x_perm) and the fused call (rows gathered from x)
    bitwise against the staged one."""
    cfg = mx4_mid_cfg(f"mx4_rows{most_rows}", T=T, seed=seed)
    st, res, inputs = run_staged_and_check(cfg)
    assert int(res.perm.counts.max()) == most_rows
    b = runner.forward(runner.DeviceInputs.from_host(inputs))
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y)


@pytest.mark.parametrize("d,F", [(2048, 2048), (4096, 2048)])
def test_mxfp4_two_stage_scale_loads_mid(d, F):
    """K a multiple of 2048: the GEMMs split K in four with an even number of 256-element stages
    per part, so scale bytes come two stages per load (the form the Mixtral shapes use): one
    two-stage cycle per output group at K = 2048, two at K = 4096 (gate/up of the second case).
    A Zipf-skewed router gives one expert 4 token tiles (the last ragged) and the others 1 or 2,
    with several output groups per workgroup; the fused call bitwise against the staged calls."""
    cfg = mx4_mid_cfg(f"mx4_q2_{d}_{F}", T=60, d_model=d, d_ff=F, wg_std=d ** -0.5,
                      router_bias="zipf1.2", seed=38)
    st, res, inputs = run_staged_and_check(cfg)
    assert int(res.perm.counts.max()) > 48
    b = runner.forward(runner.DeviceInputs.from_host(inputs))
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y)


def test_mxfp4_forward_matches_staged():
    cfg = mx4_mid_cfg("mx4_fwd", T=48, seed=35)
    inp = synthetic.make_inputs(cfg)
    say("MXFP4 moe_forward vs the staged calls")
    di = runner.DeviceInputs.from_host(inp)
    st = runner.staged(di)
    b = runner.forward(di)
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y)


def test_decode_mxfp4_config_full():
    run_staged_and_check(synthetic.CONFIGS["decode_mxfp4"], inputs=cached_inputs("decode_mxfp4"))


def test_longctx_fp8_config_sampled():
    """Gated against the oracle with the declared fp8 activation quantisation; also reports (not
    gated) the error against the dequantised-weight oracle without activation quantisation and
    against the unquantised weights the fp8 codes were drawn from ('How Mixtral 8x7B uses mixture
    of experts', 'Quantization asymmetry': the pages quantise the experts only)."""
    cfg = synthetic.CONFIGS["longctx_fp8"]
    inp = cached_inputs("longctx_fp8")
    base = oracle.forward(inp, tokens=[])
    toks = sample_tokens(base, n_random=16)
    st, res, _ = run_staged_and_check(cfg, inputs=inp, tokens=toks, check_h=True)
    gpu_ids = to_np(st["topk_ids"])
    override = {int(t): tuple(int(v) for v in gpu_ids[t]) for t in oracle.near_tie_tokens(base)}
    y = to_np(st["y"].float())[toks]
    deq = oracle.forward(inp, tokens=toks, override=override, fp8_act_quant=False)
    fro_deq, mx_deq = rel_errors(y, deq.y[toks])
    w1, w3, w2 = synthetic.unquantized_weights(cfg)
    raw = synthetic.MoEInputs(cfg.replace(w_dtype="f32"), inp.x, inp.w_gate, inp.router_bias,
                              w1, w3, w2)
    unq = oracle.forward(raw, tokens=toks, override=override)
    del w1, w3, w2, raw
    fro_unq, mx_unq = rel_errors(y, unq.y[toks])
    fro_act, _ = rel_errors(res.y[toks], deq.y[toks])
    say(f"  report only: vs dequantised weights without activation quantisation "
        f"rel_frob={fro_deq:.3e}; vs unquantised weights rel_frob={fro_unq:.3e}; "
        f"oracle's own activation-quantisation effect {fro_act:.3e}")
    record("longctx_fp8_report_only", y_rel_frob_vs_dequant_no_act_quant=fro_deq,
           y_rel_max_vs_dequant_no_act_quant=mx_deq, y_rel_frob_vs_unquantized=fro_unq,
           y_rel_max_vs_unquantized=mx_unq, oracle_act_quant_vs_no_act_quant=fro_act,
           tokens_checked=len(toks))


# ------------------------------------- general top-k, many experts, shared ---

def fg_cfg(name, **kw):
    base = dict(name=name, T=300, d_model=512, d_ff=256, n_experts=64, top_k=8, n_shared=1,
                act_dtype="bf16", w_dtype="bf16", x_std=1.0, wg_std=512 ** -0.5, w13_std=0.05,
                w2_std=0.05, seed=41)
    base.update(kw)
    return synthetic.MoEConfig(**base)


@pytest.mark.parametrize("E,k", [(256, 8), (100, 5), (64, 1), (17, 7), (8, 8), (129, 2), (33, 3)])
def test_route_general_topk(E, k):
    cfg = synthetic.MoEConfig(name=f"route_E{E}_k{k}", T=333, d_model=256, d_ff=64, n_experts=E,
                              top_k=k, wg_std=256 ** -0.5, seed=42)
    inp = synthetic.make_inputs(cfg, with_weights=False)
    say(f"route E={E} k={k} T=333 d=256 bf16 (+ ranks k+1, k+2)")
    shape = moe.shape_of(cfg)
    ids = torch.empty(cfg.T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, k, dtype=torch.float32, device="cuda")
    lg = torch.empty(cfg.T, E, dtype=torch.float32, device="cuda")
    nx = torch.empty(cfg.T, 2, dtype=torch.int32, device="cuda")
    moe.moe_route_topk(shape, inp.x.cuda(), inp.w_gate.cuda(), None, ids, w, lg, nx)
    torch.cuda.synchronize()
    res = oracle.forward(inp, tokens=[])
    check_routing(res, to_np(ids), to_np(w), to_np(lg), 3e-4)
    check_next(res, to_np(nx), to_np(ids))
    if k == 1:
        assert np.all(to_np(w) == 1.0)


@pytest.mark.parametrize("E,k", [(64, 5), (40, 1), (3, 3)])
def test_route_general_topk_fp32(E, k):
    cfg = synthetic.MoEConfig(name=f"route32_E{E}_k{k}", T=257, d_model=128, d_ff=64, n_experts=E,
                              top_k=k, act_dtype="f32", w_dtype="f32", wg_std=128 ** -0.5, seed=43)
    inp = synthetic.make_inputs(cfg, with_weights=False)
    say(f"route fp32 E={E} k={k} T=257 d=128")
    shape = moe.shape_of(cfg)
    ids = torch.empty(cfg.T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, k, dtype=torch.float32, device="cuda")
    lg = torch.empty(cfg.T, E, dtype=torch.float32, device="cuda")
    nx = torch.empty(cfg.T, 2, dtype=torch.int32, device="cuda")
    moe.moe_route_topk(shape, inp.x.cuda(), inp.w_gate.cuda(), None, ids, w, lg, nx)
    torch.cuda.synchronize()
    res = oracle.forward(inp, tokens=[])
    check_routing(res, to_np(ids), to_np(w), to_np(lg), 1e-5)
    check_next(res, to_np(nx), to_np(ids))


def test_route_general_topk_ties():
    """Duplicated router rows give exactly equal logits: the lower index always ranks first."""
    say("route E=256 k=8 with duplicated router rows (exact ties)")
    cfg = synthetic.MoEConfig(name="ties_k8", T=200, d_model=128, d_ff=64, n_experts=256, top_k=8,
                              wg_std=128 ** -0.5, seed=44)
    inp = synthetic.make_inputs(cfg, with_weights=False)
    wg = inp.w_gate.clone()
    for e in (40, 77, 200, 255):
        wg[e] = wg[13]
    inp.w_gate = wg
    ids = torch.empty(cfg.T, 8, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, 8, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(moe.shape_of(cfg), moe.MOE_CALL_ROUTE), dtype=torch.uint8,
                     device="cuda")
    moe.moe_route_topk(moe.shape_of(cfg), inp.x.cuda(), wg.cuda(), None, ids, w, None, None, ws)
    torch.cuda.synchronize()
    g = to_np(ids)
    res = oracle.forward(inp, tokens=[])
    assert np.array_equal(g, res.routing.ids)
    # wherever several of the tied experts are picked they appear consecutively, 13 first
    for row in g:
        tied = [e for e in row if e in (13, 40, 77, 200, 255)]
        assert tied == sorted(tied)
    # all rows equal: experts 0..7 with weights 1/8
    wg[:] = wg[0]
    moe.moe_route_topk(moe.shape_of(cfg), inp.x.cuda(), wg.cuda(), None, ids, w, None, None, ws)
    torch.cuda.synchronize()
    assert np.all(to_np(ids) == np.arange(8)) and np.all(to_np(w) == np.float32(0.125))


def test_finegrained_mid_prefill_path():
    # 64 experts x ~37 rows and a 300-row shared expert: the tiled bf16 path (> 64 rows)
    run_staged_and_check(fg_cfg("fg_mid"))


def test_finegrained_256_experts_prefill_path():
    # 257 expert groups in the tiled kernel's LDS offset table
    st, res, _ = run_staged_and_check(fg_cfg("fg_e256", T=500, d_model=256, n_experts=256, seed=45))
    assert to_np(st["expert_counts"])[256] == 500 and np.count_nonzero(res.perm.counts[:256]) > 200


def test_finegrained_decode_path():
    run_staged_and_check(fg_cfg("fg_decode", T=40, n_experts=128, top_k=6, seed=46))
    run_staged_and_check(fg_cfg("fg_t1", T=1, n_experts=256, seed=47))


@pytest.mark.parametrize("E,shared", [(31, 0), (32, 0), (31, 1)])
def test_decode_many_experts_threshold(E, shared):
    """Weight streaming with 32 or more expert groups maps its work differently (gate/up: a
    persistent grid over the token tiles that exist; down: a contiguous eighth of the groups per
    XCD): 31 groups take the grid over all groups, 32 or 31 + shared the other forms; top-8
    of about 32 experts at 64 tokens gives many experts two token tiles.  Staged calls against the
    oracle, the fused call bitwise against them."""
    cfg = fg_cfg(f"fg_many_E{E}_S{shared}", T=64, n_experts=E, top_k=8, n_shared=shared, seed=49)
    st, res, inputs = run_staged_and_check(cfg)
    assert int(res.perm.counts[:E].max()) > 16
    b = runner.forward(runner.DeviceInputs.from_host(inputs))
    torch.cuda.synchronize()
    assert torch.equal(st["y"], b.y)


def test_general_topk_without_shared_and_edge_k():
    run_staged_and_check(fg_cfg("fg_k1", T=200, n_experts=16, top_k=1, n_shared=0, seed=48))
    run_staged_and_check(fg_cfg("fg_kE", T=120, n_experts=8, top_k=8, n_shared=0, seed=49))
    run_staged_and_check(fg_cfg("fg_e2s", T=150, n_experts=2, top_k=2, n_shared=1, seed=50))


def test_general_topk_capacity_with_shared():
    T = 600
    # capacity below the mean load (600 * 3 / 16 = 112.5) so that every expert drops
    cfg = fg_cfg("fg_cap", T=T, n_experts=16, top_k=3, capacity=100, seed=51)
    st, res, _ = run_staged_and_check(cfg)
    assert (~res.keep).sum() > 0 and res.perm.counts[16] == T
    # capacity 0: only the shared expert contributes
    st, res, _ = run_staged_and_check(fg_cfg("fg_cap0", T=100, n_experts=16, top_k=4, capacity=0,
                                             seed=52))
    assert to_np(st["drop_mask"]).all() and to_np(st["expert_counts"]).tolist() == [0] * 16 + [100]


def test_general_topk_fp32_fp8_mxfp4():
    run_staged_and_check(fg_cfg("fg_f32", T=96, d_model=128, d_ff=128, n_experts=32, top_k=4,
                                act_dtype="f32", w_dtype="f32", wg_std=128 ** -0.5, seed=53))
    run_staged_and_check(fg_cfg("fg_fp8", T=300, n_experts=32, top_k=4, d_ff=384,
                                w_dtype="fp8_e4m3", seed=54))
    run_staged_and_check(fg_cfg("fg_mx4", T=16, n_experts=64, top_k=8, d_ff=512, w_dtype="mxfp4",
                                seed=55))


def test_general_topk_forward_matches_staged():
    """moe_forward equals the staged calls bitwise.  fg_fwd, fg_fwd_tall and fg_fwd_noshared take the
    256 x 320 tile path, where moe_forward's gate/up reads the token rows of x through perm_src instead
    of the permuted copy (ragged 320-row tiles, capacity, no shared expert, k = 2); fg_fwd_dec is the
    weight-streaming path."""
    for cfg in (fg_cfg("fg_fwd", T=260, n_experts=64, top_k=8, capacity=40, seed=56),
                fg_cfg("fg_fwd_tall", T=700, n_experts=16, top_k=4, seed=59),
                fg_cfg("fg_fwd_noshared", T=1000, n_experts=8, top_k=2, n_shared=0, seed=60),
                fg_cfg("fg_fwd_dec", T=24, n_experts=256, top_k=8, seed=57)):
        inp = synthetic.make_inputs(cfg)
        say(f"moe_forward vs staged: {cfg.name}")
        di = runner.DeviceInputs.from_host(inp)
        st = runner.staged(di)
        b = runner.forward(di)
        b2 = runner.forward(di)
        torch.cuda.synchronize()
        # no optional outputs: the router's logit buffer then lives in the workspace
        b3 = runner.forward(di, runner.alloc_forward(cfg, with_outputs=False))
        torch.cuda.synchronize()
        assert torch.equal(st["y"], b.y) and torch.equal(b.y, b2.y) and torch.equal(b.y, b3.y)
        assert torch.equal(st["topk_ids"], b.topk_ids) and torch.equal(st["expert_counts"], b.expert_counts)


def test_combine_general_topk_isolated():
    cfg = fg_cfg("fg_combine", T=200, n_experts=32, top_k=5, capacity=30, seed=58)
    inp = synthetic.make_inputs(cfg)
    say("combine in isolation (k=5, shared, capacity)")
    st = runner.staged(runner.DeviceInputs.from_host(inp))
    torch.cuda.synchronize()
    yp = to_np(st["y_perm"])
    s2r = to_np(st["slot_to_row"])
    g = to_np(st["topk_weights"]).astype(np.float64)
    T, k = cfg.T, cfg.top_k
    ref = np.zeros((T, cfg.d_model))
    for s_ in range(k):
        rr = s2r[:T * k].reshape(T, k)[:, s_]
        ok = rr >= 0
        ref[ok] += g[ok, s_, None] * yp[rr[ok]]
    ref += yp[s2r[T * k:]]
    got = to_np(st["y"].float())
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


def test_finegrained_decode_config_full():
    run_staged_and_check(synthetic.CONFIGS["finegrained_decode_bf16"],
                         inputs=cached_inputs("finegrained_decode_bf16"))


def test_finegrained_prefill_config_sampled():
    cfg = synthetic.CONFIGS["finegrained_prefill_bf16"]
    inp = cached_inputs("finegrained_prefill_bf16")
    base = oracle.forward(inp, tokens=[])
    # experts average 256 rows: the tiled GEMMs take 320-row token tiles here; the first and
    # last row of every tile of all 257 groups (about 290 tokens)
    toks = sample_tokens(base, n_random=12, tile_rows=320)
    run_staged_and_check(cfg, inputs=inp, tokens=toks, check_h=True, tile_rows=320)


@pytest.mark.parametrize("E,k,S,T,cap,overflow", [
    (8, 2, 0, 2049, 500, "next_best"),   # top-2 grouping: 3 chunks of 1024 tokens, the last holds 1
    (64, 2, 0, 3071, -1, "drop"),        # top-2, 64 experts, dropless, ragged last chunk
    (256, 8, 1, 2049, 60, "drop"),       # general grouping: many experts, capacity, shared expert
    (40, 3, 0, 1025, -1, "drop"),        # general grouping without a shared expert
])
def test_grouping_over_token_chunks(E, k, S, T, cap, overflow):
    """Grouping runs one workgroup per 1024-token chunk; each derives the experts' totals and its
    own start inside each expert from all assignments.  Counts, offsets, perm_src, slot_to_row and
    drop marks must equal the oracle's exactly across chunk boundaries and a ragged last chunk
    ("How Mixtral 8x7B uses mixture of experts", simplified forward pass: tokens batched by expert
    in a fixed order, results written back per token)."""
    cfg = synthetic.MoEConfig(name=f"chunks_E{E}_k{k}", T=T, d_model=64, d_ff=64, n_experts=E,
                              top_k=k, n_shared=S, capacity=cap, overflow=overflow,
                              act_dtype="bf16", w_dtype="bf16", x_std=1.0, wg_std=64 ** -0.5,
                              w13_std=0.05, w2_std=0.05, seed=3000 + E + k)
    st, res, _ = run_staged_and_check(cfg)
    if cap >= 0:
        assert (~res.keep).sum() > 0, "the capacity case must drop assignments"


def sweep_cfg(seed):
    """A seeded random shape of the whole layer: expert count, top-k, shared expert, batch (the
    weight-streaming and the tiled paths), widths, capacity and overflow, and weight dtype, drawn
    within what the library supports."""
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([2, 3, 8, 13, 40, 64, 65, 100, 256]))
    k = int(rng.integers(1, min(8, E) + 1))
    S = int(rng.integers(0, 2))
    w = str(rng.choice(["bf16", "bf16", "fp8_e4m3", "mxfp4"]))
    unit = {"bf16": 64, "fp8_e4m3": 128, "mxfp4": 256}[w]
    d = unit * int(rng.integers(1, 512 // unit + 1))
    F = unit * int(rng.integers(1, max(1, 448 // unit) + 1))
    T = int(rng.choice([1, 7, 33, 64] if w == "mxfp4" else [1, 7, 33, 64, 200, 700, 1100]))
    cap, overflow = -1, "drop"
    if rng.random() < 0.4:
        cap = int(rng.integers(0, 2 * T * k // E + 2))
        if k == 2 and rng.random() < 0.5:
            overflow = "next_best"
    return synthetic.MoEConfig(name=f"sweep{seed}", T=T, d_model=d, d_ff=F, n_experts=E, top_k=k,
                               n_shared=S, capacity=cap, overflow=overflow, act_dtype="bf16",
                               w_dtype=w, x_std=1.0, wg_std=d ** -0.5, w13_std=0.05, w2_std=0.05,
                               seed=2000 + seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_sweep(seed):
    cfg = sweep_cfg(seed)
    st, res, _ = run_staged_and_check(cfg)
    # the staged path and the fused call agree bit for bit on the same shape
    di = runner.DeviceInputs.from_host(synthetic.make_inputs(cfg))
    y = runner.forward(di).y
    torch.cuda.synchronize()
    assert torch.equal(y, st["y"]), "fused forward differs from the staged calls"
