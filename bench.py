"""Benchmark of the sparse top-k MoE layer on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step is one pass of the whole layer over one batch of synthetic input:
router + top-k -> (capacity) -> permute -> gate/up GEMM + SwiGLU -> down GEMM
-> combine, enqueued through the C ABI on one stream.  The timed step issues
the five boundary calls (the same kernels, in the same order, that the fused
moe_forward enqueues) so that HIP events can bracket the dominant kernel
inside the timed region; moe_forward itself is timed right after over the
same number of steps and reported as ``fused_ms_per_step``.

Default workload: the Mixtral-shape decode batch (16 tokens, bf16).  The
decode step alternates between two copies of the expert weights so that the
256 MB last-level cache cannot serve a step from the previous one.

Prints ONE JSON line.  Only ``--gpus 1`` is supported (one GPU per box).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % roofline (HBM GB/s decode, MFMA TFLOP/s prefill)"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "fp8_e4m3": 5000.0, "f32": 157.3}   # dense matrix-core peaks
DEFAULTS = {"decode_bf16": (200, 20), "prefill_bf16": (20, 3), "skewed_capacity_bf16": (20, 3),
            "longctx_fp8": (10, 3), "tiny_fp32": (200, 20), "finegrained_decode_bf16": (100, 10),
            "finegrained_prefill_bf16": (10, 3)}
# Sources of the dominant (gate/up) kernel of each weight dtype: a committed
# traffic measurement counts only while the hash of these files is unchanged.
_CSRC = "sparse_mixture_experts_topk_amd/csrc/"
KERNEL_SOURCES = {
    "bf16": (_CSRC + "gemm_bf16.hip", _CSRC + "gemm_bf16_decode.hip", _CSRC + "lds_stream.hpp",
             _CSRC + "persistent_tiles.hpp", _CSRC + "device_common.hpp"),
    "fp8_e4m3": (_CSRC + "gemm_fp8.hip", _CSRC + "lds_stream.hpp", _CSRC + "persistent_tiles.hpp",
                 _CSRC + "device_common.hpp"),
    "mxfp4": (_CSRC + "gemm_mxfp4_decode.hip", _CSRC + "lds_stream.hpp", _CSRC + "device_common.hpp"),
    "f32": (_CSRC + "gemm_f32.hip", _CSRC + "device_common.hpp"),
}


def kernel_source_sha(cfg) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[cfg.w_dtype]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def is_decode(cfg) -> bool:
    # the library's weight-streaming path: no expert can receive more than 64 rows
    # (a shared expert receives all T)
    cap = cfg.T if cfg.capacity < 0 or cfg.n_shared else min(cfg.T, cfg.capacity)
    return cap <= 64


def gate_up_work(cfg, counts):
    """Algorithmic bytes and flops of one gate/up launch (counts: rows per expert group,
    the shared expert's included)."""
    d, F = cfg.d_model, cfg.d_ff
    n_kept = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    # weight bytes per element: MXFP4 = half a byte of code + one scale byte per 32
    wb = {"bf16": 2, "f32": 4, "fp8_e4m3": 1, "mxfp4": 0.5 + 1 / 32}[cfg.w_dtype]
    ab = 1 if cfg.w_dtype == "fp8_e4m3" else (4 if cfg.act_dtype == "f32" else 2)
    weight_bytes = int(touched * 2 * F * d * wb)             # w1 + w3 rows of touched experts
    act_bytes = n_kept * d * ab + n_kept * F * ab            # x_perm read + h written
    flops = 4.0 * n_kept * d * F                             # two [n, d] x [d, F] products
    return weight_bytes + act_bytes, flops, touched, n_kept


def read_traffic(cfg_name: str, sha: str):
    """HBM bytes per gate/up launch from committed rocprofv3 counter runs, if current."""
    p = os.path.join(ROOT, "profiles", f"gate_up_{cfg_name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None          # the kernel changed since the counters were taken
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inputs, budget_tokens, min_seconds=10.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = min(len(os.sched_getaffinity(0)), 16)
    T = cfg.T
    toks = np.arange(T) if T <= budget_tokens else np.linspace(0, T - 1, budget_tokens).astype(int)
    reps = 0
    t0 = time.perf_counter()
    # repeat the sample until at least min_seconds of CPU work have been timed
    while reps == 0 or time.perf_counter() - t0 < min_seconds:
        if threadpool_limits is not None:
            with threadpool_limits(limits=cores):
                oracle.forward(inputs, tokens=toks)
        else:
            oracle.forward(inputs, tokens=toks)
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": reps * len(toks) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(toks)} of {T} tokens through the fp64 oracle (routing, grouping and "
                      f"capacity over all {T} tokens; expert FFN + combine for the sample), "
                      f"repeated {reps}x, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="decode_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the MoE layer runs on one GPU only: its kernels are "
                                   "single-device; --gpus N > 1 is not supported"}))
        sys.exit(2)

    import torch
    from sparse_mixture_experts_topk_amd import runner, synthetic
    import sparse_mixture_experts_topk_amd as moe

    if a.calibrate_copy_mib:
        n = a.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 5}))
        return

    cfg = synthetic.CONFIGS[a.config]
    steps, warmup = DEFAULTS.get(a.config, (20, 3))
    steps = a.steps if a.steps is not None else steps
    warmup = a.warmup if a.warmup is not None else warmup

    inputs = synthetic.make_inputs(cfg)
    di = runner.DeviceInputs.from_host(inputs)
    copies = [di]
    if is_decode(cfg):
        copies.append(di.with_weights(di.w1.clone(), di.w3.clone(), di.w2.clone()))
    shape = moe.shape_of(cfg)
    st = runner.staged(di)          # allocates every intermediate once (and warms the path)
    stream = torch.cuda.current_stream()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

    def step(i, timed):
        d = copies[i % len(copies)]
        fallback = cfg.capacity >= 0 and cfg.overflow == "next_best"
        moe.moe_route_topk(shape, d.x, d.w_gate, d.router_bias, st["topk_ids"],
                           st["topk_weights"], None, st["next_ids"] if fallback else None,
                           st["route_ws"], stream)
        moe.moe_permute(shape, st["topk_ids"], st["topk_weights"],
                        st["next_ids"] if fallback else None, d.x, st["expert_counts"],
                        st["expert_offsets"], st["perm_src"], st["slot_to_row"],
                        st["drop_mask"] if cfg.capacity >= 0 else None,
                        st["x_perm"], st["x_perm_scale"], None, stream)
        if timed:
            ev0[i].record(stream)
        moe.moe_expert_gemm_gate_up(shape, st["x_perm"], st["x_perm_scale"], st["expert_offsets"],
                                    d.w1, d.w3, d.w1_scale, d.w3_scale, st["h"], st["h_scale"],
                                    None, stream)
        if timed:
            ev1[i].record(stream)
        moe.moe_expert_gemm_down(shape, st["h"], st["h_scale"], st["expert_offsets"], d.w2,
                                 d.w2_scale, st["y_perm"], st["down_ws"], stream)
        moe.moe_combine(shape, st["y_perm"], st["slot_to_row"], st["topk_weights"], st["y"], stream)

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = sum(ev0[i].elapsed_time(ev1[i]) for i in range(steps)) / steps

    # the fused call, same alternation
    bufs = [runner.alloc_forward(cfg, with_outputs=False) for _ in range(1)]
    for i in range(warmup):
        runner.forward(copies[i % len(copies)], bufs[0], stream)
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    for i in range(steps):
        runner.forward(copies[i % len(copies)], bufs[0], stream)
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - f0) * 1e3 / steps

    counts = st["expert_counts"].cpu().tolist()
    nbytes, flops, touched, n_kept = gate_up_work(cfg, counts)
    decode = is_decode(cfg)
    sha = kernel_source_sha(cfg)
    traffic = read_traffic(cfg.name, sha)
    if decode:
        achieved = nbytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        peak = PEAK_TFLOPS[cfg.w_dtype if cfg.w_dtype != "f32" else "f32"]
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic}
    roof.update({"kernel": "moe_expert_gemm_gate_up", "kernel_avg_ms": round(kernel_ms, 4),
                 "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                 "experts_touched": touched, "rows": n_kept, "kernel_source_sha": sha})

    ms = elapsed * 1e3 / steps
    layer_flops = 6.0 * cfg.d_model * cfg.d_ff * n_kept + 2.0 * cfg.T * cfg.d_model * cfg.n_experts
    out = {
        "metric": METRIC, "value": round(cfg.T * steps / elapsed, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8_e4m3", "f32": "f32", "mxfp4": "mxfp4"}[cfg.w_dtype],
        "data": ("synthetic (seeded, fine-grained: 256 routed experts top-8 + 1 shared; random "
                 "weights)" if cfg.n_shared or cfg.n_experts > 8 else
                 "synthetic (seeded, Mixtral-shaped; random weights)"),
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "n_shared": cfg.n_shared,
                   "capacity": None if cfg.capacity < 0 else cfg.capacity,
                   "overflow": cfg.overflow if cfg.capacity >= 0 else None,
                   "act_dtype": cfg.act_dtype, "w_dtype": cfg.w_dtype,
                   "weight_copies_alternated": len(copies)},
        "fused_ms_per_step": round(fused_ms, 4),
        "layer_tflops": round(layer_flops / (ms * 1e-3) / 1e12, 2),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, a.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
