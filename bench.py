"""Benchmark of the sparse top-k MoE layer on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step is one pass of the whole layer over one batch of synthetic input:
router + top-k -> (capacity) -> permute -> gate/up GEMM + SwiGLU -> down GEMM
-> combine, enqueued through the C ABI on one stream.

The headline ``value`` is T / the median step time of the fused call
``moe_forward``: K steps, each bracketed by HIP events recorded on the stream
the layer runs on, between device synchronisations (p10 / p90 and the
wall-clock mean of the same K steps are reported beside it).  A second timed
pass issues the five boundary calls (the same kernels, in the same order) with
events between them: that gives each stage's time and algorithmic bytes, and
the dominant kernel's average launch time for ``roofline``.

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


def mfma_peak(cfg) -> float:
    """Dense matrix-core peak (TFLOP/s) of the type the expert GEMMs run in: fp8 e4m3 codes, fp32,
    or bf16 (bf16 experts, and MXFP4 experts, which are dequantised to bf16 in the kernel)."""
    if cfg.w_dtype == "fp8_e4m3":
        return PEAK_TFLOPS["fp8_e4m3"]
    return PEAK_TFLOPS["f32"] if cfg.act_dtype == "f32" else PEAK_TFLOPS["bf16"]


def roofline_of(cfg, nbytes: float, flops: float, kernel_ms: float) -> dict:
    """Roofline of one launch: the bound is the one whose minimum time is the longer, algorithmic
    bytes at the HBM peak or algorithmic flops at the matrix-core peak (decode batches are HBM-bound,
    large Mixtral batches MFMA-bound; many small experts with a narrow FFN can be HBM-bound at
    prefill because every expert's weights are read once for few rows).  The other bound's figure
    is kept beside it."""
    sec = kernel_ms * 1e-3
    hbm = {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    peak = mfma_peak(cfg)
    mfma = {"bound": "mfma", "achieved": round(flops / sec / 1e12, 1), "peak": peak, "unit": "TFLOP/s"}
    for r in (hbm, mfma):
        r["frac"] = round(r["achieved"] / r["peak"], 4)
    hbm_first = nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (peak * 1e12)
    main, other = (hbm, mfma) if hbm_first else (mfma, hbm)
    return {**main, "other_bound": other}


DEFAULTS = {"decode_bf16": (200, 20), "prefill_bf16": (20, 3), "skewed_capacity_bf16": (20, 3),
            "longctx_fp8": (10, 3), "tiny_fp32": (200, 20), "finegrained_decode_bf16": (100, 10),
            "finegrained_prefill_bf16": (10, 3)}
# Sources of the dominant (gate/up) kernel of each weight dtype: a committed
# traffic measurement counts only while the hash of these files is unchanged.
_CSRC = "sparse_mixture_experts_topk_amd/csrc/"
KERNEL_SOURCES = {
    "bf16": (_CSRC + "gemm_bf16.hip", _CSRC + "gemm_bf16_decode.hip", _CSRC + "lds_stream.hpp",
             _CSRC + "persistent_tiles.hpp", _CSRC + "device_common.hpp", _CSRC + "lane_ops.hpp"),
    "fp8_e4m3": (_CSRC + "gemm_fp8.hip", _CSRC + "lds_stream.hpp", _CSRC + "persistent_tiles.hpp",
                 _CSRC + "device_common.hpp"),
    "mxfp4": (_CSRC + "gemm_mxfp4_decode.hip", _CSRC + "lds_stream.hpp", _CSRC + "device_common.hpp",
              _CSRC + "lane_ops.hpp"),
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


def stage_work(cfg, counts):
    """Algorithmic bytes (and flops) of each boundary call of one step (counts: rows per expert
    group, the shared expert's included)."""
    T, d, F, E, k, S = cfg.T, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k, cfg.n_shared
    s_act = 4 if cfg.act_dtype == "f32" else 2
    fp8 = cfg.w_dtype == "fp8_e4m3"
    s_perm = 1 if fp8 else s_act                 # x_perm / h element bytes
    n_kept = int(sum(counts))
    touched = int(sum(1 for c in counts if c > 0))
    wb = {"bf16": 2, "f32": 4, "fp8_e4m3": 1, "mxfp4": 0.5 + 1 / 32}[cfg.w_dtype]
    gu_bytes, gu_flops, _, _ = gate_up_work(cfg, counts)
    scale_x = n_kept * (d // 32) if fp8 else 0
    scale_h = n_kept * (F // 32) if fp8 else 0
    return {
        # x and W_g read, ids and weights written
        "route": (T * d * s_act + E * d * s_act + T * k * 8, 2.0 * T * d * E),
        # ids read, kept rows of x read, x_perm (+ scales) and the index arrays written
        "permute": (T * k * 4 + n_kept * d * s_act + n_kept * d * s_perm + scale_x
                    + 2 * T * (k + S) * 4, 0.0),
        "gate_up": (gu_bytes + scale_x + scale_h, gu_flops),
        # w2 of touched experts, h (+ scales) read, y_perm written
        "down": (int(touched * d * F * wb) + n_kept * F * s_perm + scale_h + n_kept * d * 4,
                 2.0 * n_kept * d * F),
        # kept rows of y_perm read, y written, slot map and weights read
        "combine": (n_kept * d * 4 + T * d * s_act + T * (k + S) * 4 + T * k * 4, 0.0),
    }


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


def _counter_values(csv_path: str, counter: str, kernel_re: str):
    """Per-dispatch values of one counter from a rocprofv3 ``--pmc`` CSV, for dispatches whose
    kernel name matches ``kernel_re`` (values summed over a dispatch's rows)."""
    import csv
    import re
    per, names = {}, set()
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or not re.search(kernel_re, row.get("Kernel_Name", "")):
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
            m = re.search(r"(grouped_gemm_\w+)<", row["Kernel_Name"])
            names.add(m.group(1) if m else row["Kernel_Name"][:80])
    return list(per.values()), sorted(names)


def write_traffic(cfg, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_mib):
    """HBM bytes per gate/up launch from two rocprofv3 counter runs of this workload (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads for the plain
    device copy of ``cal_mib`` MiB (``--calibrate-copy-mib``).  Writes
    profiles/gate_up_<workload>_traffic.json stamped with the current kernel-source hash."""
    gate_up = r"grouped_gemm_\w+<true"          # the dual (gate/up) instance of each GEMM family
    fetch, kernels = _counter_values(fetch_csv, "FETCH_SIZE", gate_up)
    write, _ = _counter_values(write_csv, "WRITE_SIZE", gate_up)
    if not fetch or not write:
        raise SystemExit("no gate/up dispatches in the counter files")
    cal_kib = (cal_mib << 20) / 1024.0

    def factor(path, counter):
        v, _ = _counter_values(path, counter, r".")
        big = sorted(x for x in v if x >= 0.25 * max(v))      # the copy dispatches (the fill reads nothing)
        return cal_kib / big[len(big) // 2]

    ff, wf = factor(cal_fetch_csv, "FETCH_SIZE"), factor(cal_write_csv, "WRITE_SIZE")
    fk, wk = sum(fetch) / len(fetch), sum(write) / len(write)
    out = {"workload": cfg.name, "kernel": ", ".join(kernels), "fetch_size_kib": round(fk, 1), "write_size_kib": round(wk, 1),
           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
           "hbm_bytes_per_launch": int(round((fk * ff + wk * wf) * 1024)),
           "launches": len(fetch), "kernel_source_sha": kernel_source_sha(cfg)}
    p = os.path.join(ROOT, "profiles", f"gate_up_{cfg.name}_traffic.json")
    with open(p, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(cfg, inputs, budget_tokens, min_seconds=10.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
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
    return {"value": reps * len(toks) / dt, "unit": "tokens/s", "cores": cores,
            "blas_threads": cores if threadpool_limits is not None else None, "kind": "oracle",
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
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="no GPU work: turn the rocprofv3 counter CSVs of this workload and of the "
                         "copy calibration into profiles/gate_up_<workload>_traffic.json")
    ap.add_argument("--calibration-mib", type=int, default=1024,
                    help="size of the calibration copy behind --write-traffic")
    a = ap.parse_args()

    if a.write_traffic:
        from sparse_mixture_experts_topk_amd import synthetic
        write_traffic(synthetic.CONFIGS[a.config], *a.write_traffic, a.calibration_mib)
        return

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
    fallback = cfg.capacity >= 0 and cfg.overflow == "next_best"
    stages = ("route", "permute", "gate_up", "down", "combine")

    def staged_step(d, ev):
        ev[0].record(stream)
        moe.moe_route_topk(shape, d.x, d.w_gate, d.router_bias, st["topk_ids"],
                           st["topk_weights"], None, st["next_ids"] if fallback else None,
                           st["route_ws"], stream)
        ev[1].record(stream)
        moe.moe_permute(shape, st["topk_ids"], st["topk_weights"],
                        st["next_ids"] if fallback else None, d.x, st["expert_counts"],
                        st["expert_offsets"], st["perm_src"], st["slot_to_row"],
                        st["drop_mask"] if cfg.capacity >= 0 else None,
                        st["x_perm"], st["x_perm_scale"], None, stream)
        ev[2].record(stream)
        moe.moe_expert_gemm_gate_up(shape, st["x_perm"], st["x_perm_scale"], st["expert_offsets"],
                                    d.w1, d.w3, d.w1_scale, d.w3_scale, st["h"], st["h_scale"],
                                    None, stream)
        ev[3].record(stream)
        moe.moe_expert_gemm_down(shape, st["h"], st["h_scale"], st["expert_offsets"], d.w2,
                                 d.w2_scale, st["y_perm"], st["down_ws"], stream)
        ev[4].record(stream)
        moe.moe_combine(shape, st["y_perm"], st["slot_to_row"], st["topk_weights"], st["y"], stream)
        ev[5].record(stream)

    def new_events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    # ---- headline: the fused call, one event pair per step on the layer's stream
    buf = runner.alloc_forward(cfg, with_outputs=False)
    for i in range(warmup):
        runner.forward(copies[i % len(copies)], buf, stream)
    fev = [new_events(2) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fev[i][0].record(stream)
        runner.forward(copies[i % len(copies)], buf, stream)
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fused = sorted(e[0].elapsed_time(e[1]) for e in fev)

    def pct(v, q):
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]

    med_ms = pct(fused, 0.5)

    # ---- the five boundary calls, events between the stages
    for i in range(warmup):
        staged_step(copies[i % len(copies)], new_events(6))
    sev = [new_events(6) for _ in range(steps)]
    torch.cuda.synchronize()
    s0 = time.perf_counter()
    for i in range(steps):
        staged_step(copies[i % len(copies)], sev[i])
    torch.cuda.synchronize()
    staged_wall_ms = (time.perf_counter() - s0) * 1e3 / steps
    stage_ms = {name: sum(e[j].elapsed_time(e[j + 1]) for e in sev) / steps
                for j, name in enumerate(stages)}
    kernel_ms = stage_ms["gate_up"]

    counts = st["expert_counts"].cpu().tolist()
    nbytes, flops, touched, n_kept = gate_up_work(cfg, counts)
    sha = kernel_source_sha(cfg)
    traffic = read_traffic(cfg.name, sha)
    roof = roofline_of(cfg, nbytes, flops, kernel_ms)
    roof["traffic"] = traffic
    roof.update({"kernel": "moe_expert_gemm_gate_up", "kernel_avg_ms": round(kernel_ms, 4),
                 "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                 "experts_touched": touched, "rows": n_kept, "kernel_source_sha": sha})

    work = stage_work(cfg, counts)
    stage_out = {}
    for name in stages:
        b, f = work[name]
        ms_ = stage_ms[name]
        stage_out[name] = {"ms": round(ms_, 4), "bytes": int(b), "GB/s": round(b / (ms_ * 1e-3) / 1e9, 1)}
        if f:
            stage_out[name]["TFLOP/s"] = round(f / (ms_ * 1e-3) / 1e12, 1)
    layer_flops = 6.0 * cfg.d_model * cfg.d_ff * n_kept + 2.0 * cfg.T * cfg.d_model * cfg.n_experts
    layer_bytes = sum(b for b, _ in work.values())
    out = {
        "metric": METRIC, "value": round(cfg.T / (med_ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(med_ms, 4),
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
        "timing": {"call": "moe_forward", "stat": "median of per-step HIP events",
                   "p10_ms": round(pct(fused, 0.1), 4), "p50_ms": round(med_ms, 4),
                   "p90_ms": round(pct(fused, 0.9), 4),
                   "wall_mean_ms": round(elapsed * 1e3 / steps, 4),
                   "staged_wall_mean_ms": round(staged_wall_ms, 4)},
        "layer_tflops": round(layer_flops / (med_ms * 1e-3) / 1e12, 2),
        "layer_hbm_gbs": round(layer_bytes / (med_ms * 1e-3) / 1e9, 1),
        "stages": stage_out,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, a.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
