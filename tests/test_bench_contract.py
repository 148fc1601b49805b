"""bench.py's contract that needs no GPU: one GPU only, and the workload table it times."""
import json
import os
import subprocess
import sys

import bench
from sparse_mixture_experts_topk_amd import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_every_benched_workload_is_a_config_with_kernel_sources():
    for name in bench.DEFAULTS:
        cfg = synthetic.CONFIGS[name]
        assert len(bench.kernel_source_sha(cfg)) == 16
    # the headline line is the 16-token decode batch
    assert bench.DEFAULTS["decode_bf16"][0] >= 100


def test_gate_up_work_counts_touched_experts_and_rows():
    cfg = synthetic.CONFIGS["decode_bf16"]
    nbytes, flops, touched, rows = bench.gate_up_work(cfg, [4, 0, 4, 4, 4, 4, 4, 8])
    assert touched == 7 and rows == 32
    assert nbytes == 7 * 2 * 14336 * 4096 * 2 + 32 * 4096 * 2 + 32 * 14336 * 2
    assert flops == 4.0 * 32 * 4096 * 14336
    mx = synthetic.CONFIGS["decode_mxfp4"]
    nb4, _, _, _ = bench.gate_up_work(mx, [4] * 8)
    assert nb4 == int(8 * 2 * 14336 * 4096 * (0.5 + 1 / 32)) + 32 * 4096 * 2 + 32 * 14336 * 2


def test_roofline_names_the_binding_bound():
    # decode: bytes bind
    cfg = synthetic.CONFIGS["decode_bf16"]
    nb, fl, _, _ = bench.gate_up_work(cfg, [4] * 8)
    r = bench.roofline_of(cfg, nb, fl, 0.25)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["other_bound"]["bound"] == "mfma"
    assert r["frac"] == round(nb / 0.25e-3 / 1e9 / 8000.0, 4)
    # Mixtral prefill: 2048 rows per expert, flops bind
    cfg = synthetic.CONFIGS["prefill_bf16"]
    nb, fl, _, _ = bench.gate_up_work(cfg, [2048] * 8)
    r = bench.roofline_of(cfg, nb, fl, 3.0)
    assert r["bound"] == "mfma" and r["peak"] == 2500.0
    assert r["achieved"] == round(fl / 3e-3 / 1e12, 1)
    # 256 experts with d_ff 2048 at 256 rows each (+ a shared expert): every expert's weights
    # are read once for few rows, so bytes bind at prefill too
    cfg = synthetic.CONFIGS["finegrained_prefill_bf16"]
    nb, fl, _, _ = bench.gate_up_work(cfg, [256] * 256)
    assert nb / 8e12 > fl / 2.5e15
    assert bench.roofline_of(cfg, nb, fl, 2.7)["bound"] == "hbm"
    # fp8 experts are priced at the fp8 peak, MXFP4 experts at bf16 (dequantised in the kernel)
    assert bench.mfma_peak(synthetic.CONFIGS["longctx_fp8"]) == 5000.0
    assert bench.mfma_peak(synthetic.CONFIGS["decode_mxfp4"]) == 2500.0
    assert bench.mfma_peak(synthetic.CONFIGS["tiny_fp32"]) == 157.3


def test_decode_detection_follows_the_rows_per_expert_bound():
    assert bench.is_decode(synthetic.CONFIGS["decode_bf16"])
    assert not bench.is_decode(synthetic.CONFIGS["prefill_bf16"])
    assert bench.is_decode(synthetic.CONFIGS["finegrained_decode_bf16"])
    # a shared expert takes every token, so a capacity does not bound its rows
    cfg = synthetic.CONFIGS["finegrained_prefill_bf16"].replace(capacity=32)
    assert not bench.is_decode(cfg)


def _pmc_csv(path, counter, rows):
    """A rocprofv3 --pmc CSV with the columns bench.py reads: (dispatch, kernel name, value)."""
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for disp, name, val in rows:
            w.writerow([disp, name, counter, val])


def test_write_traffic_scales_gate_up_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    gu = "void moe::(anonymous namespace)::grouped_gemm_bf16_prefill<true, 64, 2, 2, 4, 6, 2, false>(...)"
    dn = "void moe::(anonymous namespace)::grouped_gemm_bf16_prefill<false, 64, 2, 4, 2, 3, 4, true>(...)"
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(1, gu, 1000.0), (2, dn, 9e9), (3, gu, 3000.0)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(1, gu, 10.0), (2, dn, 9e9), (3, gu, 30.0)])
    # 1 MiB copy: FETCH reads half of it (factor 2), WRITE all of it; the fill (dispatch 1) reads nothing
    _pmc_csv(tmp_path / "cf.csv", "FETCH_SIZE", [(1, "fill", 0.0), (2, "copy", 512.0), (3, "copy", 512.0)])
    _pmc_csv(tmp_path / "cw.csv", "WRITE_SIZE", [(1, "fill", 1024.0), (2, "copy", 1024.0), (3, "copy", 1024.0)])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    cfg = synthetic.CONFIGS["prefill_bf16"]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda c: "0123456789abcdef")
    bench.write_traffic(cfg, str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                        str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1)
    out = json.load(open(tmp_path / "profiles" / "gate_up_prefill_bf16_traffic.json"))
    assert out["kernel"] == "grouped_gemm_bf16_prefill" and out["launches"] == 2
    assert out["fetch_factor"] == 2.0 and out["write_factor"] == 1.0
    assert out["hbm_bytes_per_launch"] == (2000.0 * 2 + 20.0) * 1024
    assert bench.read_traffic("prefill_bf16", "0123456789abcdef") == out["hbm_bytes_per_launch"]
    assert bench.read_traffic("prefill_bf16", "fedcba9876543210") is None   # stale after a change
