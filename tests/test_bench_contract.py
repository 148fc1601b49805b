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


def test_decode_detection_follows_the_rows_per_expert_bound():
    assert bench.is_decode(synthetic.CONFIGS["decode_bf16"])
    assert not bench.is_decode(synthetic.CONFIGS["prefill_bf16"])
    assert bench.is_decode(synthetic.CONFIGS["finegrained_decode_bf16"])
    # a shared expert takes every token, so a capacity does not bound its rows
    cfg = synthetic.CONFIGS["finegrained_prefill_bf16"].replace(capacity=32)
    assert not bench.is_decode(cfg)
