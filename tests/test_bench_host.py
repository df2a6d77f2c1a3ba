"""CPU checks of bench.py's host side: the one-GPU contract, the flop counts the metric uses, and
the CPU-baseline leg (the oracle timed on a row sample) on a tiny workload."""
import dataclasses
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from head_attention_streaming_amd import synthetic  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _brute_visible(Lq, Lk, causal, window):
    """Count visible keys per query row by testing every (query, key) pair."""
    shift = Lk - Lq
    out = []
    for i in range(Lq):
        p = i + shift
        n = 0
        for j in range(Lk):
            ok = True
            if causal and j > p:
                ok = False
            if window is not None:
                left, right = window
                if left >= 0 and j < p - left:
                    ok = False
                if right >= 0 and j > p + right:
                    ok = False
            n += ok
        out.append(n)
    return np.array(out)


@pytest.mark.parametrize("Lq,Lk,causal,window", [
    (37, 37, False, None), (20, 50, True, None), (50, 50, False, (7, 0)), (30, 45, False, (5, 3)),
    (40, 40, False, (-1, 2)), (25, 60, False, (100, 100)),
])
def test_visible_keys_match_brute_force(Lq, Lk, causal, window):
    w = dataclasses.replace(synthetic.WORKLOADS["mha_257_bf16"], Lq=Lq, Lk=Lk, causal=causal, attn_window=window)
    assert np.array_equal(bench.visible_keys(w, np.arange(Lq)), _brute_visible(Lq, Lk, causal, window))


def test_metric_flops_follow_the_formula():
    w = synthetic.WORKLOADS["mha_20480_bf16"]
    assert bench.workload_flops(w) == 4.0 * 1 * 56 * 20480 * 20480 * 128
    win = synthetic.WORKLOADS["window_4096_w256_f16"]
    vis = bench.visible_keys(win, np.arange(win.Lq))
    assert bench.workload_flops(win) == 4.0 * win.B * win.Hq * win.d * vis.sum()
    assert vis.max() == 257 and vis.min() == 1
    assert abs(bench.PEAK_MFMA_FP8_F16 - 1.0 / (0.5 / 5033.2 + 0.5 / 2516.6)) < 1e-9


def test_cpu_baseline_reports_the_oracle_on_a_row_sample():
    w = dataclasses.replace(synthetic.WORKLOADS["mha_257_bf16"], Lq=64, Lk=80, Hq=2, Hkv=2)
    q, k, v = synthetic.attention_inputs(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.d, w.dtype, seed=1)
    r = bench.cpu_baseline(w, (q, k, v), target_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "query rows" in r["sample"]
    # the whole problem at the sample's rate, labelled as an extrapolation
    sampled = int(r["sample"].split(" of ")[0])
    total = w.B * w.Lq * w.Hq
    assert r["full_problem_seconds_extrapolated"] >= r["seconds"] * 0.99 * min(1.0, total / sampled) - 0.05
    if sampled == total:
        assert abs(r["full_problem_seconds_extrapolated"] - r["seconds"]) <= 0.1
