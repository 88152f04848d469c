"""Host-side checks of bench.py: the one-GPU contract and the algorithmic bytes and flops it
divides by (no GPU needed)."""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_algorithmic_bytes_at_768p():
    # Q, K, V read once and O written once, bf16: (B H F n) tokens x (d + dv) x 2 bytes per
    # stage, plus the text tokens' K and V for the statistics -- 8.921 GB for the step
    w = W.by_name("768p_bf16")
    a = bench.algorithmic(w)
    video = 1 * 24 * 90 * 4032
    assert a["stats"]["bytes"] == (video + 24 * 256) * (128 + 128) * 2
    assert a["readout"]["bytes"] == video * (128 * 2 + 128 * 2)
    assert a["scan"]["bytes"] == 0
    assert abs((a["stats"]["bytes"] + a["readout"]["bytes"]) / 1e9 - 8.921) < 0.001


def test_fp8_inputs_halve_the_bytes_read():
    w = W.by_name("768p_fp8")
    a = bench.algorithmic(w)
    video = 24 * 90 * 4032
    assert a["stats"]["bytes"] == (video + 24 * 256) * 256 * 1
    assert a["readout"]["bytes"] == video * (128 * 1 + 128 * 2)  # FP8 Q in, bf16 O out


def test_gated_readout_adds_weights_and_the_two_projections():
    w = W.by_name("768p_bf16")
    plain, gated = bench.algorithmic(w), bench.algorithmic(w, gated=True)
    video = 24 * 90 * 4032
    assert gated["readout"]["bytes"] - plain["readout"]["bytes"] == 24 * (2 * 128 * 128 * 2 + 128 * 4)
    assert gated["readout"]["flops"] - plain["readout"]["flops"] == video * 2 * 2 * 128 * 128
