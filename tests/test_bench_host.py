"""bench.py's host-side contract without a GPU: more than one GPU is refused
with a message before anything touches a device, and the algorithmic byte and
FLOP counts the roofline uses follow from the block-24 shapes."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_counts():
    B, N, H, D = 1, 37810, 56, 128
    assert bench.attn_flops() == 4 * B * N * N * D * H == 40989379379200
    npad = 37888
    # Q, K, V codes read once (int8 / e4m3, padded), bf16 output written once
    assert bench.attn_bytes() == 3 * H * npad * D + 2 * N * H * D == 1356787712
    q = bench.quant_bytes()
    e = N * H * D
    assert q["qk_quantize"] == 6 * e + 2 * H * npad * D
    assert q["v_quantize"] == 4 * e + H * npad * D
    r = bench.rope_bytes()
    assert r["norm_rope"] == 8 * e + N * D * 4
    assert r["qkv_rope"] == q["qk_quantize"] + q["v_quantize"] + 2 * N * D * 4


def test_stats_percentiles():
    s = bench.stats_ms([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s["min"] == 1.0 and s["max"] == 5.0 and s["p50"] == 3.0 and s["mean"] == 3.0 and s["count"] == 5
    assert s["p90"] == 5.0 and s["p99"] == 5.0
