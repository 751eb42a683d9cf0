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
    # every 128-query block of every head stages its head's padded K and V codes into LDS once
    assert bench.kv_restream_bytes() == 296 * 2 * npad * D * H == 160_776_060_928
    r = bench.rope_bytes()
    assert r["norm_rope"] == 8 * e + N * D * 4
    assert r["qkv_rope"] == q["qk_quantize"] + q["v_quantize"] + 2 * N * D * 4


def test_stats_percentiles():
    s = bench.stats_ms([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s["min"] == 1.0 and s["max"] == 5.0 and s["p50"] == 3.0 and s["mean"] == 3.0 and s["count"] == 5
    assert s["p90"] == 5.0 and s["p99"] == 5.0


def _tiny_oracle():
    import oracle
    from quantized_softmax_attention_amd import inputs
    from tests.helpers import oracle_view

    case = inputs.config("tiny")
    q, k, v = (oracle_view(t) for t in (case.q, case.k, case.v))
    qc, qs = oracle.quant_q(q, 32)
    kc, ks = oracle.quant_k(k, oracle.kmean(k), 64)
    vc, vs = oracle.quant_v(v)
    return case, (qc, qs, kc, ks, vc, vs)


def test_parity_vs_method_is_exact_on_the_method_and_local():
    """The bench's parity check: zero when the 'timed output' is the oracle's own bf16 result at the
    sampled rows, and one wrong element in one row trips the per-row gate while the whole-set figure
    would not."""
    import math

    import numpy as np
    import oracle
    import torch
    from quantized_softmax_attention_amd import inputs

    case, (qc, qs, kc, ks, vc, vs) = _tiny_oracle()
    B, N, H, D = case.B, case.N, case.H, case.D
    rows = inputs.sample_rows(B, H, N, count=64, tail=16)
    meth = oracle.attn_method(qc, qs, kc, ks, vc, vs, 1.0 / math.sqrt(D), rows)
    full = oracle.attn_method(qc, qs, kc, ks, vc, vs, 1.0 / math.sqrt(D))          # [B, H, N, D]
    out = torch.from_numpy(full.transpose(0, 2, 1, 3).reshape(B, N, H * D)).float().to(torch.bfloat16)
    p = bench.parity_vs_method(out, rows, meth)
    assert p["rel_l2_vs_method"] == 0.0 and p["max_row_rel_l2"] == 0.0 and p["rows"] == B * H * 64
    assert p["max_row_err_vs_typical_row"] == 0.0
    r = int(rows[0, 1, 5])
    bad = out.clone()
    bad[0, r, 1 * D + 17] = -bad[0, r, 1 * D + 17] * 3 + 1
    p = bench.parity_vs_method(bad, rows, meth)
    assert p["max_row_err_vs_typical_row"] > 3 * bench.PARITY_ROW_GATE
    assert p["rel_l2_vs_method"] < p["max_row_err_vs_typical_row"]
    assert p["worst_rows"][0]["row"] == r and p["worst_rows"][0]["h"] == 1


def test_rescale_fraction_counts_moved_maxima():
    """The share of tiles where a 32-query wave rescales: every tile after the first for a one-tile-per-step
    workload whose scores grow monotonically with the key index, none when they shrink."""
    import numpy as np

    N, H = 256, 1
    kc = np.zeros((1, H, N, 128), np.int8)
    qc = np.zeros((1, H, N, 128), np.int8)
    qc[..., 0] = 1
    kc[0, 0, :, 0] = (np.arange(N) // 2).astype(np.int8)        # scores rise with the key index
    qs = np.ones((1, H, N // 32), np.float32)
    ks = np.ones((1, H, N // 64), np.float32)
    assert bench.rescale_fraction((qc, qs, kc, ks), N, H, waves_per_head=2, head_step=1) == 1.0
    kc[0, 0, :, 0] = (127 - np.arange(N) // 2).astype(np.int8)  # falling: the first tile holds the maximum
    assert bench.rescale_fraction((qc, qs, kc, ks), N, H, waves_per_head=2, head_step=1) == 0.0
    _, (qc, qs, kc, ks, _, _) = _tiny_oracle()
    f = bench.rescale_fraction((qc, qs, kc, ks), 256, 2, waves_per_head=4, head_step=1)
    assert 0.0 < f <= 1.0


def test_side_parity_passes_the_oracles_own_rows_and_catches_a_wrong_row():
    # the bench's check of the bf16 and INT8-QK paths, fed the oracle's own results (as a correct kernel's
    # would be, up to rounding) passes; one row replaced by another row's values fails its per-row bound
    import numpy as np
    import torch

    import oracle
    from quantized_softmax_attention_amd import inputs
    from tests.helpers import oracle_view

    case = inputs.packed_case(1, 300, 2, seed=77)
    q, k, v = (oracle_view(t) for t in (case.q, case.k, case.v))
    km = oracle.kmean(k)
    (qc, qs), (kc, ks) = oracle.quant_q(q, 32), oracle.quant_k(k, km, 64)
    rows = inputs.sample_rows(1, 2, 300, count=40, tail=8)
    sm = 1.0 / np.sqrt(128.0)
    exact = oracle.attn_exact(q, k, v, sm, rows)
    meth = torch.from_numpy(oracle.attn_int8qk(qc, qs, kc, ks, v, sm, rows)).float().to(torch.bfloat16).double()
    got16 = torch.from_numpy(exact).float().to(torch.bfloat16).double().numpy()
    res = bench.side_parity(case, (qc, qs, kc, ks), rows, got16, meth.numpy())
    assert res["bf16_path"]["ok"] and res["int8qk_path"]["ok"]
    assert res["bf16_path"]["rel_l2"] < 5e-3 and res["int8qk_path"]["rel_l2"] == 0.0
    bad = meth.numpy().copy()
    bad[0, 1, 3] = bad[0, 1, 4]
    res = bench.side_parity(case, (qc, qs, kc, ks), rows, got16, bad)
    assert not res["int8qk_path"]["ok"] and res["int8qk_path"]["max_row_err_vs_typical_row"] > 3e-2


def test_out_rows_gathers_token_major_rows():
    import numpy as np
    import torch

    B, N, H, D = 2, 5, 3, 128
    out = torch.arange(B * N * H * D, dtype=torch.float32).reshape(B, N, H * D).to(torch.bfloat16)
    rows = np.array([[[4, 0], [1, 1], [2, 3]], [[0, 0], [3, 2], [4, 4]]], dtype=np.int32)   # [B, H, R]
    got = bench.out_rows(out, rows)
    for b in range(B):
        for h in range(H):
            for r in range(2):
                n = rows[b, h, r]
                assert np.array_equal(got[b, h, r], out[b, n, h * D:(h + 1) * D].double().numpy())
