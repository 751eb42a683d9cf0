"""INT8 Q K^T with an unquantised bf16 P.V (sage_attn_fwd_int8qk) on the GPU
through the C ABI, against the oracle.

Gates: within rel-L2 1e-3 of the step-by-step oracle of the same precision split
(oracle.attn_int8qk, output bf16-rounded on both sides as for the quantised
kernel), and within 2e-2 of the exact fp64 result on the Gaussian workloads --
the accuracy target the fully quantised method cannot reach.  On the stress
workload (x10 outlier channels in Q and K) the INT8 scores alone cost more than
that, so there the bound is the oracle's own distance to the exact result
plus 1e-3."""
import hashlib

import numpy as np
import pytest
import torch

from quantized_softmax_attention_amd import inputs, sage
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

ROWS = {"tiny": None, "mid": (128, 64), "block24": (96, 64), "stress": (64, 64)}


def _rows(case, spec):
    if spec is None:
        return inputs.sample_rows(case.B, case.H, case.N, count=case.N)
    return inputs.sample_rows(case.B, case.H, case.N, count=spec[0], tail=spec[1])


def test_int8qk_parity_long_sequence():
    # 4096 full 64-key tiles and a 37-key tail on two heads
    N = 4096 * 64 + 37
    print("int8qk parity long sequence N =", N, flush=True)
    case = inputs.packed_case(1, N, 2, seed=901)
    ref = G.OracleRef(case)
    out, _ = G.run_attn_int8qk(G.gpu_case(case))
    rows = _rows(case, (48, 16))
    got = G.out_rows(out, rows)
    G.gate(got, G.bf16_round(ref.int8qk(rows)), 1e-3, "N=%d vs int8qk oracle" % N)
    assert G.rel_l2(got, ref.exact(rows)) <= 2e-2


@pytest.mark.parametrize("name", ["tiny", "mid", "block24", "stress"])
def test_int8qk_parity_workloads(name):
    print("int8qk parity:", name, flush=True)
    ref = G.config_ref(name)
    case = ref.case
    out, _ = G.run_attn_int8qk(G.gpu_case(case))
    rows = _rows(case, ROWS[name])
    got = G.out_rows(out, rows)
    meth = ref.int8qk(rows)
    exact = ref.exact(rows)
    G.gate(got, G.bf16_round(meth), 1e-3, "%s vs int8qk oracle" % name)
    e_x = G.rel_l2(got, exact)
    floor = G.rel_l2(meth, exact)
    print("%s: rel-L2 vs exact %.3e, oracle floor %.3e" % (name, e_x, floor), flush=True)
    if name == "stress":
        assert e_x <= floor + 1e-3
    else:
        assert e_x <= 2e-2


@pytest.mark.parametrize("N", [1, 2, 32, 33, 63, 64, 65, 129, 257, 1000, 4095])
def test_int8qk_parity_ragged(N):
    print("int8qk parity ragged N =", N, flush=True)
    case = inputs.packed_case(2, N, 2, seed=300 + N, stress=(N % 2 == 0))
    ref = G.OracleRef(case)
    out, _ = G.run_attn_int8qk(G.gpu_case(case))
    rows = _rows(case, (256, 64) if N > 1000 else None)
    got = G.out_rows(out, rows)
    G.gate(got, G.bf16_round(ref.int8qk(rows)), 1e-3, "int8qk ragged N=%d" % N)
    if N == 1:   # one key: the output is v_0 itself
        assert torch.equal(out.cpu()[:, 0], case.v[:, 0])


def test_int8qk_layouts_byte_identical_and_deterministic():
    case = inputs.packed_case(1, 777, 3, seed=23)
    hnd = inputs.Case("hnd", 1, 777, 3, 128, *(t.transpose(1, 2).contiguous().transpose(1, 2)
                                               for t in (case.q, case.k, case.v)))
    a, buf = G.run_attn_int8qk(G.gpu_case(case))
    b, _ = G.run_attn_int8qk(G.gpu_case(hnd))
    c, _ = G.run_attn_int8qk(G.gpu_case(case), buf)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ha = hashlib.sha256(a.cpu().view(torch.int16).numpy().tobytes()).hexdigest()
    hc = hashlib.sha256(c.cpu().view(torch.int16).numpy().tobytes()).hexdigest()
    assert ha == hc


def test_int8qk_rows_beyond_n_untouched():
    case = G.gpu_case(inputs.packed_case(1, 70, 2, seed=4))
    buf = G.run_quant(case)
    big = torch.full((1, 128, 2 * 128), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, :70].view(1, 70, 2, 128)
    sage.sage_attn_fwd_int8qk(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, case.v, view, G.SM)
    torch.cuda.synchronize()
    assert torch.all(big[:, 70:] == 7.0)
    assert np.isfinite(big[:, :70].float().cpu().numpy()).all()
