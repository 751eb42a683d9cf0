"""Quantiser parity on the GPU through the C ABI: K mean, Q/K INT8 codes and
scales, V E4M3 codes and scales must equal the oracle's bit for bit, at the
five workloads' shapes (full size) and at ragged edge shapes."""
import numpy as np
import pytest
import torch

from quantized_softmax_attention_amd import inputs, sage
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _check_bitexact(case: inputs.Case, ref: G.OracleRef, fused: bool = False):
    G.check_quant_bitexact(G.run_quant(G.gpu_case(case), fused), ref)


def test_kappa_matches_binding():
    assert np.array_equal(G.kappa(), sage.v_token_order().numpy())
    assert sorted(G.kappa()) == list(range(64))


@pytest.mark.parametrize("fused", [False, True], ids=["qk+v", "qkv"])
@pytest.mark.parametrize("name", ["tiny", "mid", "block24", "stress"])
def test_quantizers_bitexact_workloads(name, fused):
    print("quantizer parity:", name, "fused" if fused else "", flush=True)
    ref = G.config_ref(name)
    _check_bitexact(ref.case, ref, fused)


@pytest.mark.parametrize("fused", [False, True], ids=["qk+v", "qkv"])
@pytest.mark.parametrize("N", [1, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257, 4095])
def test_quantizers_bitexact_ragged(N, fused):
    print("quantizer parity ragged N =", N, "fused" if fused else "", flush=True)
    case = inputs.packed_case(2, N, 3, seed=N, stress=(N % 2 == 1))
    _check_bitexact(case, G.OracleRef(case), fused)


def test_quantizers_hnd_and_packed_layouts_agree():
    case = inputs.packed_case(1, 300, 4, seed=7)
    hnd = inputs.Case("hnd", 1, 300, 4, 128, *(t.transpose(1, 2).contiguous().transpose(1, 2)
                                               for t in (case.q, case.k, case.v)))
    a, b = G.run_quant(G.gpu_case(case)), G.run_quant(G.gpu_case(hnd))
    for name in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_quantizers_special_values():
    # zero blocks, a constant K channel, a zero V channel, ties, tiny and large values
    B, N, H, D = 1, 200, 2, 128
    x = torch.zeros(B, N, H, D)
    x[0, :, 0, 5] = 3.0                                   # constant K channel -> code 0
    x[0, 40:, 1] = torch.linspace(-1000, 1000, (N - 40) * D).reshape(N - 40, D)
    x[0, 7, 1, 9] = 2.0 ** -120                           # tiny
    q = x.clone(); q[0, 64:96] = 0                        # an all-zero Q block
    v = x.clone(); v[0, :, 0, 11] = 0                     # an all-zero V channel
    v[0, 3, 0, 12] = -(2.0 ** -30)
    case = inputs.Case("special", B, N, H, D, q.to(torch.bfloat16), x.to(torch.bfloat16), v.to(torch.bfloat16))
    _check_bitexact(case, G.OracleRef(case))


def test_quantizers_repeatable():
    case = inputs.config("tiny")
    g = G.gpu_case(case)
    a, b = G.run_quant(g), G.run_quant(g)
    for name in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
