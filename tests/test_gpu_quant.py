"""Quantiser parity on the GPU through the C ABI: K mean, Q/K INT8 codes and
scales, V E4M3 codes and scales must equal the oracle's bit for bit, at the
five workloads' shapes (full size) and at ragged edge shapes."""
import numpy as np
import pytest
import torch

import oracle
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


@pytest.mark.parametrize("fused", [False, True], ids=["qk+v", "qkv"])
def test_quantizers_unit_scale_ties(fused):
    # Blocks whose scale is exactly 1 (amax 127 for INT8, 448 for E4M3), so every quotient is the value itself:
    # exact ties k + 1/2 for the INT8 rounding, every E4M3 rounding boundary with both signs, both zeros, the
    # boundary to zero 2^-10 and values next to it.  K pairs token n with N - 1 - n negated, so k_mean is
    # exactly 0 and smoothing changes nothing.
    B, N, H, D = 1, 300, 2, 128
    g = torch.Generator().manual_seed(11)
    ties = torch.arange(-127, 127, dtype=torch.float64) + 0.5            # 254 exact ties
    q = ties[torch.randint(0, ties.numel(), (B, N, H, D), generator=g)]
    q[0, ::32, :, 0] = 127.0                                              # every 32-token Q block: scale 1
    half = ties[torch.randint(0, ties.numel(), (B, N // 2, H, D), generator=g)]
    half[0, ::32, :, 1] = 127.0
    k = torch.cat([half, -half.flip(1)], dim=1)                           # every 64-token K block: scale 1
    table = torch.from_numpy(oracle.e4m3_decode(np.arange(0x7F)))
    mids = (table[1:] + table[:-1]) / 2                                   # every rounding boundary
    vals = torch.cat([table, mids, -table, -mids, torch.tensor([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10),
                                                                  3 * 2.0 ** -11, 2.0 ** -11])])
    v = vals[torch.randint(0, vals.numel(), (B, N, H, D), generator=g)]
    v[0, 5, :, :] = 448.0                                                 # every channel: scale 1
    v[0, 6, 0, 3] = -0.0
    case = inputs.Case("ties", B, N, H, D, q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16))
    assert torch.equal(case.q.double(), q) and torch.equal(case.k.double(), k) and torch.equal(case.v.double(), v)
    ref = G.OracleRef(case)
    assert float(np.abs(ref.km).max()) == 0.0
    _check_bitexact(case, ref, fused)


def test_quantizers_repeatable():
    case = inputs.config("tiny")
    g = G.gpu_case(case)
    a, b = G.run_quant(g), G.run_quant(g)
    for name in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
