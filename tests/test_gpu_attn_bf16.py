"""The unquantised bf16 MFMA path on the GPU through the C ABI, against the
exact fp64 oracle: rel-L2 <= 5e-3 (P is rounded to bf16, 8 significant bits)."""
import numpy as np
import pytest
import torch

from quantized_softmax_attention_amd import inputs
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,spec", [("tiny", None), ("mid", (128, 64)), ("block24_bf16", (96, 64))])
def test_bf16_parity_workloads(name, spec):
    print("bf16 parity:", name, flush=True)
    ref = G.config_ref(name)
    case = ref.case
    out = G.run_attn_bf16(G.gpu_case(case))
    rows = (inputs.sample_rows(case.B, case.H, case.N, count=case.N) if spec is None
            else inputs.sample_rows(case.B, case.H, case.N, count=spec[0], tail=spec[1]))
    G.gate(G.out_rows(out, rows), ref.exact(rows), 5e-3, "%s bf16 path vs exact" % name)


@pytest.mark.parametrize("N", [1, 2, 33, 64, 65, 129, 257, 1000])
def test_bf16_parity_ragged(N):
    case = inputs.packed_case(2, N, 2, seed=200 + N, stress=(N % 2 == 1))
    ref = G.OracleRef(case)
    out = G.run_attn_bf16(G.gpu_case(case))
    rows = inputs.sample_rows(case.B, case.H, case.N, count=N)
    G.gate(G.out_rows(out, rows), ref.exact(rows), 5e-3, "bf16 ragged N=%d" % N)
    if N == 1:
        assert torch.equal(out.cpu()[:, 0], case.v[:, 0])


def test_bf16_layouts_byte_identical_and_deterministic():
    case = inputs.packed_case(1, 500, 3, seed=9)
    hnd = inputs.Case("hnd", 1, 500, 3, 128, *(t.transpose(1, 2).contiguous().transpose(1, 2)
                                               for t in (case.q, case.k, case.v)))
    a = G.run_attn_bf16(G.gpu_case(case))
    b = G.run_attn_bf16(G.gpu_case(hnd))
    c = G.run_attn_bf16(G.gpu_case(case))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert np.isfinite(a.float().cpu().numpy()).all()
