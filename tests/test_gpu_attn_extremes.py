"""The quantised forward at the edges of its inputs, on the GPU through the C ABI,
each checked against the method oracle and against what the mathematics fixes
for it:

* a long sequence: 131072 keys in one head (2048 tiles of running maximum and
  rescaling, sums of 131072 terms);
* K constant along the tokens: smoothing subtracts exactly that constant, so the
  K codes and scales are zero, every score is zero, and the output is the plain
  mean of the dequantised V;
* one key that dominates every query (score ~180 above the rest): every other
  weight underflows, so the output is that key's dequantised V row.

The unquantised bf16 path and the INT8-QK / bf16-PV path get the same cases
(against the exact oracle and their own oracle, with V itself in the closed
forms)."""
import numpy as np
import pytest
import torch

from oracle import e4m3_decode
from quantized_softmax_attention_amd import inputs
from tests import gpu_common as G

PATHS = ["i8f8", "int8qk", "bf16"]


def _run(path, case):
    """Output of one path on case, and the buffers when it quantises."""
    g = G.gpu_case(case)
    if path == "i8f8":
        return G.run_attn(g)
    if path == "int8qk":
        return G.run_attn_int8qk(g)
    return G.run_attn_bf16(g), None


def _gate(path, ref, out, rows):
    """rel-L2 of the sampled rows against the path's own oracle, and its bound (every row is also held to
    the per-row bound of gpu_common.gate)."""
    got = G.out_rows(out, rows)
    if path == "i8f8":
        want, bound = G.bf16_round(ref.method(rows)), 1e-3
    elif path == "int8qk":
        want, bound = G.bf16_round(ref.int8qk(rows)), 1e-3
    else:
        want, bound = ref.exact(rows), 5e-3
    return G.gate(got, want, bound, path), bound


def _v_used(path, ref):
    """The V values a path multiplies by, [B, H, N, D]: dequantised E4M3 codes or the bf16 V."""
    if path == "i8f8":
        return _dequantised_v(ref)
    v = ref.case.v.float().numpy()                                   # [B, N, H, D]
    return v.transpose(0, 2, 1, 3).astype(np.float64)

pytestmark = pytest.mark.gpu


def _dequantised_v(ref):
    vc, vs = ref.vq                                                  # [B, H, N, D] codes, [B, H, D]
    return e4m3_decode(vc).reshape(vc.shape) * vs[:, :, None, :]


def test_long_sequence_parity():
    N = 131072
    print("long sequence N =", N, flush=True)
    case = inputs.packed_case(1, N, 1, seed=77)
    ref = G.OracleRef(case)
    out, buf = G.run_attn(G.gpu_case(case))
    G.check_quant_bitexact(buf, ref)
    rows = inputs.sample_rows(1, 1, N, count=96, tail=32)
    got = G.out_rows(out, rows)
    meth, exact = ref.method(rows), ref.exact(rows)
    e_m, floor = G.gate(got, G.bf16_round(meth), 1e-3, "N=%d vs method" % N), G.rel_l2(meth, exact)
    print("N=%d: method floor %.3e" % (N, floor), flush=True)
    assert G.rel_l2(got, exact) <= floor + 1e-3


@pytest.mark.parametrize("path", ["int8qk", "bf16"])
def test_long_sequence_other_paths(path):
    N = 131072
    print("long sequence", path, "N =", N, flush=True)
    case = inputs.packed_case(1, N, 1, seed=77)
    ref = G.OracleRef(case)
    out, _ = _run(path, case)
    rows = inputs.sample_rows(1, 1, N, count=96, tail=32)
    e, bound = _gate(path, ref, out, rows)
    print("%s N=%d: rel-L2 vs its oracle %.3e" % (path, N, e), flush=True)
    assert e <= bound


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("N", [1, 64, 333])
def test_k_constant_along_tokens(N, path):
    print("constant K, N =", N, flush=True)
    B, H = 1, 2
    base = inputs.packed_case(B, N, H, seed=78)
    k = base.k[:, :1].expand(B, N, H, 128).contiguous()             # every token's K row = token 0's
    case = inputs.Case("kconst", B, N, H, 128, base.q.contiguous(), k, base.v.contiguous())
    ref = G.OracleRef(case)
    out, buf = _run(path, case)
    if buf is not None:
        G.check_quant_bitexact(buf, ref)
        assert not buf.k_codes.any() and not buf.k_scale.any()
    got = out.float().cpu().numpy().transpose(0, 2, 1, 3)            # [B, H, N, D]
    mean = _v_used(path, ref).mean(axis=2, keepdims=True)            # [B, H, 1, D]
    # bf16 output rounding plus the fp32 accumulation of N terms in the MFMA (the
    # absolute part covers channels whose mean nearly cancels)
    assert np.allclose(got, mean, rtol=2 ** -7, atol=1e-3 * np.abs(mean).max())
    e, bound = _gate(path, ref, out, inputs.sample_rows(B, H, N, count=N))
    assert e <= bound


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("star", [100, 332])
def test_one_dominant_key(star, path):
    print("dominant key at", star, flush=True)
    B, N, H, D = 1, 333, 1, 128
    g = torch.Generator().manual_seed(79)
    u = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0)    # a +-1 direction, |u|^2 = 128
    q = (4.0 * u).expand(B, N, H, D).contiguous()
    k = 0.5 * torch.randn(B, N, H, D, generator=g)
    k[0, star, 0] = 4.0 * u                                           # score (16 * 128) / sqrt(128) = 181
    v = torch.randn(B, N, H, D, generator=g)
    case = inputs.Case("dominant", B, N, H, D, *(t.to(torch.bfloat16) for t in (q, k, v)))
    ref = G.OracleRef(case)
    out, buf = _run(path, case)
    if buf is not None:
        G.check_quant_bitexact(buf, ref)
    got = out.float().cpu().numpy()[0, :, 0]                         # [N, D]
    vstar = _v_used(path, ref)[0, 0, star]                           # [D]
    assert np.allclose(got, np.broadcast_to(vstar, got.shape), rtol=2 ** -8, atol=0)
    e, bound = _gate(path, ref, out, inputs.sample_rows(B, H, N, count=N))
    assert e <= bound
