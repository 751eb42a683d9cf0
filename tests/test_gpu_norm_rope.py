"""RMSNorm + RoPE of Q and K on the GPU through the C ABI.

* sage_qk_norm_rope (in place): the transformed Q and K equal the oracle's
  evaluation (the exact sum of squares rounded once to fp32, then fixed fp32
  steps) bit for bit, on HND and packed strided views, ragged N, the block-24
  workload and rows built to take the kernel's exact integer path; nothing
  outside the two views changes.
* sage_quantize_qkv_rope (fused): every code, scale and k_mean equals the
  oracle's quantisers applied to the oracle's transformed Q and K, bit for bit,
  and equals sage_qk_norm_rope followed by sage_quantize_qkv on the GPU; the
  inputs are left untouched.  The attention over the fused codes matches the
  method oracle on the transformed inputs."""
import hashlib

import numpy as np
import pytest
import torch

import oracle
from quantized_softmax_attention_amd import inputs, sage
from tests import gpu_common as G
from tests.helpers import oracle_view

pytestmark = pytest.mark.gpu


def _bits_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _oracle_transformed(case: inputs.Case, nr: inputs.NormRope) -> inputs.Case:
    """The case with Q and K replaced by the oracle's transform (contiguous
    [B, N, H, D]); V as it was."""
    tq = oracle.norm_rope(oracle_view(case.q), nr.gamma_q.numpy(), nr.rope.numpy(), nr.eps)
    tk = oracle.norm_rope(oracle_view(case.k), nr.gamma_k.numpy(), nr.rope.numpy(), nr.eps)
    return inputs.Case(case.name + "+rope", case.B, case.N, case.H, case.D, _bits_tensor(tq), _bits_tensor(tk),
                       case.v)


def _storage_hash(t: torch.Tensor) -> str:
    return hashlib.sha256(t.cpu().view(torch.int16).numpy().tobytes()).hexdigest()


CASES = {
    "tiny": lambda: inputs.config("tiny"),
    "packed_ragged": lambda: inputs.packed_case(2, 300, 3, seed=31, stress=True),
    "one_token": lambda: inputs.packed_case(1, 1, 1, seed=32),
    "n65": lambda: inputs.packed_case(1, 65, 4, seed=33),
    "block24": lambda: inputs.config("block24"),
    "stress": lambda: inputs.config("stress"),        # B=2, x10 outlier channels, Student-t V
    "long": lambda: inputs.packed_case(1, 4096 * 64 + 37, 2, seed=34),   # 4096 full blocks + a ragged tail
    "many_heads": lambda: inputs.packed_case(3, 65, 700, seed=35),       # large (b, h) indices, ragged N
}


@pytest.mark.parametrize("name", list(CASES))
def test_norm_rope_in_place_bitexact(name):
    print("norm_rope in place:", name, flush=True)
    case = CASES[name]()
    nr = inputs.norm_rope_params(case.N, seed=3)
    want = _oracle_transformed(case, nr)
    g = G.gpu_case(case)
    before_v = _storage_hash(g.v.contiguous())
    packed_before = None if g.packed is None else g.packed.clone()
    sage.sage_qk_norm_rope(g.q, g.k, nr.to("cuda").gamma_q, nr.to("cuda").gamma_k, nr.rope.cuda(), nr.eps)
    torch.cuda.synchronize()
    assert torch.equal(g.q.cpu().view(torch.int16), want.q.view(torch.int16)), "Q"
    assert torch.equal(g.k.cpu().view(torch.int16), want.k.view(torch.int16)), "K"
    assert _storage_hash(g.v.contiguous()) == before_v, "V changed"
    if packed_before is not None:
        HD = case.H * case.D
        assert torch.equal(g.packed[:, :, 2 * HD:], packed_before[:, :, 2 * HD:])


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_qkv_rope_bitexact_vs_oracle(name):
    print("quantize_qkv_rope vs oracle:", name, flush=True)
    case = CASES[name]()
    nr = inputs.norm_rope_params(case.N, seed=4)
    ref = G.OracleRef(_oracle_transformed(case, nr))
    g = G.gpu_case(case)
    src_before = _storage_hash(g.packed if g.packed is not None else torch.cat([g.q, g.k, g.v]))
    buf = sage.Buffers(case.B, case.N, case.H)
    for t in (buf.q_codes, buf.k_codes, buf.v_codes):
        t.view(torch.uint8).fill_(0x5A)
    for t in (buf.q_scale, buf.k_scale, buf.k_mean, buf.v_scale):
        t.fill_(float("nan"))
    sage.quantize_qkv_rope(g.q, g.k, g.v, nr.to("cuda"), buf)
    torch.cuda.synchronize()
    G.check_quant_bitexact(buf, ref)
    assert _storage_hash(g.packed if g.packed is not None else torch.cat([g.q, g.k, g.v])) == src_before


@pytest.mark.parametrize("N", [1, 33, 64, 129, 1000])
def test_fused_equals_in_place_then_quantize(N):
    print("fused vs unfused N =", N, flush=True)
    case = inputs.packed_case(2, N, 3, seed=40 + N, stress=(N % 2 == 1))
    nr = inputs.norm_rope_params(N, seed=5).to("cuda")
    a = G.gpu_case(case)
    fused = sage.Buffers(case.B, N, case.H)
    sage.quantize_qkv_rope(a.q, a.k, a.v, nr, fused)
    b = G.gpu_case(case)
    sage.sage_qk_norm_rope(b.q, b.k, nr.gamma_q, nr.gamma_k, nr.rope, nr.eps)
    unfused = sage.Buffers(case.B, N, case.H)
    sage.quantize_qkv(b.q, b.k, b.v, unfused)
    torch.cuda.synchronize()
    for f in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale"):
        assert torch.equal(getattr(fused, f), getattr(unfused, f)), f


def test_attention_over_fused_codes_matches_method():
    case = inputs.config("tiny")
    nr = inputs.norm_rope_params(case.N, seed=6)
    ref = G.OracleRef(_oracle_transformed(case, nr))
    g = G.gpu_case(case)
    buf = sage.Buffers(case.B, case.N, case.H)
    sage.quantize_qkv_rope(g.q, g.k, g.v, nr.to("cuda"), buf)
    out, _ = G.run_attn(g, buf)
    rows = inputs.sample_rows(case.B, case.H, case.N, count=case.N)
    got = G.out_rows(out, rows)
    G.gate(got, G.bf16_round(ref.method(rows)), 1e-3, "attention after fused norm+rope quantisation vs method")


def test_norm_rope_extreme_rows_bitexact():
    # rows spanning the bf16 range, rows of zeros, single large or tiny entries,
    # results in the bf16 subnormal range (tiny rows with a large eps): the
    # in-place result and the fused codes stay bit-exact against the oracle
    B, N, H, D = 1, 96, 3, 128
    rng = np.random.default_rng(17)
    x = rng.standard_normal((B, N, 3 * H, D))
    scale = np.exp2(rng.integers(-100, 100, size=(B, N, 3 * H, 1)).astype(np.float64))
    x = x * scale
    x[0, 5] = 0.0                                    # a zero token (all heads of Q, K, V)
    x[0, 6, :, 1:] = 0.0                             # one nonzero channel per row
    x[0, 7] = 2.0 ** -133                            # bf16 subnormal inputs
    x[0, 8, :, :64] = 3.0e38 / 128                   # large values
    packed = torch.from_numpy(x.reshape(B, N, 3 * H * D)).float().to(torch.bfloat16)
    HD = H * D
    q, k, v = (packed[:, :, i * HD:(i + 1) * HD].unflatten(2, (H, D)) for i in range(3))
    case = inputs.Case("extreme", B, N, H, D, q, k, v, packed)
    for eps in (1e-6, 1e3):                          # a large eps pushes tiny rows into subnormals
        nr = inputs.norm_rope_params(N, seed=9, eps=eps)
        want = _oracle_transformed(case, nr)
        g = G.gpu_case(case)
        sage.sage_qk_norm_rope(g.q, g.k, nr.to("cuda").gamma_q, nr.to("cuda").gamma_k, nr.rope.cuda(), nr.eps)
        torch.cuda.synchronize()
        assert torch.equal(g.q.cpu().view(torch.int16), want.q.view(torch.int16)), ("Q", eps)
        assert torch.equal(g.k.cpu().view(torch.int16), want.k.view(torch.int16)), ("K", eps)
        ref = G.OracleRef(want)
        g2 = G.gpu_case(case)
        buf = sage.Buffers(B, N, H)
        sage.quantize_qkv_rope(g2.q, g2.k, g2.v, nr.to("cuda"), buf)
        torch.cuda.synchronize()
        G.check_quant_bitexact(buf, ref)


def test_norm_rope_exact_sum_rows_bitexact():
    """Rows whose sum of squares an fp64 sum cannot round correctly (ties broken by a square far below the
    fp64 ulp), rows spanning the whole bf16 exponent range (the exact integer path of the kernel), rows
    whose squares overflow fp32, in blocks where every 16-lane row group takes the exact path at once and
    in blocks where only some do: in place and fused, bit-exact against the oracle."""
    B, N, H, D = 1, 192, 3, 128
    rng = np.random.default_rng(29)
    x = rng.standard_normal((B, N, 3 * H, D))
    tie = np.zeros(D)
    tie[:2] = (1.0, 2.0 ** -12)                                       # 1 + 2^-24: a tie, rounds to even
    broken = tie.copy()
    broken[2] = 2.0 ** -60                                            # + 2^-120: rounds up
    odd = np.zeros(D)
    odd[:4] = (1.0, 2.0 ** -12, 2.0 ** -12, 2.0 ** -12)              # a tie above an odd value
    for n in range(0, 64):                                            # block 0: every row takes the exact path
        x[0, n] = rng.standard_normal((3 * H, D)) * np.exp2(rng.integers(-133, 100, (3 * H, D)).astype(np.float64))
    for n in range(64, 128):                                          # block 1: constructed rows, mixed
        kind = n % 4
        if kind == 0:
            x[0, n, :, :] = broken * rng.choice([1.0, 2.0 ** 20, 2.0 ** -40], (3 * H, 1))
        elif kind == 1:
            x[0, n, :, :] = tie
        elif kind == 2:
            x[0, n, :, :] = odd * 2.0 ** -30
    x[0, 130] = 2.0 ** 70                                             # squares past the fp32 range
    x[0, 131, :, :8] = 2.0 ** -133                                    # subnormals beside normal values
    packed = torch.from_numpy(x.reshape(B, N, 3 * H * D)).float().to(torch.bfloat16)
    HD = H * D
    q, k, v = (packed[:, :, i * HD:(i + 1) * HD].unflatten(2, (H, D)) for i in range(3))
    case = inputs.Case("exact_sum", B, N, H, D, q, k, v, packed)
    nr = inputs.norm_rope_params(N, seed=10)
    want = _oracle_transformed(case, nr)
    g = G.gpu_case(case)
    sage.sage_qk_norm_rope(g.q, g.k, nr.to("cuda").gamma_q, nr.to("cuda").gamma_k, nr.rope.cuda(), nr.eps)
    torch.cuda.synchronize()
    assert torch.equal(g.q.cpu().view(torch.int16), want.q.view(torch.int16)), "Q"
    assert torch.equal(g.k.cpu().view(torch.int16), want.k.view(torch.int16)), "K"
    g2 = G.gpu_case(case)
    buf = sage.Buffers(B, N, H)
    sage.quantize_qkv_rope(g2.q, g2.k, g2.v, nr.to("cuda"), buf)
    torch.cuda.synchronize()
    G.check_quant_bitexact(buf, G.OracleRef(want))
