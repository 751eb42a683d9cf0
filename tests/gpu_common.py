"""Helpers for the GPU parity tests: run the library through its C ABI, bring
results back, and compute (cached) oracle references for the same seeded
inputs.  Oracle inputs are always the seeded CPU tensors, never GPU output."""
import functools
import math

import numpy as np
import torch

import oracle
from quantized_softmax_attention_amd import inputs, sage
from tests.helpers import oracle_view

SM = 1.0 / math.sqrt(128.0)


def kappa():
    """Token (within a 64-key tile) of byte p of a V-code row, as the public
    header defines it: p = 32u + j -> 32*(j/16) + 8*((j%16)/4) + 4u + j%4."""
    p = np.arange(64)
    u, j = p // 32, p % 32
    return 32 * (j // 16) + 8 * ((j % 16) // 4) + 4 * u + (j % 4)


def unpermute_v(vc_tiles: np.ndarray, N: int) -> np.ndarray:
    """[B, H, T, D, 64] tile-major codes -> logical [B, H, N, D] (plus a check
    that the padding tokens are zero)."""
    B, H, T, D, P = vc_tiles.shape
    logical = np.empty((B, H, T * 64, D), np.uint8)
    k = kappa()
    for p in range(64):
        logical[:, :, k[p]::64, :] = vc_tiles[:, :, :, :, p]
    assert not logical[:, :, N:].any(), "padding tokens must hold 0x00"
    return logical[:, :, :N]


def gpu_case(case: inputs.Case) -> inputs.Case:
    return case.to("cuda")


def run_quant(gcase: inputs.Case, fused: bool = False):
    """Quantise on the GPU (quantize_qk + quantize_v, or the single quantize_qkv
    call); return the buffers.  Code buffers start filled with 0x5A so that a
    missed write cannot pass as a zero."""
    buf = sage.Buffers(gcase.B, gcase.N, gcase.H)
    for t in (buf.q_codes, buf.k_codes, buf.v_codes):
        t.view(torch.uint8).fill_(0x5A)
    for t in (buf.q_scale, buf.k_scale, buf.k_mean, buf.v_scale):
        t.fill_(float("nan"))
    if fused:
        sage.quantize_qkv(gcase.q, gcase.k, gcase.v, buf)
    else:
        sage.quantize(gcase.q, gcase.k, gcase.v, buf)
    torch.cuda.synchronize()
    return buf


def check_quant_bitexact(buf, ref: "OracleRef"):
    """Every quantiser output in buf (GPU) equals the oracle's for ref's case,
    bit for bit, with zero codes and scales in the padding."""
    case = ref.case
    B, N, H = case.B, case.N, case.H
    npad = sage.sage_npad(N)
    nq, nk = -(-N // 32), -(-N // 64)
    km = buf.k_mean.cpu().numpy()
    assert np.array_equal(km.view(np.uint32), ref.km.view(np.uint32)), "k_mean"
    qc, qs = buf.q_codes.cpu().numpy(), buf.q_scale.cpu().numpy()
    kc, ks = buf.k_codes.cpu().numpy(), buf.k_scale.cpu().numpy()
    (rqc, rqs), (rkc, rks) = ref.qq, ref.kq
    assert np.array_equal(qc[:, :, :N], rqc), "q_codes"
    assert np.array_equal(kc[:, :, :N], rkc), "k_codes"
    assert not qc[:, :, N:].any() and not kc[:, :, N:].any(), "padding codes"
    assert np.array_equal(qs[:, :, :nq].view(np.uint32), rqs.view(np.uint32)), "q_scale"
    assert np.array_equal(ks[:, :, :nk].view(np.uint32), rks.view(np.uint32)), "k_scale"
    assert not qs[:, :, nq:].any() and not ks[:, :, nk:].any(), "padding scales"
    assert qs.shape == (B, H, npad // 32) and ks.shape == (B, H, npad // 64)
    vc = unpermute_v(buf.v_codes.cpu().numpy(), N)
    rvc, rvs = ref.vq
    assert np.array_equal(buf.v_scale.cpu().numpy().view(np.uint32), rvs.view(np.uint32)), "v_scale"
    assert np.array_equal(vc, rvc), "v_codes"


def run_attn(gcase: inputs.Case, buf=None):
    if buf is None:
        buf = run_quant(gcase)
    out = sage.token_major_out(gcase.B, gcase.N, gcase.H)
    sage.sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, out, SM)
    torch.cuda.synchronize()
    return out, buf


def run_attn_bf16(gcase: inputs.Case):
    out = sage.token_major_out(gcase.B, gcase.N, gcase.H)
    sage.sage_attn_fwd_bf16(gcase.q, gcase.k, gcase.v, out, SM)
    torch.cuda.synchronize()
    return out


def run_attn_int8qk(gcase: inputs.Case, buf=None):
    """INT8 Q K^T (codes from sage_quantize_qk) with the bf16 V view unquantised."""
    if buf is None:
        buf = run_quant(gcase)
    out = sage.token_major_out(gcase.B, gcase.N, gcase.H)
    sage.sage_attn_fwd_int8qk(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, gcase.v, out, SM)
    torch.cuda.synchronize()
    return out, buf


def out_rows(out: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """[B, N, H, D] output -> [B, H, R, D] float64 at the sampled rows."""
    o = out.float().cpu().numpy()
    B, N, H, D = o.shape
    res = np.empty((B, H, rows.shape[2], D))
    for b in range(B):
        for h in range(H):
            res[b, h] = o[b, rows[b, h], h]
    return res


class OracleRef:
    """Oracle results for one seeded CPU case (quantisation at full size;
    attention on the requested rows)."""

    def __init__(self, case: inputs.Case):
        self.case = case
        self.q, self.k, self.v = (oracle_view(t) for t in (case.q, case.k, case.v))

    @functools.cached_property
    def km(self):
        return oracle.kmean(self.k)

    @functools.cached_property
    def qq(self):
        return oracle.quant_q(self.q, 32)

    @functools.cached_property
    def kq(self):
        return oracle.quant_k(self.k, self.km, 64)

    @functools.cached_property
    def vq(self):
        return oracle.quant_v(self.v)

    def exact(self, rows):
        return oracle.attn_exact(self.q, self.k, self.v, SM, rows)

    def method(self, rows):
        (qc, qs), (kc, ks), (vc, vs) = self.qq, self.kq, self.vq
        return oracle.attn_method(qc, qs, kc, ks, vc, vs, SM, rows)

    def int8qk(self, rows):
        (qc, qs), (kc, ks) = self.qq, self.kq
        return oracle.attn_int8qk(qc, qs, kc, ks, self.v, SM, rows)


@functools.lru_cache(maxsize=5)
def config_ref(name: str) -> OracleRef:
    return OracleRef(inputs.config(name))


def rel_l2(a, b) -> float:
    return oracle.rel_l2(a, b)


# Per-row bound: every compared row's L2 error within this fraction of the typical (RMS) row norm of the
# reference.  The whole-set rel-L2 of a large sample dilutes a local error (one wrong element among 1.15 M
# adds ~1e-3); per row, one wrong element of typical size is ~1/sqrt(128) = 0.088 of a row.  Rows of a
# diffuse attention have small norms, so the bound is taken against the typical norm, not each row's own.
# A correct kernel legitimately reaches ~1.5e-2 in a row where one large p lies at an E4M3 rounding midpoint
# and fp32 arithmetic rounds it to the other neighbour than the fp64 oracle (a step of 32/448 of that key's
# weight; block-24 head 20 row 24736: 1.35e-2, as close to the exact result as the oracle itself), so the
# bound leaves room for that and still fails a wrong element by 3x.
ROW_BOUND = 3e-2


def row_error(got, ref) -> float:
    """Largest row L2 error of got [..., D] against ref, relative to ref's RMS row norm."""
    err = np.sqrt(((np.asarray(got, np.float64) - ref) ** 2).sum(-1))
    typical = np.sqrt((np.asarray(ref, np.float64) ** 2).sum(-1).mean())
    return float(err.max() / typical) if typical > 0 else float(err.max())


def gate(got, ref, bound: float, label: str = "", row_bound: float = ROW_BOUND) -> float:
    """Assert the whole-set rel-L2 <= bound and every row within row_bound (row_error); return the rel-L2."""
    e, r = rel_l2(got, ref), row_error(got, ref)
    print("%s: rel-L2 %.3e (bound %.0e), worst row %.3e of the typical row norm (bound %.0e)"
          % (label, e, bound, r, row_bound), flush=True)
    assert e <= bound, (label, e, bound)
    assert r <= row_bound, (label, "row", r, row_bound)
    return e


def bf16_round(x: np.ndarray) -> np.ndarray:
    """The library's output rounding (bf16, nearest even) applied to an fp64
    oracle result, so that GPU bf16 outputs compare against the same definition."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float64)).float().to(torch.bfloat16).double().numpy()
