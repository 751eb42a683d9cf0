"""Instruction probes on the GPU: the facts the attention kernels rely on.

* v_mfma_i32_32x32x32_i8, v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, unit scales)
  and v_mfma_f32_32x32x16_bf16 take A and B with the SAME k-order per (half-wave,
  byte) and return lane l, register r = element (8*(r/4) + 4*(l/32) + r%4, l%32).
* The FP8 MFMA is not an exact dot product: products are summed in groups of 8
  aligned to the group's largest product with about 12 fractional bits (smaller
  terms are truncated); the group sums and the input accumulator are added in
  fp32.  Measured: |error| <= 2^-10 of the largest product of a dot product.
* v_cvt_pk_fp8_f32 rounds like the oracle's E4M3FN codec on [0, 460], and on [-448.0001, 448.0001]
  with both zeros and fp32 subnormals (the V quantiser's quotients).
* v_permlane32_swap(x, x) gives each lane the values of lanes l%32 and l%32 + 32.
* v_exp_f32 is exact at integers and within a few ulp elsewhere.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_softmax_attention_amd import sage

pytestmark = pytest.mark.gpu
PROBE = os.path.join(os.path.dirname(sage.LIB_PATH), "libsage_probe.so")


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return ctypes.CDLL(PROBE)


def _run(fn, *tensors):
    assert fn(*(ctypes.c_void_p(t.data_ptr()) for t in tensors)) == 0


def _acc_to_matrix(d):
    """[64 lanes][16 regs] -> 32x32 by the assumed accumulator layout."""
    M = np.zeros((32, 32), d.dtype)
    for l in range(64):
        for r in range(16):
            M[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = d[l, r]
    return M


def _operands(A, Bm, per_lane):
    """Lane l holds A[l%32][k0 + e] and B[k0 + e][l%32], k0 = per_lane * (l // 32)."""
    a = np.zeros((64, per_lane), A.dtype)
    b = np.zeros((64, per_lane), Bm.dtype)
    for l in range(64):
        k0 = per_lane * (l // 32)
        a[l] = A[l % 32, k0:k0 + per_lane]
        b[l] = Bm[k0:k0 + per_lane, l % 32]
    return a, b


def test_mfma_i8_layout(probe):
    rng = np.random.default_rng(0)
    A = rng.integers(-127, 128, (32, 32)).astype(np.int8)
    Bm = rng.integers(-127, 128, (32, 32)).astype(np.int8)
    a, b = _operands(A, Bm, 16)
    ta, tb = (torch.from_numpy(x.copy()).cuda() for x in (a, b))
    td = torch.zeros(64, 16, dtype=torch.int32, device="cuda")
    _run(probe.sage_probe_mfma_i8, ta, tb, td)
    got = _acc_to_matrix(td.cpu().numpy())
    assert np.array_equal(got, A.astype(np.int64) @ Bm.astype(np.int64))


def _f8_run(probe, A, Bm, C=None):
    a, b = _operands(A, Bm, 32)
    ta, tb = (torch.from_numpy(x.copy()).cuda() for x in (a, b))
    td = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    if C is None:
        _run(probe.sage_probe_mfma_f8, ta, tb, td)
    else:
        c = np.zeros((64, 16), np.float32)
        for l in range(64):
            for r in range(16):
                c[l, r] = C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
        _run(probe.sage_probe_mfma_f8_acc, ta, tb, torch.from_numpy(c).cuda(), td)
    return _acc_to_matrix(td.cpu().numpy()).astype(np.float64)


def _dec(x):
    return oracle.e4m3_decode(x).reshape(x.shape)


def test_mfma_f8_layout(probe):
    rng = np.random.default_rng(1)
    codes = np.array([c for c in range(256) if (c & 0x7F) <= 0x58], np.uint8)   # |x| <= 16
    for trial in range(4):
        A = rng.choice(codes, (32, 64))
        Bm = rng.choice(codes, (64, 32))
        got = _f8_run(probe, A, Bm)
        want = _dec(A) @ _dec(Bm)
        maxprod = np.max(np.abs(_dec(A)[:, :, None] * _dec(Bm)[None, :, :]), axis=1)
        assert np.all(np.abs(got - want) <= 2.0 ** -10 * maxprod), trial


def test_mfma_f8_accumulation_model(probe):
    # single products are exact
    A = np.zeros((32, 64), np.uint8); Bm = np.zeros((64, 32), np.uint8)
    A[:, 5] = oracle.e4m3_encode(np.linspace(-448, 448, 32))
    Bm[5, :] = oracle.e4m3_encode(np.linspace(2.0 ** -9, 3.5, 32))
    assert np.array_equal(_f8_run(probe, A, Bm), _dec(A) @ _dec(Bm))
    # 256 + 63 products of 2^-6: the 7 sharing 256's group of 8 are truncated away
    A = np.zeros((32, 64), np.uint8); Bm = np.zeros((64, 32), np.uint8)
    A[:, 0] = oracle.e4m3_encode([16.0] * 32); Bm[0, :] = oracle.e4m3_encode([16.0] * 32)
    A[:, 1:] = oracle.e4m3_encode(np.full(32 * 63, 2.0 ** -3)).reshape(32, 63)
    Bm[1:, :] = oracle.e4m3_encode(np.full(63 * 32, 2.0 ** -3)).reshape(63, 32)
    got = _f8_run(probe, A, Bm)
    assert np.all(got == 256 + 56 * 2.0 ** -6)
    # the input accumulator is added in fp32: 65536 + small exact sums stay exact
    rng = np.random.default_rng(3)
    A = oracle.e4m3_encode(rng.choice([1.0, -1.0, 1.5, 0.75], 32 * 64)).reshape(32, 64)
    Bm = oracle.e4m3_encode(rng.choice([1.0, 0.5, -1.25], 64 * 32)).reshape(64, 32)
    C = np.full((32, 32), 65536.0)
    assert np.array_equal(_f8_run(probe, A, Bm, C), C + _dec(A) @ _dec(Bm))


def test_mfma_bf16_layout(probe):
    rng = np.random.default_rng(2)
    A = torch.randn(32, 16, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    Bm = torch.randn(16, 32, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    a, b = _operands(A.view(torch.int16).numpy(), Bm.view(torch.int16).numpy(), 8)
    ta, tb = (torch.from_numpy(x.copy()).cuda() for x in (a, b))
    td = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    _run(probe.sage_probe_mfma_bf16, ta, tb, td)
    got = _acc_to_matrix(td.cpu().numpy()).astype(np.float64)
    want = A.double().numpy() @ Bm.double().numpy()
    assert np.max(np.abs(got - want)) <= 1e-5
    del rng


def test_cvt_pk_fp8_matches_codec(probe):
    table = oracle.e4m3_decode(np.arange(0x7F))
    mids = (table[1:] + table[:-1]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([table, mids, rng.uniform(0, 448, 100000), np.exp(rng.uniform(-12, np.log(448), 100000)),
                        [448.0, 448.001, 450.0, 455.0, 459.9, 2.0 ** -10, 3 * 2.0 ** -11, 0.0]]).astype(np.float32)
    x = np.concatenate([x, np.zeros((-len(x)) % 4, np.float32)])
    tx = torch.from_numpy(x).cuda()
    out = torch.zeros(len(x), dtype=torch.uint8, device="cuda")
    assert probe.sage_probe_cvt_fp8(ctypes.c_void_p(tx.data_ptr()), len(x), ctypes.c_void_p(out.data_ptr())) == 0
    got = out.cpu().numpy()
    want = oracle.e4m3_encode(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_cvt_pk_fp8_matches_codec_signed_and_tiny(probe):
    """The V quantiser's quotients: |y| <= 448 (1 + 2^-22) of either sign, both zeros, every
    rounding boundary and its fp32 neighbours, magnitudes down to the fp32 subnormals."""
    table = oracle.e4m3_decode(np.arange(0x7F)).astype(np.float32)
    mids = ((table[1:].astype(np.float64) + table[:-1]) / 2).astype(np.float32)   # exact in fp32
    rng = np.random.default_rng(6)
    mags = np.concatenate([
        table, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
        rng.uniform(0, 448, 100000).astype(np.float32),
        np.exp2(rng.uniform(-150, np.log2(448), 200000)).astype(np.float32),   # to the fp32 subnormals
        np.array([448.0, np.nextafter(np.float32(448), np.float32(np.inf)), 448 * (1 + 2.0 ** -22), 2.0 ** -10,
                  2.0 ** -126, 2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -127], np.float32)])
    x = np.concatenate([mags, -mags]).astype(np.float32)
    x = np.concatenate([x, np.zeros((-len(x)) % 4, np.float32)])
    assert np.signbit(x).any() and (x == 0).any() and (np.abs(x[x != 0]) < 2.0 ** -126).any()
    tx = torch.from_numpy(x).cuda()
    out = torch.zeros(len(x), dtype=torch.uint8, device="cuda")
    assert probe.sage_probe_cvt_fp8(ctypes.c_void_p(tx.data_ptr()), len(x), ctypes.c_void_p(out.data_ptr())) == 0
    got = out.cpu().numpy()
    want = oracle.e4m3_encode(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_permlane32_swap_pairs(probe):
    x = torch.arange(64, dtype=torch.int32, device="cuda") * 7 + 3
    out = torch.zeros(128, dtype=torch.int32, device="cuda")
    _run(probe.sage_probe_swap, x, out)
    o = out.cpu().numpy().reshape(2, 64)
    xs = x.cpu().numpy()
    for l in range(64):
        assert sorted(o[:, l]) == sorted([xs[l % 32], xs[l % 32 + 32]])


def test_exp2_accuracy(probe):
    rng = np.random.default_rng(6)
    x = np.concatenate([np.arange(-20, 10, dtype=np.float32), rng.uniform(-30, 9, 100000).astype(np.float32),
                        [-np.inf]]).astype(np.float32)
    tx = torch.from_numpy(x).cuda()
    out = torch.zeros_like(tx)
    assert probe.sage_probe_exp2(ctypes.c_void_p(tx.data_ptr()), len(x), ctypes.c_void_p(out.data_ptr())) == 0
    got = out.cpu().numpy().astype(np.float64)
    want = np.exp2(x.astype(np.float64))
    assert np.array_equal(got[:30], want[:30]) and got[-1] == 0.0
    fin = np.isfinite(x)
    rel = np.abs(got[fin] - want[fin]) / want[fin]
    assert rel.max() <= 4 * 2.0 ** -23, rel.max()


def test_ds_read_tr16_b64_lane_rule(probe):
    # Within each 16-lane group the 16 lanes' 8-byte reads form a 16x4 matrix
    # M[s][c] (s = lane in group, c = element); output lane i holds
    # M[4j + i//4][i % 4] for j = 0..3.
    vals = torch.arange(4096, dtype=torch.int16, device="cuda")
    rng = np.random.default_rng(7)
    addr = (rng.integers(0, 4096 // 4 - 1, 64) * 8).astype(np.int32)    # random 8-byte aligned rows
    ta = torch.from_numpy(addr).cuda()
    out = torch.zeros(64 * 4, dtype=torch.int16, device="cuda")
    assert probe.sage_probe_tr16(ctypes.c_void_p(vals.data_ptr()), ctypes.c_void_p(ta.data_ptr()),
                                 ctypes.c_void_p(out.data_ptr())) == 0
    got = out.cpu().numpy().reshape(64, 4)
    src = (addr // 2)[:, None] + np.arange(4)[None, :]        # element indices each lane reads
    for lane in range(64):
        g, i = lane // 16, lane % 16
        want = [src[16 * g + 4 * j + i // 4, i % 4] for j in range(4)]
        assert list(got[lane]) == want, lane
