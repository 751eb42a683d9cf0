"""Pins of the oracle's quantisers (K mean, INT8 Q/K blocks, E4M3 V channels):
hand cases with exact ties, closed forms, and library re-computations with
torch/numpy (torch.round is round-half-to-even; torch's float8_e4m3fn cast is
the OCP codec)."""
import numpy as np
import pytest
import torch

import oracle
from quantized_softmax_attention_amd import inputs
from tests.helpers import bnhd, oracle_view


def _f32(t):
    return t.float().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float32)


# ------------------------------------------------------------------ K mean
def test_kmean_constant_channel_is_exact():
    B, N, H, D = 1, 200, 2, 4
    x = np.zeros((B, N, H, D), np.float32)
    x[..., 0] = 0.75
    x[..., 1] = -3.5
    x[0, :, 1, 2] = 1.0 / 64
    km = oracle.kmean(oracle_view(bnhd(x)))
    assert km[0, 0, 0] == 0.75 and km[0, 1, 1] == -3.5 and km[0, 1, 2] == 1.0 / 64 and km[0, 0, 3] == 0.0


def test_kmean_matches_fp64_library_mean():
    c = inputs.hnd_case(2, 1000, 3, D=16, seed=5)
    km = oracle.kmean(oracle_view(c.k))
    ref = c.k.double().mean(dim=1).float().numpy()          # [B, H, D]
    assert np.array_equal(km, ref)


def test_kmean_arithmetic_sequence_closed_form():
    # k_n = n / 8 for n < N (exact in bf16 for N <= 256*8): mean = (N - 1) / 16
    B, N, H, D = 1, 777, 1, 2
    x = np.broadcast_to((np.arange(N, dtype=np.float32) / 8)[None, :, None, None], (B, N, H, D)) % 32
    km = oracle.kmean(oracle_view(bnhd(x)))
    assert km[0, 0, 0] == np.float32(np.sum(x[0, :, 0, 0].astype(np.float64)) / N)
    y = np.broadcast_to((np.arange(256, dtype=np.float32) / 8)[None, :, None, None], (1, 256, 1, 2))
    assert oracle.kmean(oracle_view(bnhd(y)))[0, 0, 0] == np.float32(255 / 16)


def test_kmean_layout_independent():
    c = inputs.packed_case(1, 300, 3, D=128, seed=2)
    hnd = c.k.transpose(1, 2).contiguous().transpose(1, 2)
    assert np.array_equal(oracle.kmean(oracle_view(c.k)), oracle.kmean(oracle_view(hnd)))


# ------------------------------------------------------------- INT8 blocks
def test_quant_q_hand_cases_ties_to_even():
    D = 8
    x = np.zeros((1, 64, 1, D), np.float32)
    # block 0: amax 127 -> scale exactly 1, so x / scale = x and ties are visible
    x[0, 0, 0, :] = [127, 2.5, 3.5, -2.5, -3.5, 126.5, 0.5, -127]
    x[0, 1, 0, :3] = [1.5, -0.5, 0.25]
    # block 1 (rows 32..63): all zero
    codes, scales = oracle.quant_q(oracle_view(bnhd(x)), blk=32)
    assert scales[0, 0, 0] == 1.0 and scales[0, 0, 1] == 0.0
    assert list(codes[0, 0, 0]) == [127, 2, 4, -2, -4, 126, 0, -127]
    assert list(codes[0, 0, 1, :3]) == [2, 0, 0]
    assert not codes[0, 0, 32:].any()


def test_quant_q_single_nonzero_and_negative_amax():
    x = np.zeros((1, 40, 1, 4), np.float32)
    x[0, 3, 0, 2] = -0.3125
    x[0, 35, 0, 1] = 6.0
    x[0, 36, 0, 0] = -1.5
    codes, scales = oracle.quant_q(oracle_view(bnhd(x)), blk=32)
    assert scales.shape == (1, 1, 2)
    assert scales[0, 0, 0] == np.float32(0.3125) / np.float32(127)
    assert codes[0, 0, 3, 2] == -127 and np.count_nonzero(codes[0, 0, :32]) == 1
    # second (ragged, 8-token) block: amax 6 -> scale 6/127; -1.5/scale = -31.75 -> -32
    assert scales[0, 0, 1] == np.float32(6.0) / np.float32(127)
    assert codes[0, 0, 35, 1] == 127 and codes[0, 0, 36, 0] == -32


def _torch_int8(x_blocks):
    """Library re-computation for one block: torch fp32 division and round-half-even."""
    x = torch.from_numpy(np.ascontiguousarray(x_blocks, np.float32))
    amax = x.abs().max()
    if amax == 0:
        return torch.zeros_like(x, dtype=torch.int8).numpy(), np.float32(0)
    s = amax / torch.tensor(127.0)
    return torch.clamp(torch.round(x / s), -127, 127).to(torch.int8).numpy(), np.float32(s.item())


@pytest.mark.parametrize("N", [1, 31, 32, 33, 100, 257])
def test_quant_q_matches_library_recomputation(N):
    c = inputs.hnd_case(1, N, 2, D=128, seed=N)
    codes, scales = oracle.quant_q(oracle_view(c.q), blk=32)
    q = _f32(c.q)                        # [B, N, H, D]
    for h in range(2):
        for t in range(-(-N // 32)):
            blk = q[0, t * 32:(t + 1) * 32, h]
            rc, rs = _torch_int8(blk)
            assert scales[0, h, t] == rs
            assert np.array_equal(codes[0, h, t * 32:(t + 1) * 32], rc)


def test_quant_reconstruction_bound():
    c = inputs.hnd_case(1, 256, 2, D=128, seed=9)
    codes, scales = oracle.quant_q(oracle_view(c.q), blk=32)
    q = _f32(c.q).transpose(0, 2, 1, 3)            # [B, H, N, D]
    s = np.repeat(scales, 32, axis=2)[..., None]
    err = np.abs(q - codes * s.astype(np.float64))
    # half a step, plus the rounding of the fp32 quotient x / scale (|x / scale| <= 127)
    assert np.all(err <= s * (0.5 + 127 * 2.0 ** -23))
    assert err.max() / s.max() > 0.45               # the bound is nearly attained
    assert np.all(np.abs(codes) <= 127)


def test_quant_k_smoothing_matches_library_recomputation():
    c = inputs.hnd_case(1, 150, 2, D=128, seed=3)
    km = oracle.kmean(oracle_view(c.k))
    codes, scales = oracle.quant_k(oracle_view(c.k), km, blk=64)
    k = _f32(c.k)
    assert scales.shape == (1, 2, 3)
    for h in range(2):
        xs = (torch.from_numpy(k[0, :, h]) - torch.from_numpy(km[0, h])).numpy()   # fp32 subtraction
        for t in range(3):
            rc, rs = _torch_int8(xs[t * 64:(t + 1) * 64])
            assert scales[0, h, t] == rs
            assert np.array_equal(codes[0, h, t * 64:(t + 1) * 64], rc)


def test_quant_k_constant_channels_give_zero():
    x = np.zeros((1, 130, 1, 4), np.float32)
    x[..., 0] = 2.5
    x[..., 3] = -0.125
    km = oracle.kmean(oracle_view(bnhd(x)))
    codes, scales = oracle.quant_k(oracle_view(bnhd(x)), km, blk=64)
    assert not codes.any() and not scales.any()


# -------------------------------------------------------------- V channels
def test_quant_v_matches_library_recomputation():
    c = inputs.packed_case(1, 333, 2, D=128, seed=4, stress=True)
    codes, scales = oracle.quant_v(oracle_view(c.v))
    v = torch.from_numpy(_f32(c.v)).permute(0, 2, 1, 3)     # [B, H, N, D]
    amax = v.abs().amax(dim=2)                                 # [B, H, D]
    sv = amax / torch.tensor(448.0)
    assert np.array_equal(scales, sv.numpy())
    x = torch.clamp(v / sv[:, :, None, :], -448.0, 448.0)     # saturation
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # the amax element of every channel maps to +-448
    top = v.abs().argmax(dim=2)
    got = np.take_along_axis(codes, top.numpy()[:, :, None, :], axis=2)
    assert np.all((got & 0x7F) == 0x7E)


def test_quant_v_zero_channel_and_single_token():
    x = np.zeros((1, 5, 1, 4), np.float32)
    x[0, :, 0, 1] = [1, -2, 0.5, 0, 3]
    x[0, 2, 0, 2] = -7.0
    codes, scales = oracle.quant_v(oracle_view(bnhd(x)))
    assert scales[0, 0, 0] == 0 and not codes[0, 0, :, 0].any()
    assert scales[0, 0, 1] == np.float32(3) / np.float32(448)
    assert codes[0, 0, 4, 1] == 0x7E and codes[0, 0, 2, 2] == 0xFE
    assert codes[0, 0, 0, 2] == 0x00 and codes[0, 0, 3, 1] == 0x00
