"""Pins of the oracle's RMSNorm + RoPE of Q and K (the in-place transform before
quantisation), against closed forms and invariants that do not restate its
formula: unit RMS per head row, exact power-of-two weights, exact quarter and
half turns of each channel pair (which catch a wrong pairing, sign or index),
eps inside the square root, one-hot rows, row independence, and agreement of
the fixed-order fp32 evaluation with an unrounded fp64 one."""
import math

import numpy as np
import pytest

import oracle
from quantized_softmax_attention_amd import inputs
from tests.helpers import oracle_view

D = 128


def bf16(x):
    """fp64 -> the nearest bf16 value (RNE) as float64, via fp32 (exact for the
    values used here, which are fp32 already or need one rounding only)."""
    x = np.asarray(x, np.float64).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lower, upper = u & 0xFFFF, u >> 16
    upper = upper + ((lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1)))
    return (upper.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def view_of(x64):
    """A contiguous [B, N, H, D] oracle view of bf16 values."""
    return oracle.View.from_bnhd(np.asarray(bf16(x64), np.float32).view(np.uint32).__rshift__(16).astype(np.uint16))


def values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def identity_table(N):
    t = np.zeros((N, D // 2, 2), np.float32)
    t[:, :, 0] = 1.0
    return t


def rand_x(B, N, H, seed, head_scale=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, H, D))
    if head_scale:
        x *= np.exp2(rng.integers(-8, 9, size=(B, N, H, 1)))
    return bf16(x)


def test_unit_rms_per_head_row():
    x = rand_x(2, 9, 5, seed=1)
    y = values(oracle.norm_rope(view_of(x), np.ones(D), identity_table(9), 1e-12))
    ms = (y * y).mean(axis=-1)
    assert np.abs(ms - 1.0).max() < 4e-3          # bf16 storage only
    # the direction of every row is kept
    cos = (x * y).sum(-1) / np.sqrt((x * x).sum(-1) * (y * y).sum(-1))
    assert cos.min() > 1 - 1e-4


def test_power_of_two_weights_scale_exactly():
    x = rand_x(1, 7, 3, seed=2)
    g = np.exp2(np.arange(D) % 3 - 1.0)            # 0.5, 1, 2, ...
    base = values(oracle.norm_rope(view_of(x), np.ones(D), identity_table(7), 1e-6))
    y = values(oracle.norm_rope(view_of(x), g, identity_table(7), 1e-6))
    assert np.array_equal(y, base * g)


def test_quarter_and_half_turns_of_each_pair():
    N = 6
    x = rand_x(1, N, 2, seed=3)
    n = values(oracle.norm_rope(view_of(x), np.ones(D), identity_table(N), 1e-6))
    tab = identity_table(N)
    # pair i turned by a quarter turn for odd i, a half turn for i % 4 == 2
    tab[:, 1::2] = (0.0, 1.0)
    tab[:, 2::4] = (-1.0, 0.0)
    y = values(oracle.norm_rope(view_of(x), np.ones(D), tab, 1e-6))
    a, b = n[..., 0::2], n[..., 1::2]
    ya, yb = y[..., 0::2], y[..., 1::2]
    i = np.arange(D // 2)
    q, h, e = (i % 2 == 1), (i % 4 == 2), (i % 4 == 0)
    assert np.array_equal(ya[..., q], -b[..., q]) and np.array_equal(yb[..., q], a[..., q])
    assert np.array_equal(ya[..., h], -a[..., h]) and np.array_equal(yb[..., h], -b[..., h])
    assert np.array_equal(ya[..., e], a[..., e]) and np.array_equal(yb[..., e], b[..., e])


def test_rotation_keeps_pair_norms_and_angles():
    N = 40
    x = rand_x(1, N, 3, seed=4)
    tab = inputs.video_rope_table(N).numpy()
    # a table of exact angle pairs is what the test checks against: unit length
    assert np.allclose(np.hypot(tab[..., 0], tab[..., 1]), 1.0, atol=1e-6)
    n = oracle.norm_rope_f64(view_of(x), np.ones(D), identity_table(N), 1e-6)
    y = oracle.norm_rope_f64(view_of(x), np.ones(D), tab, 1e-6)
    r0 = np.hypot(n[..., 0::2], n[..., 1::2])
    r1 = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.allclose(r0, r1, rtol=1e-6, atol=0)
    # the angle of each pair advances by the table's angle (complex product)
    zn = n[..., 0::2] + 1j * n[..., 1::2]
    zy = y[..., 0::2] + 1j * y[..., 1::2]
    zt = tab[None, :, None, :, 0].astype(np.float64) + 1j * tab[None, :, None, :, 1]
    assert np.allclose(zy, zn * zt, rtol=0, atol=1e-12 * np.abs(zn).max() + 1e-6 * np.abs(zn))


def test_eps_sits_inside_the_square_root():
    N = 2
    x = np.full((1, N, 1, D), 2.0 ** -40)
    y = values(oracle.norm_rope(view_of(x), np.ones(D), identity_table(N), 1e-6))
    want = 2.0 ** -40 / math.sqrt(2.0 ** -80 + 1e-6)
    assert np.allclose(y, want, rtol=2 ** -8)
    x = np.ones((1, N, 1, D))
    y = values(oracle.norm_rope(view_of(x), np.ones(D), identity_table(N), 0.25))
    assert np.allclose(y, 1 / math.sqrt(1.25), rtol=2 ** -8)


def test_one_hot_row():
    x = np.zeros((1, 1, 2, D))
    x[0, 0, 0, 37] = -3.0
    x[0, 0, 1, 0] = 0.125
    y = values(oracle.norm_rope(view_of(x), np.ones(D), identity_table(1), 1e-12))
    assert y[0, 0, 0, 37] == bf16(-math.sqrt(D)) and np.count_nonzero(y[0, 0, 0]) == 1
    assert y[0, 0, 1, 0] == bf16(math.sqrt(D)) and np.count_nonzero(y[0, 0, 1]) == 1


def test_rows_are_independent():
    N = 5
    x = rand_x(1, N, 4, seed=6)
    tab = inputs.video_rope_table(N).numpy()
    g = inputs.norm_rope_params(N).gamma_q.numpy()
    y = oracle.norm_rope(view_of(x), g, tab, 1e-6)
    x2 = x.copy()
    x2[0, 2, 1] *= 3.0
    x2[0, 4] = 0.0
    y2 = oracle.norm_rope(view_of(x2), g, tab, 1e-6)
    changed = np.zeros((1, N, 4), bool)
    changed[0, 2, 1] = True
    changed[0, 4] = True
    same = (y == y2).all(axis=-1)
    assert same[~changed].all()
    assert not values(y2[0, 4]).any()               # zero rows stay zero (eps > 0), up to the sign


@pytest.mark.parametrize("stress", [False, True])
def test_fp32_order_close_to_fp64(stress):
    case = inputs.packed_case(1, 300, 3, seed=8, stress=stress)
    prm = inputs.norm_rope_params(300)
    for t, g in ((case.q, prm.gamma_q), (case.k, prm.gamma_k)):
        v = oracle_view(t)
        y32 = values(oracle.norm_rope(v, g.numpy(), prm.rope.numpy(), prm.eps))
        y64 = oracle.norm_rope_f64(v, g.numpy(), prm.rope.numpy(), prm.eps)
        # within one bf16 rounding of the exact value, and equal to its bf16
        # rounding except where fp32 error crosses a rounding boundary
        assert np.all(np.abs(y32 - y64) <= 2.0 ** -8 * np.abs(y64) + 1e-30)
        assert (y32 != bf16(y64)).mean() < 2e-3
