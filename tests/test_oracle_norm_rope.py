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


# ---- the sum of squares: the exact sum, rounded once to fp32 ----------------
from fractions import Fraction  # noqa: E402


def rn32(F: Fraction) -> float:
    """The fp32 value nearest to the exact non-negative rational F (ties to even; +inf from 2^128 on)."""
    if F == 0:
        return 0.0
    e = F.numerator.bit_length() - F.denominator.bit_length()      # 2^e <= F < 2^(e+2)
    if Fraction(2) ** e > F:
        e -= 1
    p = max(e - 23, -149)                                              # the fp32 quantum at F
    scaled = F / Fraction(2) ** p
    q = scaled.numerator // scaled.denominator
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    v = Fraction(q) * Fraction(2) ** p
    return float("inf") if v >= Fraction(2) ** 128 else float(v)      # exact: an fp32 value fits in fp64


def exact_ss(bits) -> Fraction:
    vals = (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return sum((Fraction(float(v)) ** 2 for v in vals), Fraction(0))


def bits_of(x):
    return (bf16(x).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rows_to_check():
    rng = np.random.default_rng(21)
    rows = [bits_of(rng.standard_normal(D) * 2.0 ** rng.integers(-60, 60)) for _ in range(120)]
    # exponents spread over the whole bf16 range, subnormals included
    for _ in range(40):
        rows.append(bits_of(rng.standard_normal(D) * np.exp2(rng.integers(-140, 120, D).astype(np.float64))))
    # squares past the fp32 range (ss = +inf) and just inside it
    rows.append(bits_of(np.full(D, 2.0 ** 70)))
    rows.append(bits_of(np.r_[2.0 ** 63 * 1.5, np.zeros(D - 1)]))
    # exact ties between two fp32 values, and ties broken by a square 2^96 times smaller than the ulp
    one_tie = np.zeros(D)
    one_tie[:2] = (1.0, 2.0 ** -12)                       # 1 + 2^-24: halfway between 1 and 1 + 2^-23
    rows.append(bits_of(one_tie))
    broken = one_tie.copy()
    broken[2] = 2.0 ** -60                                 # 1 + 2^-24 + 2^-120: rounds up
    rows.append(bits_of(broken))
    odd_tie = np.zeros(D)
    odd_tie[:4] = (1.0, 2.0 ** -12, 2.0 ** -12, 2.0 ** -12)    # 1 + 3 * 2^-24: halfway above an odd value
    rows.append(bits_of(odd_tie))
    rows.append(np.zeros(D, np.uint16))                    # all zero (and -0)
    rows.append(np.full(D, 0x8000, np.uint16))
    rows.append(np.arange(1, D + 1, dtype=np.uint16))      # bf16 subnormals only: ss is an fp32 subnormal or 0
    return np.stack(rows)


def test_sum_squares_is_the_rounded_exact_sum():
    rows = _rows_to_check()
    got = oracle.sum_squares(rows)
    want = np.array([rn32(exact_ss(r)) for r in rows], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.isinf(got[120 + 40]) and np.isfinite(got[120 + 41])
    tie, broken, odd = got[162], got[163], got[164]
    assert tie == 1.0 and broken == np.float32(1 + 2.0 ** -23) and odd == np.float32(1 + 2.0 ** -22)


def test_sum_squares_is_not_an_fp64_sum():
    # the tie-breaking square is far below an fp64 ulp of the total: an fp64 sum in any order, rounded
    # to fp32, lands on the tie and rounds to even, while the exact sum rounds up
    row = _rows_to_check()[163]
    sq = ((row.astype(np.uint32) << 16).view(np.float32).astype(np.float64)) ** 2
    assert np.float32(sq.sum()) == 1.0 and np.float32(sq[::-1].sum()) == 1.0
    assert oracle.sum_squares(row[None])[0] == np.float32(1 + 2.0 ** -23)


def test_norm_uses_the_exact_sum():
    # the transform of the tie-broken row equals the formula evaluated with rn32(exact sum) for ss
    row = _rows_to_check()[163].astype(np.uint32)
    x = (row << 16).view(np.float32)
    view = oracle.View.from_bnhd(row.astype(np.uint16).reshape(1, 1, 1, D))
    eps = np.float32(1e-6)
    got = oracle.norm_rope(view, np.ones(D), identity_table(1), float(eps))
    ss = np.float32(rn32(exact_ss(row.astype(np.uint16))))
    r = np.float32(1.0) / np.sqrt(np.float32(ss / np.float32(D) + eps))
    want = bits_of((x * r) * np.float32(1.0))
    assert np.array_equal(got.reshape(-1), want)
