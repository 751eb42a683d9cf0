"""Pins of the oracle's OCP microscaling (MX) quantiser: the E2M1 element table,
nearest-even rounding by brute force, hand-computed blocks, and properties that
must hold for any input (scale from the block maximum, idempotence, every
element the nearest representable value)."""
import math

import numpy as np
import pytest

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_and_roundtrip():
    # OCP E2M1: exponent bias 1, one mantissa bit; 0 and 0.5 are subnormal
    for c in range(16):
        sign = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        mag = (m / 2) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert mag == E2M1[c & 7]
        assert oracle.e2m1_decode([c])[0] == sign * mag
        assert oracle.e2m1_encode([sign * mag])[0] == c


def test_e2m1_nearest_even_bruteforce():
    grid = np.arange(0, 7.5, 1 / 64)
    got = oracle.e2m1_decode(oracle.e2m1_encode(grid))
    for x, g in zip(grid, got):
        d = [abs(x - v) for v in E2M1]
        best = min(d)
        cands = [i for i in range(8) if d[i] == best]
        want = E2M1[cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]]
        assert g == want, (x, g, want)
    assert oracle.e2m1_encode([100.0])[0] == 7 and oracle.e2m1_encode([-100.0])[0] == 15


def test_mx_hand_blocks():
    x = np.zeros((4, 64))
    x[1, :32] = 1.0                   # max 2^0 -> X = -8 (E4M3), 1.0 * 2^8 = 256 -> code 0x78
    x[1, 32] = 1.9                    # max 1.9 -> X = -8, 1.9 * 256 = 486.4 saturates to 448 (0x7E)
    x[1, 33] = -0.5                   # -128 -> 0xF0
    x[2, :32] = 2.0 ** -130           # max below 2^-127 * 2^8: X clamps to -127, 2^-130 * 2^127 = 0.125 -> 0x20
    x[3, 0] = -0.0                    # an all-zero block keeps signed zeros
    c, s = oracle.mx_quantize(x, oracle.MX_E4M3)
    assert list(s[0]) == [0, 0] and not c[0].any()
    assert s[1, 0] == 127 - 8 and np.all(c[1, :32] == 0x78)
    assert s[1, 1] == 127 - 8 and c[1, 32] == 0x7E and c[1, 33] == 0xF0 and not c[1, 34:].any()
    assert s[2, 0] == 0 and np.all(c[2, :32] == 0x20)
    assert c[3, 0] == 0x80 and s[3, 0] == 0
    # E2M1: max 6 -> X = 0; 7 -> X = 0 and saturates to 6; 1 -> code 2; max 3.9 -> X = -1
    y = np.zeros((2, 32))
    y[0, :3] = [6.0, 1.0, 7.0]
    y[1, :3] = [3.9, -1.3, 0.2]
    c4, s4 = oracle.mx_quantize(y, oracle.MX_E2M1)
    assert list(s4[:, 0]) == [127, 126]
    assert c4[0, 0] == (7 | (2 << 4)) and (c4[0, 1] & 0xF) == 7
    # 3.9 / 2^-1 = 7.8 -> 6 (code 7); -1.3 * 2 = -2.6 -> -3 (code 13); 0.2 * 2 = 0.4 -> 0.5 (code 1)
    assert c4[1, 0] == (7 | (13 << 4)) and (c4[1, 1] & 0xF) == 1


@pytest.mark.parametrize("fmt", [oracle.MX_E4M3, oracle.MX_E2M1])
def test_mx_properties_on_random_blocks(fmt):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    x[5] = 0.0
    x[6, 3] = 1e-40                   # below every scale: rounds to zero
    # bf16 values, as the library's inputs are
    x = np.frombuffer((x.astype(np.float32).view(np.uint32) & 0xFFFF0000).astype(np.uint32).tobytes(),
                      np.float32).reshape(x.shape).astype(np.float64)
    c, s = oracle.mx_quantize(x, fmt)
    emax = 8 if fmt == oracle.MX_E4M3 else 2
    blocks = x.reshape(64, 4, 32)
    amax = np.abs(blocks).max(axis=2)
    for r in range(64):
        for b in range(4):
            if amax[r, b] > 0:
                want = max(-127, min(127, math.floor(math.log2(amax[r, b])) - emax))
            else:
                want = -127
            assert int(s[r, b]) - 127 == want
    deq = oracle.mx_dequantize(c, s, fmt)
    # idempotent: quantising the dequantised values gives the same bytes
    c2, s2 = oracle.mx_quantize(deq, fmt)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    # every element is the nearest value of the scaled element grid (saturating)
    grid = (E2M1 if fmt == oracle.MX_E2M1 else sorted({abs(v) for v in oracle.e4m3_decode(np.arange(0x7F))}))
    grid = np.array(grid)
    for r in range(0, 64, 7):
        for b in range(4):
            sc = 2.0 ** (int(s[r, b]) - 127)
            for i in range(32):
                v = blocks[r, b, i]
                d = np.abs(np.abs(v) / sc - grid)
                assert abs(abs(deq[r, b * 32 + i]) / sc - grid[np.argmin(d)]) <= 0 or d.min() == np.sort(d)[1]
