"""Pins of the oracle's OCP E4M3FN codec against torch's float8_e4m3fn (a library
implementation of the same OCP format) and against brute-force nearest search."""
import numpy as np
import torch

import oracle


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_library_for_all_codes():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # format facts: largest finite magnitude 448, smallest subnormal 2^-9
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_roundtrip_all_finite_codes():
    dec = oracle.e4m3_decode(np.arange(256))
    finite = [c for c in range(256) if not np.isnan(dec[c])]
    enc = oracle.e4m3_encode(dec[finite].astype(np.float32))
    assert np.array_equal(enc, np.array(finite, dtype=np.uint8))


def test_encode_matches_library_on_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_matches_library_on_random_fp32():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 1e-2, 100000),
                        rng.normal(0, 3.0, 100000)]).astype(np.float32)
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_is_nearest_with_ties_to_even_bruteforce():
    # all non-negative finite values of the format, decoded by the library
    table = _torch_decode_all()[:0x7F]
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(0, 448, 3000), np.exp(rng.uniform(np.log(1e-4), np.log(448), 3000))])
    x = x.astype(np.float32)
    # midpoints between neighbours are exact in fp32: they must go to the even code
    mids = ((table[1:] + table[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (table[1:] + table[:-1]) / 2)
    x = np.concatenate([x, mids])
    enc = oracle.e4m3_encode(x)
    for xi, ci in zip(x.astype(np.float64), enc):
        dist = np.abs(table - xi)
        best = np.flatnonzero(dist == dist.min())
        want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        assert ci == want, (xi, ci, want)


def test_encode_saturation_signed_zero_and_tiny():
    e = lambda v: int(oracle.e4m3_encode(np.array([v], dtype=np.float32))[0])
    assert e(448.0) == 0x7E and e(449.0) == 0x7E and e(464.0) == 0x7E and e(1e30) == 0x7E
    assert e(-500.0) == 0xFE
    assert e(0.0) == 0x00 and e(-0.0) == 0x80
    assert e(2.0 ** -10) == 0x00            # tie between 0 and 2^-9 goes to the even code 0
    assert e(-(2.0 ** -11)) == 0x80         # rounds to zero and keeps the sign
    assert e(3 * 2.0 ** -10) == 0x02        # tie between 2^-9 and 2*2^-9 -> even code 2
    assert e(2.0 ** -6 - 2.0 ** -12) == 0x08  # rounds up into the smallest normal
