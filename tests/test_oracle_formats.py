"""Pins for the oracle's format tables and bf16 rounding (CPU only).

Each table is checked against something other than the oracle itself: torch's own
float8_e8m0fnu / float8_e4m3fn / bfloat16 conversions (library routines), exact rational
brute force, or the structural properties that determine the E2M1 value set uniquely.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats


def test_e2m1_table_is_forced_by_its_structure():
    """The 16 E2M1 values follow from: code 0 is +0, the smallest positive value is 0.5
    (a 1-bit subnormal with exponent bias 1), spacing below 2 is uniform, each higher
    binade doubles, the top magnitude is 6 (the MX saturation point), and codes 8..15
    are the negatives of 0..7."""
    t = formats.E2M1_TABLE
    assert len(t) == 16
    mags = t[:8]
    assert mags[0] == 0.0 and not math.copysign(1.0, mags[0]) < 0
    assert mags[1] == 0.5
    # uniform spacing over the subnormal range and the first normal binade
    assert np.all(np.diff(mags[:5]) == 0.5)
    # each further binade doubles: value(c + 2) == 2 * value(c) for normal codes
    for c in range(2, 6):
        assert mags[c + 2] == 2 * mags[c]
    assert mags[7] == 6.0
    assert np.all(np.diff(mags) > 0)
    for c in range(8):
        assert t[8 + c] == -mags[c]
        assert math.copysign(1.0, t[8 + c]) < 0
    assert sorted(set(mags.tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()
    got = oracle.e8m0_decode(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = oracle.e4m3_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    np.testing.assert_array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert oracle.E4M3_MAX == 448.0


def _bf16_bits_torch(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_binary32_inputs():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # add exact ties (low 16 bits == 0x8000) and values near the overflow edge
    ties = (rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    edge = np.array([3.3895314e38, 3.3961775e38, -3.3961775e38, 1e-45, -1e-45, 0.0, -0.0],
                    dtype=np.float32)
    x = np.concatenate([x, ties, edge])
    got = oracle.f64_to_bf16_bits(x.astype(np.float64))
    ref = _bf16_bits_torch(x)
    np.testing.assert_array_equal(got, ref)


def _nearest_bf16_fraction(v: Fraction) -> Fraction:
    """Brute force: nearest bf16 to an exact rational (ties to even mantissa)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    lo = (a // q) * q
    hi = lo + q
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    return r if v > 0 else -r


def test_bf16_rounding_of_float64_matches_exact_brute_force():
    rng = np.random.default_rng(2)
    vals = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000)),
        # exact midpoints between adjacent bf16 values, and a hair off them
        (np.arange(1, 500) * 2 + 1) * 2.0 ** -9,
        (np.arange(1, 500) * 2 + 1) * 2.0 ** -9 * (1 + 2.0 ** -40),
        (np.arange(1, 200) * 2 + 1) * 2.0 ** -134,
    ])
    got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(vals))
    for v, g in zip(vals, got):
        assert Fraction(float(g)) == _nearest_bf16_fraction(Fraction(float(v))), v


def test_bf16_ulp_closed_form():
    assert oracle.bf16_ulp(1.0) == 2.0 ** -7
    assert oracle.bf16_ulp(1.99) == 2.0 ** -7
    assert oracle.bf16_ulp(-2.0) == 2.0 ** -6
    assert oracle.bf16_ulp(0.0) == 2.0 ** -133
    assert oracle.bf16_ulp(2.0 ** -127) == 2.0 ** -133
    assert oracle.bf16_ulp(2.0 ** -126) == 2.0 ** -133


def test_bf16_widening_is_exact():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(t))
    fin = ~np.isnan(t)
    np.testing.assert_array_equal(got[fin], t[fin])


@pytest.mark.parametrize("x", [1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** 128, -(2.0 ** 129)])
def test_bf16_rounding_special_points(x):
    got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array([x])))[0]
    if abs(x) >= 2.0 ** 128:
        assert np.isinf(got) and np.sign(got) == np.sign(x)
    else:
        assert Fraction(float(got)) == _nearest_bf16_fraction(Fraction(x))
