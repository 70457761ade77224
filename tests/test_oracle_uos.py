"""Pins for the oracle's UOS scale rule (CPU only).

"MXAttention: Data-Free Optimal Scaling and Pre-Normalization Quantization for MXFP4
Attention", section "What it actually does", gives the UOS boundary constant Qmax = 7.25
for the power-of-two block scale.  The reading taken: X is the smallest power of two with
amax <= 7.25 X (the "scaling boundary"), clamped like the OCP rule.

Checked against
* exact rational brute force over every integer exponent (fractions.Fraction);
* closed forms at the boundary 7.25 * 2^j and its neighbours;
* the relation to the OCP rule through the significand of amax (1.8125 = 7.25 / 4);
* the scaled block maximum landing in (3.625, 7.25];
* a hand-worked block whose bytes and dequantized error were derived by hand.
The quality claim of the page (a lower quantization error than OCP in expectation) is
not a fixed value: it is measured (SQNR), not pinned.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.mxfp4 import block_scale_byte

QMAX = Fraction(29, 4)          # 7.25


def _brute_uos_byte(a: float) -> int:
    """Smallest integer k with a <= 7.25 * 2^k, by exact search, clamped to [-127, 127]."""
    if a == 0:
        return 0
    fa = Fraction(a)
    for k in range(-200, 200):
        if fa <= QMAX * Fraction(2) ** k:
            return min(max(k, -127), 127) + 127
    raise AssertionError("no exponent found")


def test_uos_matches_exact_brute_force():
    rng = np.random.default_rng(11)
    mags = np.ldexp(rng.uniform(1.0, 2.0, 3000), rng.integers(-140, 127, 3000))
    edges = [np.ldexp(7.25, j) for j in range(-130, 126)]
    edges += [np.nextafter(e, np.inf) for e in edges] + [np.nextafter(e, 0) for e in edges]
    edges += [np.ldexp(1.8125, j) for j in range(-128, 127)]
    a = np.concatenate([mags, np.array(edges), [0.0, 1e-45, 2.0 ** -149, np.float32(3.4028235e38)]])
    got = block_scale_byte(a, "uos")
    want = np.array([_brute_uos_byte(float(v)) for v in a], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("j", [-120, -5, 0, 1, 7, 100, 124])
def test_uos_closed_forms_at_the_boundary(j):
    at = np.ldexp(7.25, j)
    assert block_scale_byte(at, "uos") == j + 127                       # 7.25 X exactly: kept
    assert block_scale_byte(np.nextafter(at, np.inf), "uos") == j + 128  # just above: next power
    assert block_scale_byte(np.ldexp(4.0, j), "uos") == j + 127         # 4 X: same as OCP
    assert block_scale_byte(np.ldexp(4.0, j), "ocp") == j + 127


def test_uos_is_ocp_plus_one_exactly_above_significand_1_8125():
    rng = np.random.default_rng(12)
    m = rng.uniform(1.0, 2.0, 20000)
    m[:4] = [1.0, 1.8125, np.nextafter(1.8125, 2), np.nextafter(2.0, 0)]
    e = rng.integers(-120, 120, m.size)
    a = np.ldexp(m, e)
    diff = block_scale_byte(a, "uos").astype(int) - block_scale_byte(a, "ocp").astype(int)
    np.testing.assert_array_equal(diff, (m > 1.8125).astype(int))


def test_uos_scaled_maximum_lands_in_boundary_window():
    rng = np.random.default_rng(13)
    a = np.ldexp(rng.uniform(1.0, 2.0, 5000), rng.integers(-100, 100, 5000))
    k = block_scale_byte(a, "uos").astype(np.int64) - 127
    scaled = np.ldexp(a, -k)
    assert np.all(scaled <= 7.25) and np.all(scaled > 3.625)


def test_uos_hand_worked_block():
    # amax 7.5 = 1.875 * 4: UOS scale 2 (byte 0x80), OCP scale 1 (byte 0x7F).
    # UOS: 7.5/2 = 3.75 -> 4 (code 6), -3.75 -> 0xE, 1.5 -> code 3, 0.45 -> 0.5 (code 1),
    #      0.1 -> 0; packed 0xE6 0x13 0x00 ...
    # OCP: 7.5 -> 6 (saturated, code 7), -7.5 -> 0xF, 3 -> code 5, 0.9 -> 1 (code 2),
    #      0.2 -> 0; packed 0xF7 0x25 0x00 ...
    x = np.zeros((1, 32), np.float32)
    x[0, :5] = [7.5, -7.5, 3.0, 0.9, 0.2]
    cu, su = oracle.quantize_mxfp4(x, "uos")
    co, so = oracle.quantize_mxfp4(x, "ocp")
    assert su[0, 0] == 0x80 and so[0, 0] == 0x7F
    assert list(cu[0, :3]) == [0xE6, 0x13, 0x00] and not cu[0, 3:].any()
    assert list(co[0, :3]) == [0xF7, 0x25, 0x00] and not co[0, 3:].any()
    # squared error by hand: UOS 0.25+0.25+0+0.01+0.04 = 0.55, OCP 2.25+2.25+0+0.01+0.04 = 4.55
    eu = oracle.dequantize_mxfp4(cu, su, 32) - x
    eo = oracle.dequantize_mxfp4(co, so, 32) - x
    assert abs(float(np.sum(eu ** 2)) - 0.55) < 1e-6
    assert abs(float(np.sum(eo ** 2)) - 4.55) < 1e-6


def test_uos_zero_block_and_bad_rule():
    c, s = oracle.quantize_mxfp4(np.zeros((2, 64), np.float32), "uos")
    assert not c.any() and not s.any()
    with pytest.raises(ValueError):
        block_scale_byte(np.array([1.0]), "nvfp4")
