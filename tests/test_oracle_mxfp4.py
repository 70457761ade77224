"""Pins for the oracle's MXFP4 quantizer (CPU only).

The quantizer is checked against
* the E2M1 rounding written through a library round-half-even (np.rint) on each uniform
  stretch of the grid, over dense grids and every midpoint;
* exact rational brute force (nearest grid point, ties to the even code);
* the scale byte read straight off the binary32 exponent field, s = max(E(amax) - 2, 0);
* hand-worked blocks derived from the OCP MX rule X = 2^(floor(log2 amax) - 2);
* invariants: idempotence of quantize(dequantize(quantize(x))), sign symmetry and
  power-of-two equivariance.
"""

from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from oracle.mxfp4 import unpack_codes

E2M1_LITERAL = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _rint_code(a: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code through np.rint (round half to even) on the three uniform
    stretches of the grid: step 1/2 below 2, step 1 on [2, 4), step 2 from 4 up."""
    a = np.asarray(a, dtype=np.float64)
    c = np.where(a < 2, np.rint(2 * a),
                 np.where(a < 4, np.rint(a) + 2, np.minimum(np.rint(a / 2) + 4, 7)))
    return c.astype(np.uint8)


def test_encode_matches_library_rint_on_dense_grid():
    a = np.concatenate([np.arange(0, 12 * 4096 + 1) / 4096.0,      # includes every midpoint
                        np.random.default_rng(3).uniform(0, 10, 100_000),
                        [1e30, 7.0, 6.5, 6.0, 5.0 + 2 ** -40, 5.0 - 2 ** -40]])
    got = oracle.e2m1_encode(a)
    np.testing.assert_array_equal(got, _rint_code(a))
    np.testing.assert_array_equal(oracle.e2m1_encode(-a), _rint_code(a) | 8)


def _brute_code(v: Fraction) -> int:
    a = abs(v)
    best = min(range(8), key=lambda c: (abs(a - E2M1_LITERAL[c]), c % 2))
    return best | (8 if v < 0 else 0)


def test_encode_matches_rational_brute_force_at_midpoints():
    pts = []
    for i in range(7):
        mid = (E2M1_LITERAL[i] + E2M1_LITERAL[i + 1]) / 2
        for d in (Fraction(0), Fraction(1, 2 ** 30), -Fraction(1, 2 ** 30)):
            pts.append(mid + d)
    pts += [Fraction(25, 4), Fraction(100), Fraction(0)]
    for p in pts:
        for s in (1, -1):
            v = s * p
            if v == 0:
                continue
            assert int(oracle.e2m1_encode(np.array([float(v)]))[0]) == _brute_code(v), v


def _scale_from_bits(amax32: np.ndarray) -> np.ndarray:
    e = (amax32.astype(np.float32).view(np.uint32) >> 23) & 0xFF
    return np.maximum(e.astype(np.int64) - 2, 0).astype(np.uint8)


def test_scale_byte_matches_exponent_field_closed_form():
    rng = np.random.default_rng(4)
    u = rng.integers(1, 0x7F800000, size=300_000, dtype=np.int64).astype(np.uint32)
    amax = u.view(np.float32)                                 # every positive finite binade
    got = oracle.block_scale_byte(amax.astype(np.float64))
    np.testing.assert_array_equal(got, _scale_from_bits(amax))


@pytest.mark.parametrize("amax,byte", [
    (0.0, 0x00),
    (4.0, 127), (np.nextafter(np.float32(4.0), np.float32(0)), 126), (8.0, 128),
    (1.0, 125), (2.0 ** -124, 1), (2.0 ** -125, 0), (2.0 ** -149, 0),
    (float(np.finfo(np.float32).max), 0xFC), (2.0 ** 127, 0xFC), (2.0 ** 126, 0xFB),
])
def test_scale_byte_edges(amax, byte):
    assert int(oracle.block_scale_byte(np.array([amax], dtype=np.float64))[0]) == byte


def _q(block):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, : len(block)] = np.asarray(block, dtype=np.float32)
    codes, scales = oracle.quantize_mxfp4(x)
    return bytes(codes[0].tolist()), int(scales[0, 0])


def test_hand_worked_all_zero_block():
    assert _q([]) == (bytes(16), 0x00)
    assert _q([-0.0] * 32) == (bytes([0x88] * 16), 0x00)


def test_hand_worked_exactly_representable_block():
    # x_i = e2m1(i mod 16) * 8: amax = 48, floor(log2 48) = 5, scale 2^3 -> byte 0x82;
    # every element divides back onto its own code, so codes 0..F repeat twice.
    vals = [float(v) * 8 for v in E2M1_LITERAL] + [-float(v) * 8 for v in E2M1_LITERAL]
    vals[8] = -0.0
    codes, s = _q(vals * 2)
    assert s == 0x82
    assert codes == bytes([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2)
    x = np.array([vals * 2], dtype=np.float32)
    c, sc = oracle.quantize_mxfp4(x)
    np.testing.assert_array_equal(oracle.dequantize_mxfp4(c, sc, 32), x.astype(np.float64))


def test_hand_worked_saturation_and_ties_block():
    # amax 7.99 -> floor(log2) = 2 -> scale 2^0 (byte 0x7F); 7.99 and -7 saturate to +-6;
    # 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25 are ties that go to the even code;
    # 5.0001 is nearer 6 than 4.
    blk = [7.99, -7, 5, -5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, -0.25, 5.0001]
    codes, s = _q(blk)
    assert s == 0x7F
    assert codes == bytes([0xF7, 0xE6, 0x46, 0x24, 0x02, 0x78] + [0] * 10)


@pytest.mark.parametrize("amax,code", [
    (2.0 ** -130, 0x0),        # scale clamps at 2^-127: 2^-3 rounds to 0
    (1.5 * 2.0 ** -125, 0x7),  # -> 6
    (2.0 ** -126, 0x4),        # -> 2
    (1.5 * 2.0 ** -127, 0x3),  # binary32 subnormal input -> 1.5
])
def test_hand_worked_subnormal_scale_blocks(amax, code):
    codes, s = _q([amax])
    assert s == 0x00
    assert codes[0] == code and codes[1:] == bytes(15)


_mags = st.one_of(
    st.just(0.0),
    st.builds(lambda m, e: m * 2.0 ** e, st.floats(0.5, 1.0), st.integers(-135, 100)),
)
_blocks = hnp.arrays(np.float64, (3, 64), elements=st.builds(
    lambda m, s: m if s else -m, _mags, st.booleans()))


def _as_f32_exact(x):
    return x.astype(np.float32).astype(np.float64)


@settings(max_examples=200, deadline=None)
@given(_blocks)
def test_idempotent_requantization(x):
    x = _as_f32_exact(x)
    c1, s1 = oracle.quantize_mxfp4(x)
    y = oracle.dequantize_mxfp4(c1, s1, 64)
    c2, s2 = oracle.quantize_mxfp4(y)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)


@settings(max_examples=200, deadline=None)
@given(_blocks)
def test_sign_symmetry(x):
    x = _as_f32_exact(x)
    c1, s1 = oracle.quantize_mxfp4(x)
    c2, s2 = oracle.quantize_mxfp4(-x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c2, c1 ^ 0x88)


@settings(max_examples=200, deadline=None)
@given(_blocks, st.integers(-20, 20))
def test_power_of_two_equivariance(x, j):
    x = _as_f32_exact(x)
    c1, s1 = oracle.quantize_mxfp4(x)
    c2, s2 = oracle.quantize_mxfp4(np.ldexp(x, j))
    s1i, s2i = s1.astype(int), s2.astype(int)
    blocks = np.abs(x).reshape(3, 2, 32).max(axis=2)
    # only blocks whose scale is unclamped before and after the shift
    free = (s1i > 0) & (s1i + j > 0) & (s1i + j <= 254) & (blocks > 0)
    assert np.all(s2i[free] == s1i[free] + j)
    cu1 = unpack_codes(c1, 64).reshape(3, 2, 32)
    cu2 = unpack_codes(c2, 64).reshape(3, 2, 32)
    np.testing.assert_array_equal(cu1[free], cu2[free])


def test_quantize_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.zeros((2, 48), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.full((1, 32), np.inf, np.float32))


def test_nibble_order_low_is_even_element():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0       # code 7 at element 0
    x[0, 1] = -4.0      # code 0xE at element 1
    c, s = oracle.quantize_mxfp4(x)
    assert s[0, 0] == 127 and c[0, 0] == 0xE7
