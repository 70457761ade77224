"""Pins for the oracle's static FP8 E4M3 path (CPU only): torch's float8_e4m3fn
conversion (round to nearest even, no saturation) is the library reference inside the
finite range; the saturation and static-scale readings are pinned by closed forms."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_inside_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, 200_000),
        rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 8, 200_000)),
        # every midpoint between adjacent finite E4M3 values, both signs
        (oracle.formats.E4M3_TABLE[:0x7E] + oracle.formats.E4M3_TABLE[1:0x7F]) / 2,
        -(oracle.formats.E4M3_TABLE[:0x7E] + oracle.formats.E4M3_TABLE[1:0x7F]) / 2,
        [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 448.0, -448.0],
    ]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(x.astype(np.float64)), _torch_e4m3(x))


@pytest.mark.parametrize("v,code", [(464.0, 0x7E), (480.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E),
                                    (-500.0, 0xFE), (-np.inf, 0xFE)])
def test_encode_saturates_at_448(v, code):
    assert int(oracle.e4m3_encode(np.array([v]))[0]) == code


def test_decode_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)


def test_static_scales_are_correctly_rounded_quotients():
    rng = np.random.default_rng(6)
    for amax in np.concatenate([rng.uniform(0.1, 1000, 300), [448.0, 1.0, 3e-5, 7e20]]):
        a32 = np.float32(amax)
        s_a, inv_s = oracle.fp8_static_scales(a32)
        for got, exact in ((s_a, Fraction(float(a32)) / 448), (inv_s, 448 / Fraction(float(a32)))):
            lo = np.nextafter(got, np.float32(-np.inf))
            hi = np.nextafter(got, np.float32(np.inf))
            err = abs(Fraction(float(got)) - exact)
            assert err <= abs(Fraction(float(lo)) - exact)
            assert err <= abs(Fraction(float(hi)) - exact)


def test_quantize_is_one_binary32_multiply_then_e4m3():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(50_000) * 3).astype(np.float32)
    amax = float(np.max(np.abs(x)))
    _, inv_s = oracle.fp8_static_scales(amax)
    y = (torch.from_numpy(x) * torch.tensor(inv_s, dtype=torch.float32))
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()   # |y| <= 448(1 + 2^-23)
    np.testing.assert_array_equal(oracle.quantize_fp8(x, inv_s), ref)


def test_static_scale_maps_amax_to_top_code():
    x = np.array([-3.25, 1.0, 0.5], np.float32)
    _, inv_s = oracle.fp8_static_scales(3.25)
    q = oracle.quantize_fp8(x, inv_s)
    assert q[0] == 0xFE


def _torch_qdq(q: np.ndarray, s_a) -> np.ndarray:
    """The same QDQ step through torch's own conversions (a library reference): E4M3 ->
    binary32, one binary32 multiply, binary32 -> bfloat16 (round to nearest even)."""
    f = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(s_a, dtype=torch.float32)
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("s_a", [1.0, 0.0078125, 2.2321430606098147e-06, 0.3171, 7.3e-3, 1e30, -0.5, 2.0 ** -130])
def test_dequantize_fp8_matches_torch_on_every_code(s_a):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    s = np.float32(s_a)
    np.testing.assert_array_equal(oracle.dequantize_fp8(codes, s), _torch_qdq(codes, s))


def test_dequantize_fp8_nan_codes_and_exact_cases():
    got = oracle.dequantize_fp8(np.array([0x7F, 0xFF], np.uint8), np.float32(1.0))
    assert list(got) == [0x7FC0, 0xFFC0]
    # with s_a = 1 every E4M3 value is a bf16 value (4 significant bits): exact
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = oracle.bf16_bits_to_f64(oracle.dequantize_fp8(codes, np.float32(1.0)))
    np.testing.assert_array_equal(back, oracle.e4m3_decode(codes))


def test_dequantize_fp8_double_rounding_is_the_stated_reading():
    """The product is rounded to binary32 first, then to bf16.  Construct products that
    lie within half a binary32 ulp of a bf16 midpoint (code 0x3F = 1.875, scales
    s = fl32(m / 1.875) for midpoints m in [1, 2)): the binary32 rounding lands on the
    midpoint and the tie goes to even, where rounding the exact product once would go
    to its side.  The oracle must take the two-step value, and such cases must exist."""
    from fractions import Fraction
    differs = 0
    for k in range(128):
        m = Fraction(2 * (128 + k) + 1, 256)                      # bf16 midpoint in [1, 2)
        s = np.float32(float(m / Fraction(15, 8)))
        exact = Fraction(15, 8) * Fraction(float(s))
        two = oracle.dequantize_fp8(np.array([0x3F], np.uint8), s)[0]
        step = oracle.f64_to_bf16_bits(np.array([float(np.float32(float(exact)))]))[0]
        assert two == step
        # rounding the exact product once: nearest bf16 on its own side of m
        once = oracle.f64_to_bf16_bits(np.array([float(exact)]))[0] if exact != m else step
        differs += int(once != two)
    assert differs > 0
