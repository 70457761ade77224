"""The oracle against the format values the source pages print (tests/golden/page_values.txt).

Each value is checked through the oracle's behaviour, not by comparing a constant:
blocks are 32 elements (a change in one block moves only that block's scale), elements
are 4 bits, codes plus scales take 4.25 bits per element, the scale is an exact power of
two, the UOS boundary is 7.25 and the W4A8 activations are E4M3 (largest finite 448).
"""

import os

import numpy as np

import oracle
from oracle.mxfp4 import block_scale_byte

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.txt")


def _values():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = v
    return out


V = _values()


def test_block_size_is_the_unit_of_the_shared_scale():
    n = int(V["block_size"])
    assert n == int(V["scale_block_size"]) == 32
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 8 * n)).astype(np.float32)
    _, s0 = oracle.quantize_mxfp4(x)
    assert s0.shape == (3, 8)
    for b in range(8):
        y = x.copy()
        y[1, b * n + 5] = 1000.0                          # one large element in block b of row 1
        _, s1 = oracle.quantize_mxfp4(y)
        changed = np.argwhere(s1 != s0)
        assert changed.tolist() == [[1, b]]


def test_elements_are_four_bits_and_storage_is_four_and_a_quarter():
    bits, n = int(V["element_bits"]), int(V["block_size"])
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 4 * n)).astype(np.float32)
    codes, scales = oracle.quantize_mxfp4(x)
    assert codes.shape[1] * 8 == x.shape[1] * bits          # two 4-bit codes per byte
    lo, hi = codes & 0xF, codes >> 4
    assert lo.max() < 1 << bits and hi.max() < 1 << bits
    total_bits = (codes.nbytes + scales.nbytes) * 8 / x.size
    assert total_bits == bits + 8 / n == 4.25
    assert 16 / bits == int(V["bf16_footprint_ratio"])


def test_scale_is_a_power_of_two_with_no_mantissa():
    assert int(V["scale_mantissa_bits"]) == 0
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-60, 60, (64, 1)))).astype(np.float32)
    codes, scales = oracle.quantize_mxfp4(x)
    ones = np.full_like(codes, 0x22)                       # every element the E2M1 code of 1.0
    deq = oracle.dequantize_mxfp4(ones, scales, 32)        # = the block scale itself
    m, e = np.frexp(deq[:, 0])
    assert np.all(m == 0.5)                                # exact powers of two
    np.testing.assert_array_equal(e - 1, scales[:, 0].astype(int) - 127)


def test_uos_boundary():
    qmax = float(V["uos_qmax"])
    assert qmax == 7.25
    j = np.arange(-20, 21)
    at = np.ldexp(qmax, j)
    # a block maximum exactly at the boundary keeps scale 2^j; just above it moves up one
    np.testing.assert_array_equal(block_scale_byte(at, "uos").astype(int) - 127, j)
    np.testing.assert_array_equal(block_scale_byte(np.nextafter(at, np.inf), "uos").astype(int) - 127, j + 1)


def test_w4a8_activations_are_e4m3():
    assert V["w4a8_activation_format"] == "e4m3"
    # E4M3: 4 exponent bits (bias 7), 3 mantissa bits, largest finite 1.75 * 2^8 = 448
    q = oracle.quantize_fp8(np.array([[1e9, -1e9, 448.0, 1.0]], np.float32), 1.0)
    vals = oracle.e4m3_decode(q)
    np.testing.assert_array_equal(vals, [[448.0, -448.0, 448.0, 1.0]])
