"""Pins for the oracle's block-Hadamard rotation (CPU only).

* H_n against scipy.linalg.hadamard (library routine), and H_n H_n^T = n I exactly;
* the binary32 butterfly equals x H_n / sqrt(n) exactly where binary32 arithmetic is
  exact (small integers), against an int64 matrix product;
* it is its own inverse there (H_n / sqrt(n) is symmetric and orthogonal);
* on bf16-valued inputs its error against the float64 product stays within the
  log2(n) * 2^-24 * sum|x| / sqrt(n) bound of a radix-2 butterfly;
* rotating both operands leaves A W^T unchanged up to that rounding;
* the rotated MXFP4 quantizer is the plain quantizer applied to the rotated values.
"""

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle.hadamard import BLOCK_SIZES, hadamard_matrix, rotate_f32


@pytest.mark.parametrize("n", [1, 2, 4, 16, 64, 256])
def test_hadamard_matrix_matches_library_and_is_orthogonal(n):
    h = hadamard_matrix(n)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(n))
    np.testing.assert_array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", BLOCK_SIZES)
def test_rotation_exact_on_small_integers(n):
    rng = np.random.default_rng(n)
    x = rng.integers(-1024, 1025, (7, 4 * n)).astype(np.int64)
    got = rotate_f32(x.astype(np.float32), n)
    # exact: x H / sqrt(n) with sqrt(n) a power of two and sums below 2^24
    xb = x.reshape(7, 4, n)
    want = (xb @ hadamard_matrix(n)).reshape(7, 4 * n).astype(np.float64) / np.sqrt(n)
    np.testing.assert_array_equal(got.astype(np.float64), want)
    back = rotate_f32(got, n)                      # involution, still exact
    np.testing.assert_array_equal(back.astype(np.float64), x.astype(np.float64))


@pytest.mark.parametrize("n", BLOCK_SIZES)
def test_rotation_error_bound_on_bf16_inputs(n):
    rng = np.random.default_rng(100 + n)
    x = rng.standard_t(3, (64, 8 * n)).astype(np.float32)
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)      # bf16-valued
    got = rotate_f32(x, n).astype(np.float64)
    xb = x.astype(np.float64).reshape(64, 8, n)
    want = (xb @ hadamard_matrix(n)).reshape(64, 8 * n) / np.sqrt(n)
    bound = np.log2(n) * 2.0 ** -24 * (np.abs(xb).sum(axis=2, keepdims=True) / np.sqrt(n))
    bound = np.broadcast_to(bound, xb.shape).reshape(64, 8 * n)
    assert np.all(np.abs(got - want) <= bound)
    # Parseval: the norm of every run is preserved up to the same rounding
    np.testing.assert_allclose(np.linalg.norm(got.reshape(64, 8, n), axis=2),
                               np.linalg.norm(xb, axis=2), rtol=1e-5)


def test_rotating_both_operands_leaves_the_product():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((16, 512)).astype(np.float32)
    w = rng.standard_normal((24, 512)).astype(np.float32)
    for n in BLOCK_SIZES:
        ra, rw = rotate_f32(a, n).astype(np.float64), rotate_f32(w, n).astype(np.float64)
        exact = a.astype(np.float64) @ w.astype(np.float64).T
        np.testing.assert_allclose(ra @ rw.T, exact, rtol=0, atol=1e-5 * (np.abs(a) @ np.abs(w).T).max())


def test_rotated_quantizer_is_quantizer_of_rotated_values():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    for rule in ("ocp", "uos"):
        c1, s1 = oracle.quantize_mxfp4_rotated(x, 64, rule)
        c2, s2 = oracle.quantize_mxfp4(rotate_f32(x, 64), rule)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(s1, s2)


def test_rotation_rejects_bad_sizes():
    with pytest.raises(ValueError):
        rotate_f32(np.zeros((1, 64), np.float32), 32)
    with pytest.raises(ValueError):
        rotate_f32(np.zeros((1, 40), np.float32), 16)
    with pytest.raises(ValueError):
        hadamard_matrix(12)


@pytest.mark.parametrize("n", [16, 64, 256])
def test_binary32_butterfly_codes_against_the_exact_rotation(n):
    """How far the binary32 butterfly (the rotation both sides compute) moves the MXFP4
    codes from those of the exact x H / sqrt(n) (float64 products and sums, exact here:
    bf16 inputs spanning < 40 binades plus 8 bits of growth fit 53 bits).  Codes may
    differ only where the exact value sits within binary32 rounding of a rounding
    boundary: then by one step of the E2M1 grid, and rarely."""
    import workloads
    u = workloads.activations_f32(256, 4096, "student_t", seed=n, name="hd-exact").view(np.uint32)
    x = (((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)).view(np.float32)
    h = oracle.hadamard_matrix(n).astype(np.float64)
    exact = (x.astype(np.float64).reshape(-1, n) @ h / np.sqrt(n)).reshape(x.shape)
    c_exact, s_exact = oracle.quantize_mxfp4(exact)
    c_b32, s_b32 = oracle.quantize_mxfp4_rotated(x, n)
    assert np.mean(s_exact != s_b32) < 1e-3
    same_scale = np.repeat(s_exact == s_b32, 16, axis=1)
    unpack = lambda c: np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[0], -1)   # noqa: E731
    ue, ub = unpack(c_exact), unpack(c_b32)
    mag = lambda c: (c & 7).astype(int)   # noqa: E731
    diff = (ue != ub) & np.repeat(s_exact == s_b32, 32, axis=1)
    frac = diff.mean()
    print(f"n={n}: {int(diff.sum())} of {diff.size} codes differ from the exact rotation ({frac:.2e})")
    assert frac < 1e-3
    assert np.all(np.abs(mag(ue[diff]) - mag(ub[diff])) <= 1)
    assert same_scale.shape[1] * 2 == ue.shape[1]
