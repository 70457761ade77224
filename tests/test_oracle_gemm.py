"""Pins for the oracle's GEMMs and SQNR (CPU only).

* exact rational brute force (fractions.Fraction) on tiny non-square shapes, written from
  the literal E2M1 values -- catches transposed operands, wrong scale indices, dropped
  block terms and sign errors;
* special cases: a one-hot weight row reduces the GEMM to one dequantized activation
  column; all-zero activations give exactly 0; a power-of-two activation scale scales the
  output exactly; permuting whole K-blocks identically in A and W changes nothing;
* the error-budget helper flags a planted error;
* SQNR closed forms.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import gemm, sqnr
from oracle.mxfp4 import unpack_codes

E2M1_LITERAL = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _e2m1_frac(code: int) -> Fraction:
    v = E2M1_LITERAL[code & 7]
    return -v if code & 8 else v


def _e4m3_frac(code: int) -> Fraction:
    e, m = (code >> 3) & 0xF, code & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


def _pow2(e: int) -> Fraction:
    return Fraction(2) ** e


def _random_mx(rng, R, K, lo=120, hi=135):
    codes = rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(R, K // 32), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("M,N,K", [(3, 5, 32), (7, 2, 64), (8, 8, 128), (1, 6, 96)])
def test_w4a4_equals_rational_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    ac, asc = _random_mx(rng, M, K)
    wc, wsc = _random_mx(rng, N, K)
    out, tot = oracle.gemm_w4a4(ac, asc, wc, wsc, K)
    A, W = unpack_codes(ac, K), unpack_codes(wc, K)
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            t = Fraction(0)
            for k in range(K):
                b = k // 32
                p = _e2m1_frac(int(A[m, k])) * _e2m1_frac(int(W[n, k])) * \
                    _pow2(int(asc[m, b]) - 127) * _pow2(int(wsc[n, b]) - 127)
                s += p
                t += abs(p)
            assert Fraction(float(out[m, n])) == s
            assert Fraction(float(tot[m, n])) == t


@pytest.mark.parametrize("M,N,K", [(4, 3, 64), (2, 7, 128)])
def test_w4a8_equals_rational_brute_force(M, N, K):
    rng = np.random.default_rng(11 + M + N + K)
    a8 = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    a8[(a8 & 0x7F) == 0x7F] = 0x3C            # no NaN codes
    wc, wsc = _random_mx(rng, N, K)
    s_a = np.float32(0.0371)
    out, tot = oracle.gemm_w4a8(a8, s_a, wc, wsc, K)
    W = unpack_codes(wc, K)
    sa = Fraction(float(s_a))
    for m in range(M):
        for n in range(N):
            s = sum(_e4m3_frac(int(a8[m, k])) * _e2m1_frac(int(W[n, k])) *
                    _pow2(int(wsc[n, k // 32]) - 127) for k in range(K))
            # s_a multiplies one exactly accumulated float64 sum: one rounding
            assert abs(Fraction(float(out[m, n])) - sa * s) <= abs(sa * s) * Fraction(1, 2 ** 52)


def test_bf16_reference_equals_rational_brute_force():
    rng = np.random.default_rng(12)
    a = rng.integers(0, 2 ** 16, size=(3, 40), dtype=np.uint32).astype(np.uint16)
    w = rng.integers(0, 2 ** 16, size=(5, 40), dtype=np.uint32).astype(np.uint16)
    # keep finite values in a modest exponent range so the float64 sum is exact
    a = (a & 0x80FF) | 0x3C00
    w = (w & 0x80FF) | 0x3F00
    out, _ = oracle.gemm_bf16(a, w)
    A, W = oracle.bf16_bits_to_f64(a), oracle.bf16_bits_to_f64(w)
    for m in range(3):
        for n in range(5):
            s = sum(Fraction(float(A[m, k])) * Fraction(float(W[n, k])) for k in range(40))
            assert Fraction(float(out[m, n])) == s


def test_one_hot_weight_row_selects_an_activation_column():
    rng = np.random.default_rng(13)
    K = 128
    ac, asc = _random_mx(rng, 9, K)
    wc = np.zeros((4, K // 2), np.uint8)
    wsc = np.full((4, K // 32), 127, np.uint8)
    for n, k0 in enumerate([0, 33, 70, 127]):
        wc[n, k0 // 2] = 0x2 << (4 * (k0 % 2))      # e2m1 code 2 == 1.0
    out, _ = oracle.gemm_w4a4(ac, asc, wc, wsc, K)
    deq = oracle.dequantize_mxfp4(ac, asc, K)
    for n, k0 in enumerate([0, 33, 70, 127]):
        np.testing.assert_array_equal(out[:, n], deq[:, k0])


def test_zero_activations_give_exact_zero():
    rng = np.random.default_rng(14)
    wc, wsc = _random_mx(rng, 6, 64)
    out, tot = oracle.gemm_w4a4(np.zeros((3, 32), np.uint8), np.full((3, 2), 140, np.uint8),
                                wc, wsc, 64)
    assert np.all(out == 0) and np.all(tot == 0)


def test_power_of_two_activation_scale_is_exact():
    rng = np.random.default_rng(15)
    ac, asc = _random_mx(rng, 5, 128)
    wc, wsc = _random_mx(rng, 4, 128)
    o1, _ = oracle.gemm_w4a4(ac, asc, wc, wsc, 128)
    o2, _ = oracle.gemm_w4a4(ac, asc + 3, wc, wsc, 128)
    np.testing.assert_array_equal(o2, o1 * 8)


def test_block_permutation_invariance():
    rng = np.random.default_rng(16)
    K = 128
    ac, asc = _random_mx(rng, 5, K)
    wc, wsc = _random_mx(rng, 4, K)
    perm = [2, 0, 3, 1]
    pc = lambda c: np.concatenate([c[:, 16 * p:16 * p + 16] for p in perm], axis=1)
    o1, t1 = oracle.gemm_w4a4(ac, asc, wc, wsc, K)
    o2, t2 = oracle.gemm_w4a4(pc(ac), asc[:, perm], pc(wc), wsc[:, perm], K)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12 * np.max(t1))
    np.testing.assert_allclose(t2, t1, rtol=1e-15)


def test_tolerance_flags_a_planted_error():
    rng = np.random.default_rng(17)
    ac, asc = _random_mx(rng, 16, 256)
    wc, wsc = _random_mx(rng, 8, 256)
    out, tot = oracle.gemm_w4a4(ac, asc, wc, wsc, 256)
    bits = gemm.to_bf16(out)
    ok, _, _ = oracle.within_tolerance(bits, out, tot)
    assert ok.all()
    bad = bits.copy()
    bad[3, 4] = oracle.f64_to_bf16_bits(np.array([out[3, 4] * 1.05 + 1e-3 * tot[3, 4]]))[0]
    ok, _, _ = oracle.within_tolerance(bad, out, tot)
    assert not ok[3, 4] and ok.sum() == ok.size - 1


def _bf(x):
    return oracle.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_sqnr_closed_forms():
    ref = np.array([[1.0, -2.0, 3.5], [0.25, 8.0, -1.0]])
    _, _, d = sqnr.sqnr_db(_bf(ref), _bf(ref / 2))
    assert abs(d - 20 * math.log10(2)) < 1e-12
    _, _, d = sqnr.sqnr_db(_bf(ref), _bf(np.zeros_like(ref)))
    assert abs(d) < 1e-12
    _, _, d = sqnr.sqnr_db(_bf(ref), _bf(-ref))
    assert abs(d + 20 * math.log10(2)) < 1e-12
    s, n, d = sqnr.sqnr_db(_bf(ref), _bf(ref))
    assert n == 0 and d == math.inf
    assert math.isnan(sqnr.sqnr_db(_bf(np.zeros(3)), _bf(np.zeros(3)))[2])
    s, n, d = sqnr.sqnr_db(_bf([3.0, 4.0]), _bf([3.0, 3.0]))
    assert s == 25.0 and n == 1.0 and abs(d - 10 * math.log10(25)) < 1e-12


def _bound_case(ref_value, T):
    """Oracle output `ref_value` (a bf16 value) with total T; returns (out, T, ref bits, ulp)."""
    out = np.array([[ref_value]], dtype=np.float64)
    tot = np.array([[T]], dtype=np.float64)
    rb = oracle.f64_to_bf16_bits(out)
    return out, tot, rb, float(oracle.bf16_ulp(oracle.bf16_bits_to_f64(rb))[0, 0])


@pytest.mark.parametrize("ref_value,T", [(1.0, 3000.0), (-0.0625, 400.0), (12.0, 2.5e5)])
def test_tolerance_constant_is_1e5_at_the_boundary(ref_value, T):
    """The bound is 1e-5 * T + 1 ulp exactly: a GPU value whose error lands just inside it
    passes and the next bf16 value outside fails; errors between a 10x tighter and the
    stated bound pass, errors between the stated bound and a 10x looser one fail -- so
    both a 1e-6 and a 1e-4 constant would break this test."""
    out, tot, rb, ulp = _bound_case(ref_value, T)
    bound = 1e-5 * T + ulp
    ref = float(oracle.bf16_bits_to_f64(rb)[0, 0])
    # bf16 values on the grid above ref: the last one within the bound, the first outside
    vals = ref + ulp * np.arange(0, 4 * int(bound / ulp) + 8)
    bits = oracle.f64_to_bf16_bits(vals)
    back = oracle.bf16_bits_to_f64(bits)
    inside = back[np.abs(back - ref) <= bound].max()
    outside = back[np.abs(back - ref) > bound].min()
    for v, expect in ((inside, True), (outside, False)):
        ok, err, b = oracle.within_tolerance(oracle.f64_to_bf16_bits(np.array([[v]])), out, tot)
        assert bool(ok[0, 0]) is expect and abs(b[0, 0] - bound) <= 1e-12 * bound, (v, expect, err, b)
    # between 1e-6 T + ulp and 1e-5 T + ulp: accepted; between 1e-5 T + ulp and 1e-4 T + ulp: rejected
    mid_lo = ref + 0.5 * (1e-6 * T + 1e-5 * T) + ulp
    mid_hi = ref + 0.5 * (1e-5 * T + 1e-4 * T) + ulp
    for v, expect in ((mid_lo, True), (mid_hi, False)):
        vb = oracle.f64_to_bf16_bits(np.array([[v]]))
        err = abs(float(oracle.bf16_bits_to_f64(vb)[0, 0]) - ref)
        if expect:
            assert err <= bound
        else:
            assert err > bound and err <= 1e-4 * T + 2 * ulp
        ok, _, _ = oracle.within_tolerance(vb, out, tot)
        assert bool(ok[0, 0]) is expect
