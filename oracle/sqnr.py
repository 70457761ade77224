"""Whole-output SQNR against the bf16 reference (oracle; test infrastructure only).

"AMD Quark adds native W4A8 mixed-precision for Wan2.2 video generation on MI350",
section "Quark quantization pipeline and mixed-precision selection": each transformer
block is scored by the SQNR of its whole output against BF16.

Reading: one scalar per (GEMM output, mode) -- the layer's entire M x N output stands in
for the block output, not one value per 32-element MX block:
    S = sum ref^2,  N = sum (ref - test)^2,  SQNR = 10 * log10(S / N) dB,
in float64 over the bf16 values widened exactly.  N == 0 gives +inf dB; S == N == 0
gives NaN.
"""

import math

import numpy as np

from .formats import bf16_bits_to_f64


def sqnr_db(ref_bf16_bits, test_bf16_bits):
    """Return (S, N, dB) for two equally shaped arrays of bf16 bit patterns."""
    ref = bf16_bits_to_f64(ref_bf16_bits)
    test = bf16_bits_to_f64(test_bf16_bits)
    if ref.shape != test.shape:
        raise ValueError("sqnr_db: shape mismatch")
    s = float(np.sum(ref * ref))
    n = float(np.sum((ref - test) ** 2))
    if n == 0.0:
        db = math.nan if s == 0.0 else math.inf
    elif s == 0.0:
        db = -math.inf
    else:
        db = 10.0 * math.log10(s / n)
    return s, n, db
