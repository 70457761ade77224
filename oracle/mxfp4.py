"""MXFP4 block quantization (oracle; test infrastructure only).

What is computed (pages + the OCP MX rule):

1. The row of K values is split into K/32 blocks of 32 consecutive elements; every
   block shares one scale ("AMD Quark: 1.92x faster FLUX.1-dev with MXFP4 on Instinct
   MI350", section "What is MXFP4").
2. The scale is a power of two stored as an E8M0 byte ("MXAttention ...", section "What
   it actually does").  Rule: X = 2^(floor(log2(amax)) - 2), amax = max |x| over the
   block, i.e. the block maximum lands in [4, 8) after scaling, the top binade of E2M1.
   floor(log2) is taken exactly (frexp), never from a rounded log2.
   Reading (clamp): the exponent is clamped to [-127, 127], the E8M0 range without NaN.
   Reading (all-zero block): log2(0) = -inf clamps to -127, i.e. scale byte 0x00.
3. Each element is divided by X (exact: X is a power of two) and rounded to the nearest
   E2M1 magnitude, ties to the even code (mantissa bit 0); magnitudes past the top of
   the grid go to 6, which is the saturation at +-6 ("MXAttention ...", TL;DR: a
   power-of-two scale trades clipping of large values against underflow of small
   ones).  Reading (sign): the sign bit is copied from the input, so -0.0 and small
   negatives that round to zero encode as 0x8.
4. Packing (reading; layout is this library's contract): row-major, K contiguous; byte j
   of a row holds element 2j in the low nibble and 2j+1 in the high nibble.  Scales are
   row-major bytes, one per block.

Optional UOS scale rule ("MXAttention ...", section "What it actually does": Universal
Optimal Scaling, a data-free scaling boundary Qmax = 7.25).  Reading: the scale is the
smallest power of two X with amax <= Qmax * X, i.e. the block maximum lands in
(3.625, 7.25] after scaling and values above 6 but within 7.25 X saturate to 6; the same
exponent clamp and all-zero rule apply.  The page gives the constant, not the formula;
this is the plainest reading of "scaling boundary".

Non-finite inputs are outside the contract; the oracle raises on them.
"""

import numpy as np

from .formats import E2M1_MAGNITUDES, e2m1_decode, e8m0_decode

BLOCK = 32
UOS_QMAX = 7.25


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive finite float64 a, exactly (frexp: a = f*2^e, f in [0.5,1))."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def block_scale_byte(amax, rule: str = "ocp") -> np.ndarray:
    """E8M0 byte of the MX scale for block maxima ``amax`` (float64 >= 0, finite).

    rule "ocp": k = floor(log2 amax) - 2.
    rule "uos": k = the smallest integer with amax <= 7.25 * 2^k.  With e = floor(log2
    amax) the candidates are e-3 .. e-1 (7.25 * 2^(e-3) < 2^e <= amax < 2^(e+1) <
    7.25 * 2^(e-1)); each comparison is exact in float64 (7.25 * 2^k is a dyadic rational).
    Both: k clamped to [-127, 127]; byte = k + 127; amax == 0 -> byte 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    if not np.all(np.isfinite(a)) or np.any(a < 0):
        raise ValueError("block_scale_byte: amax must be finite and non-negative")
    safe = np.where(a > 0, a, 1.0)
    e = _floor_log2(safe)
    if rule == "ocp":
        k = e - 2
    elif rule == "uos":
        k = e - 1                                   # always satisfies the bound
        for cand in (e - 2, e - 3):                 # the smallest candidate that still does
            k = np.where(safe <= np.ldexp(UOS_QMAX, cand), cand, k)
    else:
        raise ValueError("block_scale_byte: rule must be 'ocp' or 'uos'")
    k = np.where(a > 0, k, -127)
    k = np.clip(k, -127, 127)
    return (k + 127).astype(np.uint8)


def e2m1_encode(v) -> np.ndarray:
    """Round already-scaled values v to E2M1 codes (uint8, 0..15).

    Nearest grid magnitude, ties to the even code; beyond the grid the nearest point is
    the top magnitude 6 (saturation).  The sign bit comes from v's sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    grid = E2M1_MAGNITUDES                       # ascending 0, 0.5, ..., 6
    hi = np.searchsorted(grid, a, side="left")   # first grid point >= a
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = np.abs(a - grid[lo])
    d_hi = np.abs(grid[hi] - a)
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    # at or past the top grid point the nearest point is the top one (saturation);
    # decided by comparison, not by float distances that lose precision far out
    pick = np.where(a >= grid[-1], len(grid) - 1, pick)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(3)
    return pick.astype(np.uint8) | sign


def quantize_mxfp4(x, rule: str = "ocp"):
    """MXFP4-quantize a 2-D array along its last axis (K).

    ``x``: float32 or float64 array [R, K] whose values are binary32-representable
    (bf16 inputs are passed widened).  K must be a multiple of 32.  ``rule``: block scale
    rule, "ocp" or "uos" (see block_scale_byte).
    Returns (codes uint8 [R, K/2], scales uint8 [R, K/32]).
    """
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("quantize_mxfp4: expected a 2-D array")
    R, K = x.shape
    if K % BLOCK != 0:
        raise ValueError("quantize_mxfp4: K must be a multiple of 32")
    x64 = x.astype(np.float64)
    if not np.all(np.isfinite(x64)):
        raise ValueError("quantize_mxfp4: non-finite input is outside the contract")
    blocks = x64.reshape(R, K // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    scales = block_scale_byte(amax, rule)
    k = scales.astype(np.int64) - 127
    v = np.ldexp(blocks, -k[:, :, None])         # exact division by the power of two
    codes = e2m1_encode(v).reshape(R, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, scales


def unpack_codes(packed, K: int) -> np.ndarray:
    """Unpack [R, K/2] bytes into [R, K] 4-bit codes (low nibble = even element)."""
    packed = np.asarray(packed, dtype=np.uint8)
    R = packed.shape[0]
    out = np.empty((R, K), dtype=np.uint8)
    out[:, 0::2] = packed[:, : K // 2] & 0xF
    out[:, 1::2] = packed[:, : K // 2] >> 4
    return out


def dequantize_mxfp4(packed, scales, K: int) -> np.ndarray:
    """Dequantize MXFP4 codes and scales to float64 [R, K]: e2m1(code) * 2^(scale - 127)."""
    codes = unpack_codes(packed, K)
    R = codes.shape[0]
    vals = e2m1_decode(codes).reshape(R, K // BLOCK, BLOCK)
    scl = e8m0_decode(np.asarray(scales)[:, : K // BLOCK])
    return (vals * scl[:, :, None]).reshape(R, K)
