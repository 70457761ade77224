"""Static FP8 E4M3 activation quantization for W4A8 (oracle; test infrastructure only).

"AMD Quark adds native W4A8 mixed-precision for Wan2.2 video generation on MI350",
section "Quark quantization pipeline and mixed-precision selection": W4A8 keeps MXFP4
weights and uses static FP8 E4M3 activations.  "Static" means the scale is fixed ahead
of time rather than derived per call.

Readings taken (the page gives no formula):
* one per-tensor scale from the tensor's absolute maximum, mapping amax onto the E4M3
  maximum 448: s_a = fl32(amax / 448) (dequantization scale) and
  inv_s = fl32(448 / amax) (quantization multiplier), both rounded once to binary32;
* q = E4M3(fl32(x * inv_s)): one binary32 multiply (round to nearest even), then
  rounding to the nearest E4M3 value, ties to the even code, saturating magnitudes
  above 448 to 448 (no NaN is ever produced); the sign bit comes from the input.

Quantize-dequantize emulation (the same section: W4A8 quality figures come from QDQ
emulation, not from native kernels).  Reading: the dequantized activation is what a
binary32 computation hands to a bf16 GEMM, y = bf16(fl32(e4m3(q) * s_a)) -- the exact
E4M3 value times s_a in one binary32 multiply, then rounded to bf16 (both steps round
to nearest even).
"""

import numpy as np

from .formats import E4M3_TABLE, E4M3_MAX, e4m3_decode, f64_to_bf16_bits

#: finite non-negative E4M3 magnitudes, ascending; index = code (0x00 .. 0x7E)
_E4M3_GRID = E4M3_TABLE[:0x7F].copy()


def fp8_static_scales(amax: float):
    """(s_a, inv_s) as binary32 for a per-tensor absolute maximum ``amax`` > 0."""
    a = np.float32(amax)
    if not np.isfinite(a) or a <= 0:
        raise ValueError("fp8_static_scales: amax must be positive and finite")
    s_a = np.float32(a / np.float32(E4M3_MAX))
    inv_s = np.float32(np.float32(E4M3_MAX) / a)
    return s_a, inv_s


def e4m3_encode(v) -> np.ndarray:
    """Round values to E4M3 codes (uint8): nearest, ties to even code, saturate at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.abs(v)
    grid = _E4M3_GRID
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = np.abs(a - grid[lo])
    d_hi = np.abs(grid[hi] - a)
    pick = np.where(d_lo < d_hi, lo, hi)
    pick = np.where(d_lo == d_hi, np.where(lo % 2 == 0, lo, hi), pick)
    # at or past 448 the nearest finite point is 448 (saturation), decided by comparison
    pick = np.where(a >= grid[-1], len(grid) - 1, pick)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    return pick.astype(np.uint8) | sign


def quantize_fp8(x, inv_s) -> np.ndarray:
    """q = E4M3(fl32(x * inv_s)) elementwise; ``x`` must be binary32-representable."""
    x32 = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("quantize_fp8: non-finite input is outside the contract")
    with np.errstate(over="ignore"):            # a product past binary32 becomes +-inf and saturates
        y = x32 * np.float32(inv_s)             # one binary32 multiply, RNE
    return e4m3_encode(y.astype(np.float64))


def dequantize_fp8(q, s_a) -> np.ndarray:
    """bf16 bit patterns (uint16) of bf16(fl32(e4m3(q) * s_a)) elementwise.  The NaN
    codes S.1111.111 (never produced by quantize_fp8) give the bf16 NaN 0x7FC0 / 0xFFC0."""
    q = np.asarray(q, dtype=np.uint8)
    nan = (q & 0x7F) == 0x7F
    v = e4m3_decode(np.where(nan, 0, q)).astype(np.float32)   # exact: 4 significant bits
    y = v * np.float32(s_a)                                    # one binary32 multiply, RNE
    bits = f64_to_bf16_bits(y.astype(np.float64))             # binary32 -> bf16, RNE
    return np.where(nan, np.uint16(0x7FC0) | ((q >> 7).astype(np.uint16) << 15), bits).astype(np.uint16)
