"""Element and scale formats, built from their bit-field definitions (oracle; test
infrastructure only).

* E2M1 (FP4): 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0
  is subnormal.  The pages say only that MXFP4 stores 4 bits per element ("AMD Quark:
  1.92x faster FLUX.1-dev with MXFP4 on Instinct MI350", section "What is MXFP4"); the
  field layout is the OCP Microscaling v1.0 one, and its top magnitude 6 is the
  saturation point of the MX rule.
* E8M0: an unsigned 8-bit power-of-two exponent with no mantissa ("MXAttention ...",
  section "What it actually does"); bias 127, 0xFF is NaN (OCP MX v1.0).
* E4M3: the OCP FP8 E4M3 variant (bias 7, no infinities, S.1111.111 is NaN, max 448),
  the static activation format of W4A8 ("AMD Quark adds native W4A8 ...", section
  "Quark quantization pipeline and mixed-precision selection").
* bf16: the top 16 bits of an IEEE binary32; the GEMM output type.
"""

import math

import numpy as np


def _e2m1_value(code: int) -> float:
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:                      # subnormal: 0.m x 2^(1 - bias), bias = 1
        mag = (man / 2.0) * 2.0 ** (1 - 1)
    else:                             # normal: 1.m x 2^(exp - bias)
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return sign * mag


#: decoded value of each of the 16 E2M1 codes (index = code); codes 8..15 are the
#: negatives of 0..7 (code 8 is -0.0)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
#: the 8 non-negative magnitudes, ascending (index = magnitude code)
E2M1_MAGNITUDES = E2M1_TABLE[:8].copy()


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (any integer array, values 0..15) to float64."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.int64) & 0xF]


def e8m0_decode(scale_bytes) -> np.ndarray:
    """Decode E8M0 bytes to float64: 2^(byte - 127); 0xFF is NaN."""
    b = np.asarray(scale_bytes, dtype=np.int64)
    out = np.ldexp(1.0, b - 127).astype(np.float64)
    return np.where(b == 0xFF, np.nan, out)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:                      # subnormal: 0.m x 2^(1 - 7)
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


#: decoded value of each of the 256 E4M3 codes (0x7F and 0xFF are NaN)
E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
#: largest finite E4M3 magnitude
E4M3_MAX = float(np.nanmax(E4M3_TABLE))


def e4m3_decode(codes) -> np.ndarray:
    """Decode FP8 E4M3 bytes to float64 (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly: a bf16 is the high half of a binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_ulp(x) -> np.ndarray:
    """One bf16 unit in the last place at the magnitude of x (float64 array).

    2^(floor(log2|x|) - 7) for |x| >= 2^-126, else the subnormal spacing 2^-133.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)                  # a = f * 2^e, f in [0.5, 1)  =>  floor(log2 a) = e - 1
    ulp = np.ldexp(1.0, (e - 1) - 7)
    return np.where(a >= 2.0 ** -126, ulp, 2.0 ** -133)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    bf16 keeps 8 significant bits over binary32's exponent range, so the rounding
    quantum at |x| is 2^(max(floor(log2|x|), -126) - 7).  Dividing by that power of two
    is exact, np.rint rounds half to even, and multiplying back is exact.  Values that
    round past the largest finite bf16 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("f64_to_bf16_bits: NaN input")
    a = np.abs(x)
    _, e = np.frexp(a)
    quantum_exp = np.maximum(e - 1, -126) - 7
    r = np.ldexp(np.rint(np.ldexp(a, -quantum_exp)), quantum_exp)
    r = np.where(np.isinf(a), np.inf, r)
    # r is now an exact bf16 magnitude (or >= 2^128, which is infinity in bf16)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.signbit(x).astype(np.uint16) << np.uint16(15)
    return bits | sign
