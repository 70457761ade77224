"""W4A4, W4A8 and bf16 reference GEMMs, accumulated in float64 (oracle; test
infrastructure only).

W is stored N x K (K contiguous, the nn.Linear weight layout); out = A @ W^T is M x N.

* W4A4 ("AMD Quark adds native W4A8 ...", section "Quark quantization pipeline":
  MXFP4 weights, dynamic MXFP4 activations; "AMD Quark: 1.92x faster FLUX.1-dev ...",
  section "MXFP4 quantization for diffusion models on AMD Instinct": the GEMM consumes
  MXFP4 directly):
      out[m, n] = sum_b 2^(SA[m,b] + SW[n,b] - 254) * sum_{i<32} e2m1(QA[m,32b+i]) * e2m1(QW[n,32b+i])
  Each block's scale factors out of its partial sum ("Exp 2026-08-22 W4A4 Reference
  Model", section "Status": a linear scale is applied in the fp32 drain).
* W4A8 (same page, static FP8 E4M3 activations):
      out[m, n] = s_a * sum_b 2^(SW[n,b] - 127) * sum_i e4m3(QA8[m,32b+i]) * e2m1(QW[n,32b+i])
* bf16 reference (BF16 is the quality ceiling in the same section):
      out[m, n] = sum_k a[m,k] * w[n,k] over the unquantized bf16 operands.

Each output is the plain dequantize-then-multiply definition: the operands are decoded
to float64 and multiplied with a float64 matrix product in row chunks (a library
primitive; no blocking or reordering beyond the chunking of independent rows).  Every
per-block product is exact in float64; only the cross-term float64 additions round.

Alongside every output the oracle returns T = sum_k |a_mk * w_nk| over the same
dequantized operands (times s_a for W4A8), the scale of the error budget
|gpu - oracle| <= 1e-5 * T + 1 bf16 ulp(oracle), where the oracle value is the float64
result rounded to bf16 (round to nearest even) -- the tolerance fixed for the GPU path.
"""

import numpy as np

from .formats import bf16_bits_to_f64, bf16_ulp, e4m3_decode, f64_to_bf16_bits
from .mxfp4 import dequantize_mxfp4

_CHUNK_ROWS = 2048


def _chunked_product(a_rows_fn, M: int, w64: np.ndarray, total: bool = True):
    """out = A @ W^T and (when ``total``) T = |A| @ |W|^T in float64, A produced chunk by
    chunk; T is None otherwise."""
    N = w64.shape[0]
    wT = w64.T
    wTabs = np.abs(w64).T if total else None
    out = np.empty((M, N), dtype=np.float64)
    tot = np.empty((M, N), dtype=np.float64) if total else None
    for r0 in range(0, M, _CHUNK_ROWS):
        r1 = min(M, r0 + _CHUNK_ROWS)
        a = a_rows_fn(r0, r1)
        out[r0:r1] = a @ wT
        if total:
            tot[r0:r1] = np.abs(a) @ wTabs
    return out, tot


def gemm_w4a4(a_codes, a_scales, w_codes, w_scales, K: int, total: bool = True):
    """W4A4: MXFP4 A [M,K] x MXFP4 W [N,K]^T.  Returns (out float64 [M,N], T [M,N] or
    None when ``total`` is False)."""
    a_codes = np.asarray(a_codes)
    a_scales = np.asarray(a_scales)
    w64 = dequantize_mxfp4(w_codes, w_scales, K)
    M = a_codes.shape[0]
    return _chunked_product(
        lambda r0, r1: dequantize_mxfp4(a_codes[r0:r1], a_scales[r0:r1], K), M, w64, total)


def gemm_w4a8(a_fp8, s_a, w_codes, w_scales, K: int, total: bool = True):
    """W4A8: FP8 E4M3 A [M,K] (dequant scale s_a) x MXFP4 W [N,K]^T -> (out, T or None)."""
    a_fp8 = np.asarray(a_fp8, dtype=np.uint8)
    s = float(np.float32(s_a))
    w64 = dequantize_mxfp4(w_codes, w_scales, K)
    M = a_fp8.shape[0]
    out, tot = _chunked_product(lambda r0, r1: e4m3_decode(a_fp8[r0:r1, :K]), M, w64, total)
    return out * s, (tot * abs(s) if total else None)


def gemm_bf16(a_bits, w_bits, total: bool = True):
    """bf16 reference: bf16 A [M,K] x bf16 W [N,K]^T over exactly widened values ->
    (out, T or None)."""
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    w64 = bf16_bits_to_f64(w_bits)
    M = a_bits.shape[0]
    return _chunked_product(lambda r0, r1: bf16_bits_to_f64(a_bits[r0:r1]), M, w64, total)


def to_bf16(out) -> np.ndarray:
    """The oracle's bf16 output bits (round to nearest even from float64)."""
    return f64_to_bf16_bits(out)


def tolerance_bound(T, oracle_bf16_bits) -> np.ndarray:
    """Per-element error budget 1e-5 * T + ulp_bf16(oracle value)."""
    ref = bf16_bits_to_f64(oracle_bf16_bits)
    return 1e-5 * np.asarray(T, dtype=np.float64) + bf16_ulp(ref)


def within_tolerance(gpu_bf16_bits, out, T):
    """Element-wise check of bf16 results against the float64 oracle.

    Returns (ok bool array, err float64 array, bound float64 array).
    """
    ref_bits = f64_to_bf16_bits(out)
    ref = bf16_bits_to_f64(ref_bits)
    got = bf16_bits_to_f64(gpu_bf16_bits)
    err = np.abs(got - ref)
    bound = tolerance_bound(T, ref_bits)
    ok = np.isfinite(got) & (err <= bound)
    return ok, err, bound
