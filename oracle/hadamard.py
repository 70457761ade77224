"""Fixed block-Hadamard rotation ahead of MXFP4 (oracle; test infrastructure only).

What is computed ("AMD Quark adds native W4A8 mixed-precision for Wan2.2 video generation
on MI350", section "Quark quantization pipeline and mixed-precision selection": a fixed,
data-free Hadamard rotation as the transform condition of the block selector; "Exp
2026-08-22 W4A4 Reference Model", section "Status": block-Hadamard composed with
per-group scales):

    y = x H_n / sqrt(n) on every run of n consecutive elements along K,

with H_n the Sylvester Hadamard matrix (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]).
Applied to activations online and to weights offline, it leaves the product unchanged
(H_n H_n^T = n I), and it spreads a block's outliers over n elements before the MX scale
is chosen.

Readings:
* n is 16, 64 or 256, so 1 / sqrt(n) is a power of two and the normalisation is exact.
* The rotated values decide MXFP4 codes, so they are computed in binary32 as the
  product is formed on the GPU: the radix-2 butterfly, stages h = 1, 2, 4, ..., n/2, each
  pair (i, i + h) with i & h == 0 becoming (x_i + x_{i+h}, x_i - x_{i+h}) rounded to
  binary32, then the multiply by 2^(-log2(n)/2).  In exact arithmetic this is x H_n / sqrt(n);
  the pins check that, and the rounding error against the float64 product.
"""

import numpy as np

from .mxfp4 import quantize_mxfp4

BLOCK_SIZES = (16, 64, 256)


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_n (int64 entries +-1), n a power of two."""
    if n < 1 or n & (n - 1):
        raise ValueError("hadamard_matrix: n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_f32(x, n: int) -> np.ndarray:
    """x H_n / sqrt(n) on runs of n elements along the last axis, in binary32 (see the
    module docstring for the operation order).  x: [..., K] with K % n == 0."""
    if n not in BLOCK_SIZES:
        raise ValueError(f"rotate_f32: n must be one of {BLOCK_SIZES}")
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    if K % n:
        raise ValueError("rotate_f32: K must be a multiple of n")
    v = x.reshape(-1, K // n, n).copy()
    h = 1
    while h < n:
        idx = np.arange(n)
        lo = idx[(idx & h) == 0]
        a = v[:, :, lo]
        b = v[:, :, lo + h]
        v[:, :, lo] = a + b          # binary32 adds (numpy float32 arithmetic)
        v[:, :, lo + h] = a - b
        h *= 2
    scale = np.float32(2.0 ** (-(int(np.log2(n)) // 2)))
    return (v * scale).reshape(x.shape)


def quantize_mxfp4_rotated(x, n: int, rule: str = "ocp"):
    """MXFP4 codes and scales of rotate_f32(x, n) (2-D x, K % n == 0, K % 32 == 0)."""
    return quantize_mxfp4(rotate_f32(x, n), rule)
