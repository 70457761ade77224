"""CPU oracle for OCP MXFP4 quantization, the W4A4 / W4A8 GEMMs that consume it, and
whole-output SQNR.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package: only
the test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, headers,
tables or helpers) and imports nothing from it.

Everything here is plain NumPy written straight from the definitions, in float64 (or
exact integer / rational arithmetic) unless the method fixes a precision:

* ``formats``  -- value tables of E2M1, E8M0, E4M3 and bf16, built from the bit-field
  definitions; bf16 round-to-nearest-even.
* ``mxfp4``    -- the MX block quantizer: 32-element blocks along K, one E8M0
  power-of-two scale per block (2^(floor(log2 amax) - 2)), E2M1 elements rounded to
  nearest with ties to even and saturated to +-6.
* ``fp8``      -- static per-tensor FP8 E4M3 activation quantization and its QDQ
  dequantization to bf16.
* ``gemm``     -- W4A4, W4A8 and bf16 reference GEMMs accumulated in float64, with the
  per-element error budget |gpu - oracle| <= 1e-5 * sum|a*b| + 1 bf16 ulp.
* ``sqnr``     -- whole-output signal-to-quantization-noise ratio in dB.
* ``hadamard`` -- the fixed block-Hadamard rotation ahead of MXFP4, in binary32.

Sources (web pages, cited by title and section):
* "AMD Quark adds native W4A8 mixed-precision for Wan2.2 video generation on MI350",
  section "Quark quantization pipeline and mixed-precision selection" -- MXFP4 weights;
  dynamic MXFP4 activations (W4A4) vs static FP8 E4M3 activations (W4A8); whole-block
  output SQNR against BF16.
* "AMD Quark: 1.92x faster FLUX.1-dev with MXFP4 on Instinct MI350", section
  "What is MXFP4" -- 4-bit elements, 32-element blocks sharing one scale; the GEMM
  consumes MXFP4 directly.
* "MXAttention: Data-Free Optimal Scaling and Pre-Normalization Quantization for MXFP4
  Attention", sections "What it actually does" / "How this relates" -- the shared
  scale is an E8M0 power of two with no mantissa.
* "Exp 2026-08-22 W4A4 Reference Model", section "Status" -- a linear per-group scale
  factors out of each group's partial sum and is applied in the fp32 drain.

Points the pages leave open (the E2M1 value set, E8M0 bias, rounding mode, saturation,
nibble order, the E4M3 variant, the static-scale formula, the SQNR definition) follow
the OCP Microscaling Formats v1.0 specification; each reading is stated where it is used.

Parity status: every public function is pinned by the ``-m "not gpu"`` tests against
closed forms, library routines, exact rational brute force or invariants.
"""

from . import formats, mxfp4, fp8, gemm, sqnr, hadamard  # noqa: F401
from .formats import (  # noqa: F401
    E2M1_MAGNITUDES, e2m1_decode, e8m0_decode, e4m3_decode, E4M3_MAX,
    bf16_bits_to_f64, f64_to_bf16_bits, bf16_ulp,
)
from .mxfp4 import block_scale_byte, quantize_mxfp4, dequantize_mxfp4, e2m1_encode  # noqa: F401
from .fp8 import fp8_static_scales, e4m3_encode, quantize_fp8, dequantize_fp8  # noqa: F401
from .gemm import (  # noqa: F401
    gemm_w4a4, gemm_w4a8, gemm_bf16, within_tolerance, tolerance_bound,
)
from .sqnr import sqnr_db  # noqa: F401
from .hadamard import hadamard_matrix, rotate_f32, quantize_mxfp4_rotated  # noqa: F401
