"""Python binding of libmxq (OCP MXFP4 quantization + W4A4 / W4A8 GEMMs for MI355X).

The functions here only marshal arguments: they check tensor devices, dtypes and shapes,
allocate outputs with torch (device memory) and call the C ABI declared in
``include/mxq.h`` on torch's current HIP stream.  Every step of the computation runs in
the library's gfx950 kernels.  Importing fails loudly if ``libmxq.so`` has not been
built (``python mxfp4_microscaled_quantization_amd/build.py``); there is no fallback.

Function names mirror the C entry points without the ``mxq_`` prefix:
``quantize``, ``quantize_fp8``, ``absmax``, ``gemm_w4a4``, ``gemm_w4a4_fused``, ``gemm_w4a8``, ``gemm_bf16``,
``sqnr``, ``dequantize``.  ``lib`` exposes the raw ctypes functions.
"""

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "lib", "MxqError", "quantize", "quantize_into", "quantize_hadamard", "SCALE_RULES", "quantize_fp8", "absmax", "fp8_static_scales",
    "gemm_w4a4", "gemm_w4a4_fused", "gemm_w4a8", "gemm_bf16", "sqnr", "sqnr_workspace_bytes", "dequantize",
    "mfma_ceiling", "MFMA_FLOP",
    "LIB_PATH", "ABI_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxq.so")

MXQ_OK, MXQ_ERR_INVALID_ARG, MXQ_ERR_UNSUPPORTED, MXQ_ERR_HIP = 0, 1, 2, 3
MXQ_F32, MXQ_BF16 = 0, 1

_i64, _ptr, _f32, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

#: every exported symbol with (restype, argtypes) -- the C ABI of include/mxq.h
ABI_SYMBOLS = {
    "mxq_quantize": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr]),
    "mxq_quantize_rule": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _ptr, _i64, _ptr, _i64, ctypes.c_int,
                                         _ptr]),
    "mxq_quantize_hadamard": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _ptr,
                                             _i64, _ptr, _i64, _ptr]),
    "mxq_quantize_fp8": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _f32, _ptr, _i64, _ptr]),
    "mxq_absmax": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _ptr, _ptr]),
    "mxq_gemm_w4a4": (ctypes.c_int, [_ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_gemm_w4a4_fused": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _ptr, _ptr, _i64, _i64, _i64, ctypes.c_int, _ptr,
                                           _i64, _ptr]),
    "mxq_gemm_w4a8": (ctypes.c_int, [_ptr, _f32, _ptr, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_gemm_bf16": (ctypes.c_int, [_ptr, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_sqnr_workspace_bytes": (_sz, [_i64]),
    "mxq_sqnr": (ctypes.c_int, [_ptr, _ptr, _i64, _i64, _i64, _i64, _ptr, _sz, _ptr, _ptr]),
    "mxq_dequantize": (ctypes.c_int, [_ptr, _i64, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_mfma_ceiling": (ctypes.c_int, [ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _ptr,
                                        _ptr]),
    "mxq_last_error": (ctypes.c_char_p, []),
    "mxq_abi_version": (ctypes.c_int, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmxq.so not found at {LIB_PATH}; build it with "
            "`python mxfp4_microscaled_quantization_amd/build.py` (hipcc, gfx950)")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in ABI_SYMBOLS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class MxqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[mxq status {status}] {message}")
        self.status = status


def _check(status: int):
    if status != MXQ_OK:
        raise MxqError(status, lib.mxq_last_error().decode(errors="replace"))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _rowmajor(t: torch.Tensor, name: str):
    """2-D tensor with unit column stride; returns its row pitch in elements."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _dtype_code(t: torch.Tensor):
    if t.dtype == torch.bfloat16:
        return MXQ_BF16
    if t.dtype == torch.float32:
        return MXQ_F32
    raise ValueError("input must be bfloat16 or float32")


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


SCALE_RULES = {"ocp": 0, "uos": 1}


def _rule_code(rule: str) -> int:
    if rule not in SCALE_RULES:
        raise ValueError(f"scale rule must be one of {sorted(SCALE_RULES)}")
    return SCALE_RULES[rule]


def quantize(x: torch.Tensor, rule: str = "ocp"):
    """MXFP4-quantize rows of ``x`` (bf16 or fp32, [R, K], K % 32 == 0).

    ``rule``: "ocp" (X = 2^(floor(log2 amax) - 2)) or "uos" (smallest power of two with
    amax <= 7.25 X).  Returns (codes uint8 [R, K/2], scales uint8 [R, K/32]).
    """
    _dev(x, "x")
    ld = _rowmajor(x, "x")
    R, K = x.shape
    codes = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib.mxq_quantize_rule(_p(x), _dtype_code(x), R, K, ld, _p(codes), K // 2, _p(scales), K // 32,
                                 _rule_code(rule), _stream()))
    return codes, scales


def quantize_into(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, rule: str = "ocp"):
    """MXFP4-quantize into caller-provided outputs (may be row-strided views)."""
    _dev(x, "x")
    ld = _rowmajor(x, "x")
    R, K = x.shape
    _check(lib.mxq_quantize_rule(_p(x), _dtype_code(x), R, K, ld, _p(codes), _rowmajor(codes, "codes"),
                                 _p(scales), _rowmajor(scales, "scales"), _rule_code(rule), _stream()))


def quantize_hadamard(x: torch.Tensor, block_n: int = 64, rule: str = "ocp"):
    """Rotate runs of ``block_n`` (16, 64, 256) elements of each row by H / sqrt(block_n)
    (Sylvester Hadamard, binary32 butterfly), then MXFP4-quantize.  Returns (codes, scales)."""
    _dev(x, "x")
    ld = _rowmajor(x, "x")
    R, K = x.shape
    codes = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib.mxq_quantize_hadamard(_p(x), _dtype_code(x), R, K, ld, int(block_n), _rule_code(rule), _p(codes), K // 2,
                                     _p(scales), K // 32, _stream()))
    return codes, scales


def fp8_static_scales(amax: float):
    """(s_a, inv_s) as binary32 for a per-tensor absolute maximum: amax/448, 448/amax."""
    a = np.float32(amax)
    return float(np.float32(a / np.float32(448.0))), float(np.float32(np.float32(448.0) / a))


def quantize_fp8(x: torch.Tensor, inv_scale: float, out=None) -> torch.Tensor:
    """Static FP8 E4M3: q = E4M3(fl32(x * inv_scale)), saturating; returns uint8 [R, K]."""
    _dev(x, "x")
    ld = _rowmajor(x, "x")
    R, K = x.shape
    q = torch.empty((R, K), dtype=torch.uint8, device=x.device) if out is None else out
    if q.dtype != torch.uint8 or q.shape != (R, K):
        raise ValueError("out must be uint8 [R, K]")
    _check(lib.mxq_quantize_fp8(_p(x), _dtype_code(x), R, K, ld, float(inv_scale), _p(q), _rowmajor(q, "out"),
                                _stream()))
    return q


def absmax(x: torch.Tensor) -> torch.Tensor:
    """max |x| as a 1-element float32 GPU tensor."""
    _dev(x, "x")
    ld = _rowmajor(x, "x")
    R, K = x.shape
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib.mxq_absmax(_p(x), _dtype_code(x), R, K, ld, _p(out), _stream()))
    return out


def _out(M, N, device, out):
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device), N
    if out.dtype != torch.bfloat16 or out.shape != (M, N):
        raise ValueError("out must be bfloat16 [M, N]")
    return out, _rowmajor(out, "out")


def _contig(t, name, dtype):
    _dev(t, name)
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")
    return t


def gemm_w4a4(a_codes, a_scales, w_codes, w_scales, out=None):
    """W4A4: MXFP4 A [M, K] x MXFP4 W [N, K]^T -> bf16 [M, N]."""
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (w_codes, "w_codes"), (w_scales, "w_scales")):
        _contig(t, n, torch.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K or a_scales.shape != (M, K // 32) or w_scales.shape != (N, K // 32):
        raise ValueError("inconsistent MXFP4 operand shapes")
    out, ld = _out(M, N, a_codes.device, out)
    _check(lib.mxq_gemm_w4a4(_p(a_codes), _p(a_scales), _p(w_codes), _p(w_scales), M, N, K, _p(out), ld, _stream()))
    return out


def gemm_w4a4_fused(a, w_codes, w_scales, rule: str = "ocp", out=None):
    """W4A4 with the activation quantization fused in: bf16 or fp32 A [M, K] (rows may be
    strided) x MXFP4 W [N, K]^T -> bf16 [M, N]; equal to gemm_w4a4(*quantize(a, rule), W)."""
    _dev(a, "a")
    ld = _rowmajor(a, "a")
    for t, n in ((w_codes, "w_codes"), (w_scales, "w_scales")):
        _contig(t, n, torch.uint8)
    M, K = a.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K or w_scales.shape != (N, K // 32):
        raise ValueError("inconsistent operand shapes")
    out, ldo = _out(M, N, a.device, out)
    _check(lib.mxq_gemm_w4a4_fused(_p(a), _dtype_code(a), ld, _p(w_codes), _p(w_scales), M, N, K, _rule_code(rule),
                                   _p(out), ldo, _stream()))
    return out


def gemm_w4a8(a_fp8, a_scale: float, w_codes, w_scales, out=None):
    """W4A8: FP8 E4M3 A [M, K] (dequant scale a_scale) x MXFP4 W [N, K]^T -> bf16 [M, N]."""
    for t, n in ((a_fp8, "a_fp8"), (w_codes, "w_codes"), (w_scales, "w_scales")):
        _contig(t, n, torch.uint8)
    M, K = a_fp8.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K or w_scales.shape != (N, K // 32):
        raise ValueError("inconsistent operand shapes")
    out, ld = _out(M, N, a_fp8.device, out)
    _check(lib.mxq_gemm_w4a8(_p(a_fp8), float(a_scale), _p(w_codes), _p(w_scales), M, N, K, _p(out), ld, _stream()))
    return out


def gemm_bf16(a, w, out=None):
    """bf16 reference: A [M, K] x W [N, K]^T -> bf16 [M, N], fp32 accumulation."""
    _contig(a, "a", torch.bfloat16)
    _contig(w, "w", torch.bfloat16)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("inconsistent operand shapes")
    out, ld = _out(M, N, a.device, out)
    _check(lib.mxq_gemm_bf16(_p(a), _p(w), M, N, K, _p(out), ld, _stream()))
    return out


#: MFMA instruction FLOP per mode, as mxq_mfma_ceiling runs them
MFMA_FLOP = {"w4a4": 2 * 32 * 32 * 64, "w4a8": 2 * 32 * 32 * 64, "bf16": 2 * 16 * 16 * 32}
_GEMM_MODES = {"w4a4": 0, "w4a8": 1, "bf16": 2}


def mfma_ceiling(mode: str, a, a_scales, w, w_scales, waves: int, iters: int, sink=None) -> int:
    """Enqueue the register-only MFMA loop of mxq_mfma_ceiling on the operand planes of a
    GEMM call (``mode`` "w4a4", "w4a8" or "bf16"; operands as for that GEMM, unused scales
    None) on the current stream; returns the FLOP it performs."""
    if mode not in _GEMM_MODES:
        raise ValueError(f"mode must be one of {sorted(_GEMM_MODES)}")
    if mode == "bf16":
        _contig(a, "a", torch.bfloat16)
        _contig(w, "w", torch.bfloat16)
        M, K = a.shape
    else:
        _contig(a, "a", torch.uint8)
        _contig(w, "w", torch.uint8)
        _contig(w_scales, "w_scales", torch.uint8)
        M = a.shape[0]
        K = a.shape[1] * (2 if mode == "w4a4" else 1)
        if mode == "w4a4":
            _contig(a_scales, "a_scales", torch.uint8)
    N = w.shape[0]
    if sink is None:
        sink = torch.empty(waves * 64, dtype=torch.float32, device=a.device)
    elif sink.dtype != torch.float32 or sink.numel() < waves * 64 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor of at least waves * 64 elements")
    _check(lib.mxq_mfma_ceiling(_GEMM_MODES[mode], _p(a), _p(a_scales) if a_scales is not None else None, _p(w),
                                _p(w_scales) if w_scales is not None else None, M, N, K, waves, iters, _p(sink),
                                _stream()))
    return waves * iters * 16 * MFMA_FLOP[mode]


def sqnr_workspace_bytes(n: int) -> int:
    return int(lib.mxq_sqnr_workspace_bytes(n))


def sqnr(ref, test, workspace=None, out3=None) -> torch.Tensor:
    """Whole-output SQNR; returns a float64 GPU tensor [S, N, dB]."""
    _dev(ref, "ref")
    _dev(test, "test")
    if ref.dtype != torch.bfloat16 or test.dtype != torch.bfloat16 or ref.shape != test.shape:
        raise ValueError("ref/test must be bf16 tensors of one shape")
    R, C = ref.shape
    nbytes = sqnr_workspace_bytes(R * C)
    if workspace is None:
        workspace = torch.empty(nbytes // 8, dtype=torch.float64, device=ref.device)
    if out3 is None:
        out3 = torch.empty(3, dtype=torch.float64, device=ref.device)
    _check(lib.mxq_sqnr(_p(ref), _p(test), R, C, _rowmajor(ref, "ref"), _rowmajor(test, "test"), _p(workspace),
                        workspace.numel() * workspace.element_size(), _p(out3), _stream()))
    return out3


def dequantize(codes, scales, K: int, out=None) -> torch.Tensor:
    """MXFP4 -> bf16 [R, K] (into ``out`` if given: bfloat16 [R, K], rows may be strided)."""
    _dev(codes, "codes")
    R = codes.shape[0]
    if out is None:
        y, ld = torch.empty((R, K), dtype=torch.bfloat16, device=codes.device), K
    else:
        if out.dtype != torch.bfloat16 or out.shape != (R, K):
            raise ValueError("out must be bfloat16 [R, K]")
        y, ld = out, _rowmajor(out, "out")
    _check(lib.mxq_dequantize(_p(codes), _rowmajor(codes, "codes"), _p(scales), _rowmajor(scales, "scales"),
                              R, K, _p(y), ld, _stream()))
    return y
