"""Python binding of libmxq (OCP MXFP4 quantization + W4A4 / W4A8 GEMMs for MI355X).

The functions here only marshal arguments: they check every tensor's device, dtype and
shape (inputs and caller-supplied output or scratch buffers, ``check_buffer``), allocate
outputs with torch (device memory) and call the C ABI declared in
``include/mxq.h`` on torch's current HIP stream.  Every step of the computation runs in
the library's gfx950 kernels.  Importing fails loudly if ``libmxq.so`` has not been
built (``python mxfp4_microscaled_quantization_amd/build.py``); there is no fallback.

Function names mirror the C entry points without the ``mxq_`` prefix:
``quantize``, ``quantize_fp8``, ``absmax``, ``gemm_w4a4``, ``gemm_w4a4_fused``, ``gemm_w4a8``, ``gemm_bf16``,
``sqnr``, ``dequantize``, ``dequantize_fp8``, ``fp8_static_scales``.  ``lib`` exposes the raw ctypes functions.
"""

import ctypes
import os

import torch

__all__ = [
    "lib", "MxqError", "quantize", "quantize_into", "quantize_hadamard", "SCALE_RULES", "quantize_fp8", "absmax", "fp8_static_scales",
    "gemm_w4a4", "gemm_w4a4_fused", "gemm_w4a8", "gemm_bf16", "sqnr", "sqnr_noalloc", "sqnr_workspace_bytes", "dequantize", "dequantize_fp8",
    "mfma_ceiling", "MFMA_FLOP", "check_buffer",
    "LIB_PATH", "ABI_SYMBOLS", "ABI_VERSION",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxq.so")

#: MXQ_ABI_VERSION of include/mxq.h that the signatures below describe
ABI_VERSION = 2

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
                                           _i64, _ptr, _sz, _ptr]),
    "mxq_gemm_w4a4_fused_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "mxq_gemm_w4a8": (ctypes.c_int, [_ptr, _f32, _ptr, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_gemm_bf16": (ctypes.c_int, [_ptr, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_sqnr_workspace_bytes": (_sz, [_i64]),
    "mxq_sqnr": (ctypes.c_int, [_ptr, _ptr, _i64, _i64, _i64, _i64, _ptr, _sz, _ptr, _ptr]),
    "mxq_sqnr_noalloc": (ctypes.c_int, [_ptr, _ptr, _i64, _i64, _i64, _i64, _ptr, _ptr]),
    "mxq_dequantize": (ctypes.c_int, [_ptr, _i64, _ptr, _i64, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_dequantize_fp8": (ctypes.c_int, [_ptr, _i64, _f32, _i64, _i64, _ptr, _i64, _ptr]),
    "mxq_fp8_static_scales": (ctypes.c_int, [_f32, ctypes.POINTER(_f32), ctypes.POINTER(_f32)]),
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
    found = handle.mxq_abi_version()
    if found != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} reports ABI version {found}, this binding expects {ABI_VERSION}: "
                          "rebuild it with `python mxfp4_microscaled_quantization_amd/build.py`")
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


def _dev(t, name: str, device=None):
    """``t`` must be a GPU tensor (on ``device`` when given)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _rowmajor(t: torch.Tensor, name: str):
    """2-D tensor with unit column stride; returns its row pitch in elements."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def check_buffer(t, name: str, dtype, shape=None, device=None, contiguous=False, min_numel=None, is_gpu=None):
    """Validate a tensor the caller hands to the library (input or output buffer).

    Checks, in order, raising ValueError before anything reaches the C ABI: a tensor;
    on a GPU (``is_gpu``, default the ``is_cuda`` test) and on ``device`` when given;
    ``dtype``; ``shape`` (a tuple, for a 2-D buffer with contiguous rows) or
    ``min_numel`` (for a flat contiguous buffer); fully contiguous when ``contiguous``.
    Returns the row pitch in elements for 2-D buffers, else None.  A pure function of
    tensor metadata, so it is unit-tested on CPU / meta tensors (``is_gpu`` lets a test
    stand those in for device tensors).
    """
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    gpu = t.is_cuda if is_gpu is None else is_gpu(t)
    if not gpu:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if min_numel is not None:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < min_numel:
            raise ValueError(f"{name} needs at least {min_numel} elements (got {t.numel()})")
        return None
    if shape is not None:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
        return _rowmajor(t, name)
    return None


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


def _input(x, name="x"):
    """A bf16 / binary32 2-D GPU input with contiguous rows: (row pitch, dtype code)."""
    _dev(x, name)
    code = _dtype_code(x)
    return _rowmajor(x, name), code


def _mx_outputs(x, R, K, codes, scales):
    if codes is None:
        codes = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    ldc = check_buffer(codes, "codes", torch.uint8, (R, K // 2), x.device)
    lds = check_buffer(scales, "scales", torch.uint8, (R, K // 32), x.device)
    return codes, ldc, scales, lds


def quantize(x: torch.Tensor, rule: str = "ocp"):
    """MXFP4-quantize rows of ``x`` (bf16 or fp32, [R, K], K % 32 == 0).

    ``rule``: "ocp" (X = 2^(floor(log2 amax) - 2)) or "uos" (smallest power of two with
    amax <= 7.25 X).  Returns (codes uint8 [R, K/2], scales uint8 [R, K/32]).
    """
    ld, dt = _input(x)
    R, K = x.shape
    codes, ldc, scales, lds = _mx_outputs(x, R, K, None, None)
    _check(lib.mxq_quantize_rule(_p(x), dt, R, K, ld, _p(codes), ldc, _p(scales), lds, _rule_code(rule), _stream()))
    return codes, scales


def quantize_into(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, rule: str = "ocp"):
    """MXFP4-quantize into caller-provided outputs: codes uint8 [R, K/2] and scales uint8
    [R, K/32] on x's device (rows may be strided views)."""
    ld, dt = _input(x)
    R, K = x.shape
    codes, ldc, scales, lds = _mx_outputs(x, R, K, codes, scales)
    _check(lib.mxq_quantize_rule(_p(x), dt, R, K, ld, _p(codes), ldc, _p(scales), lds, _rule_code(rule), _stream()))


def quantize_hadamard(x: torch.Tensor, block_n: int = 64, rule: str = "ocp"):
    """Rotate runs of ``block_n`` (16, 64, 256) elements of each row by H / sqrt(block_n)
    (Sylvester Hadamard, binary32 butterfly), then MXFP4-quantize.  Returns (codes, scales)."""
    ld, dt = _input(x)
    R, K = x.shape
    codes, ldc, scales, lds = _mx_outputs(x, R, K, None, None)
    _check(lib.mxq_quantize_hadamard(_p(x), dt, R, K, ld, int(block_n), _rule_code(rule), _p(codes), ldc,
                                     _p(scales), lds, _stream()))
    return codes, scales


def fp8_static_scales(amax: float):
    """(s_a, inv_s) for a per-tensor absolute maximum, formed by the library
    (mxq_fp8_static_scales): fl32(amax / 448) and fl32(448 / amax)."""
    s_a, inv_s = _f32(), _f32()
    _check(lib.mxq_fp8_static_scales(float(amax), ctypes.byref(s_a), ctypes.byref(inv_s)))
    return float(s_a.value), float(inv_s.value)


def quantize_fp8(x: torch.Tensor, inv_scale: float, out=None) -> torch.Tensor:
    """Static FP8 E4M3: q = E4M3(fl32(x * inv_scale)), saturating; returns uint8 [R, K]."""
    ld, dt = _input(x)
    R, K = x.shape
    q = torch.empty((R, K), dtype=torch.uint8, device=x.device) if out is None else out
    ldq = check_buffer(q, "out", torch.uint8, (R, K), x.device)
    _check(lib.mxq_quantize_fp8(_p(x), dt, R, K, ld, float(inv_scale), _p(q), ldq, _stream()))
    return q


def absmax(x: torch.Tensor) -> torch.Tensor:
    """max |x| as a 1-element float32 GPU tensor."""
    ld, dt = _input(x)
    R, K = x.shape
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib.mxq_absmax(_p(x), dt, R, K, ld, _p(out), _stream()))
    return out


def _out(M, N, device, out):
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device), N
    return out, check_buffer(out, "out", torch.bfloat16, (M, N), device)


def _contig(t, name, dtype, device=None, shape=None):
    check_buffer(t, name, dtype, device=device, contiguous=True)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _2d(t, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return t


def _mx_weights(w_codes, w_scales, K, device):
    _2d(w_codes, "w_codes")
    N = w_codes.shape[0]
    _contig(w_codes, "w_codes", torch.uint8, device, (N, K // 2))
    _contig(w_scales, "w_scales", torch.uint8, device, (N, K // 32))
    return N


def gemm_w4a4(a_codes, a_scales, w_codes, w_scales, out=None):
    """W4A4: MXFP4 A [M, K] x MXFP4 W [N, K]^T -> bf16 [M, N]."""
    _2d(a_codes, "a_codes")
    _contig(a_codes, "a_codes", torch.uint8)
    dev = a_codes.device
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    _contig(a_scales, "a_scales", torch.uint8, dev, (M, K // 32))
    N = _mx_weights(w_codes, w_scales, K, dev)
    out, ld = _out(M, N, dev, out)
    _check(lib.mxq_gemm_w4a4(_p(a_codes), _p(a_scales), _p(w_codes), _p(w_scales), M, N, K, _p(out), ld, _stream()))
    return out


def fused_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes with which gemm_w4a4_fused takes the separate-quantization route
    (0 where the fused kernel is the faster)."""
    return int(lib.mxq_gemm_w4a4_fused_workspace_bytes(M, N, K))


def gemm_w4a4_fused(a, w_codes, w_scales, rule: str = "ocp", out=None, route: bool = True):
    """W4A4 with the activation quantization fused in: bf16 or fp32 A [M, K] (rows may be
    strided) x MXFP4 W [N, K]^T -> bf16 [M, N]; equal to gemm_w4a4(*quantize(a, rule), W).
    route=True lends the call a workspace, so shapes past the fused kernel's break-even
    quantize in a pass of their own; route=False always runs the fused kernel."""
    ld, dt = _input(a, "a")
    M, K = a.shape
    N = _mx_weights(w_codes, w_scales, K, a.device)
    out, ldo = _out(M, N, a.device, out)
    nbytes = fused_workspace_bytes(M, N, K) if route else 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=a.device) if nbytes else None
    _check(lib.mxq_gemm_w4a4_fused(_p(a), dt, ld, _p(w_codes), _p(w_scales), M, N, K, _rule_code(rule),
                                   _p(out), ldo, _p(ws) if ws is not None else None, nbytes, _stream()))
    return out


def gemm_w4a8(a_fp8, a_scale: float, w_codes, w_scales, out=None):
    """W4A8: FP8 E4M3 A [M, K] (dequant scale a_scale) x MXFP4 W [N, K]^T -> bf16 [M, N]."""
    _2d(a_fp8, "a_fp8")
    _contig(a_fp8, "a_fp8", torch.uint8)
    dev = a_fp8.device
    M, K = a_fp8.shape
    N = _mx_weights(w_codes, w_scales, K, dev)
    out, ld = _out(M, N, dev, out)
    _check(lib.mxq_gemm_w4a8(_p(a_fp8), float(a_scale), _p(w_codes), _p(w_scales), M, N, K, _p(out), ld, _stream()))
    return out


def gemm_bf16(a, w, out=None):
    """bf16 reference: A [M, K] x W [N, K]^T -> bf16 [M, N], fp32 accumulation."""
    _2d(a, "a")
    _2d(w, "w")
    _contig(a, "a", torch.bfloat16)
    M, K = a.shape
    N = w.shape[0]
    _contig(w, "w", torch.bfloat16, a.device, (N, K))
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
    _2d(a, "a")
    _2d(w, "w")
    if mode == "bf16":
        _contig(a, "a", torch.bfloat16)
        M, K = a.shape
        _contig(w, "w", torch.bfloat16, a.device, (w.shape[0], K))
    else:
        _contig(a, "a", torch.uint8)
        M = a.shape[0]
        K = a.shape[1] * (2 if mode == "w4a4" else 1)
        _mx_weights(w, w_scales, K, a.device)
        if mode == "w4a4":
            _contig(a_scales, "a_scales", torch.uint8, a.device, (M, K // 32))
    N = w.shape[0]
    if sink is None:
        sink = torch.empty(waves * 64, dtype=torch.float32, device=a.device)
    check_buffer(sink, "sink", torch.float32, device=a.device, min_numel=waves * 64)
    _check(lib.mxq_mfma_ceiling(_GEMM_MODES[mode], _p(a), _p(a_scales) if a_scales is not None else None, _p(w),
                                _p(w_scales) if w_scales is not None else None, M, N, K, waves, iters, _p(sink),
                                _stream()))
    return waves * iters * 16 * MFMA_FLOP[mode]


def sqnr_workspace_bytes(n: int) -> int:
    return int(lib.mxq_sqnr_workspace_bytes(n))


def sqnr(ref, test, workspace=None, out3=None) -> torch.Tensor:
    """Whole-output SQNR; returns a float64 GPU tensor [S, N, dB]."""
    _2d(ref, "ref")
    check_buffer(ref, "ref", torch.bfloat16)
    ldr = _rowmajor(ref, "ref")
    R, C = ref.shape
    ldt = check_buffer(test, "test", torch.bfloat16, (R, C), ref.device)
    nbytes = sqnr_workspace_bytes(R * C)
    if workspace is None:
        workspace = torch.empty(nbytes // 8, dtype=torch.float64, device=ref.device)
    check_buffer(workspace, "workspace", torch.float64, device=ref.device, min_numel=nbytes // 8)
    if out3 is None:
        out3 = torch.empty(3, dtype=torch.float64, device=ref.device)
    check_buffer(out3, "out3", torch.float64, device=ref.device, min_numel=3)
    _check(lib.mxq_sqnr(_p(ref), _p(test), R, C, ldr, ldt, _p(workspace),
                        workspace.numel() * workspace.element_size(), _p(out3), _stream()))
    return out3


def sqnr_noalloc(ref, test, out3) -> torch.Tensor:
    """Whole-output SQNR into ``out3`` (float64 [3] on ref's device) with the library's
    own per-GPU workspace (mxq_sqnr_noalloc), for callers that cannot allocate device
    memory.  Calls on one GPU must not overlap."""
    _2d(ref, "ref")
    check_buffer(ref, "ref", torch.bfloat16)
    ldr = _rowmajor(ref, "ref")
    R, C = ref.shape
    ldt = check_buffer(test, "test", torch.bfloat16, (R, C), ref.device)
    check_buffer(out3, "out3", torch.float64, device=ref.device, min_numel=3)
    _check(lib.mxq_sqnr_noalloc(_p(ref), _p(test), R, C, ldr, ldt, _p(out3), _stream()))
    return out3


def dequantize(codes, scales, K: int, out=None) -> torch.Tensor:
    """MXFP4 -> bf16 [R, K] (into ``out`` if given: bfloat16 [R, K], rows may be strided)."""
    _2d(codes, "codes")
    R = codes.shape[0]
    ldc = check_buffer(codes, "codes", torch.uint8, (R, K // 2))
    lds = check_buffer(scales, "scales", torch.uint8, (R, K // 32), codes.device)
    if out is None:
        out = torch.empty((R, K), dtype=torch.bfloat16, device=codes.device)
    ld = check_buffer(out, "out", torch.bfloat16, (R, K), codes.device)
    _check(lib.mxq_dequantize(_p(codes), ldc, _p(scales), lds, R, K, _p(out), ld, _stream()))
    return out


def dequantize_fp8(q, a_scale: float, out=None) -> torch.Tensor:
    """FP8 E4M3 [R, K] -> bf16 [R, K]: bf16(fl32(e4m3(q) * a_scale)) (into ``out`` if given)."""
    _2d(q, "q")
    R, K = q.shape
    ldq = check_buffer(q, "q", torch.uint8, (R, K))
    if out is None:
        out = torch.empty((R, K), dtype=torch.bfloat16, device=q.device)
    ld = check_buffer(out, "out", torch.bfloat16, (R, K), q.device)
    _check(lib.mxq_dequantize_fp8(_p(q), ldq, float(a_scale), R, K, _p(out), ld, _stream()))
    return out
