"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/mxq.h declares, validates arguments before launching anything, and reports a
HIP failure (no device) as MXQ_ERR_HIP with a message."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import mxfp4_microscaled_quantization_amd as mxq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")

P = ctypes.c_void_p
FAKE = P(0x10000)       # 16-byte aligned, never dereferenced (validation fails first or no GPU)
FAKE_ODD = P(0x10008)   # 8-byte but not 16-byte aligned


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mxq_status|size_t|const char\*|int)\s+(mxq_\w+)\s*\(", text, re.M)))


def test_header_declarations_match_binding():
    decl = _declared()
    assert decl == sorted(mxq.ABI_SYMBOLS), (decl, sorted(mxq.ABI_SYMBOLS))


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mxq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(mxq_\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name
        assert getattr(mxq.lib, name) is not None


def test_abi_version():
    """The header's MXQ_ABI_VERSION, the library's and the binding's agree."""
    header = open(os.path.join(ROOT, "include", "mxq.h")).read()
    declared = int(re.search(r"#define MXQ_ABI_VERSION (\d+)", header).group(1))
    assert mxq.lib.mxq_abi_version() == declared == mxq.ABI_VERSION == 2


def _err():
    return mxq.lib.mxq_last_error().decode()


@pytest.mark.parametrize("call,needle", [
    (lambda L: L.mxq_quantize(FAKE, 1, 4, 48, 48, FAKE, 32, FAKE, 2, None), "multiple of 32"),
    (lambda L: L.mxq_quantize(FAKE, 1, -1, 32, 32, FAKE, 16, FAKE, 1, None), "negative"),
    (lambda L: L.mxq_quantize(FAKE, 1, 4, 64, 32, FAKE, 32, FAKE, 2, None), "ld_x"),
    (lambda L: L.mxq_quantize(FAKE, 1, 4, 64, 64, FAKE, 16, FAKE, 2, None), "ld_codes"),
    (lambda L: L.mxq_quantize(FAKE, 1, 4, 64, 64, FAKE, 32, FAKE, 1, None), "ld_scales"),
    (lambda L: L.mxq_quantize(None, 1, 4, 64, 64, FAKE, 32, FAKE, 2, None), "NULL"),
    (lambda L: L.mxq_quantize(FAKE_ODD, 1, 4, 64, 64, FAKE, 32, FAKE, 2, None), "aligned"),
    (lambda L: L.mxq_quantize(FAKE, 1, 4, 64, 68, FAKE, 32, FAKE, 2, None), "aligned"),
    (lambda L: L.mxq_quantize(FAKE, 1, 4, 64, 64, FAKE_ODD, 32, FAKE, 2, None), "multiples of 16"),
    (lambda L: L.mxq_quantize_fp8(FAKE, 1, 4, 64, 64, ctypes.c_float(0.0), FAKE, 64, None), "inv_scale"),
    (lambda L: L.mxq_quantize_fp8(FAKE, 1, 4, 24, 24, ctypes.c_float(1.0), FAKE, 32, None), "multiple of 16"),
    (lambda L: L.mxq_quantize_fp8(FAKE, 1, 4, 64, 64, ctypes.c_float(1.0), FAKE, 48, None), "ld_q"),
    (lambda L: L.mxq_absmax(FAKE, 1, 4, 64, 64, None, None), "out"),
    (lambda L: L.mxq_gemm_w4a4(FAKE, FAKE, FAKE, FAKE, 8, 8, 48, FAKE, 8, None), "multiple of 32"),
    (lambda L: L.mxq_gemm_w4a4(FAKE, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 4, None), "ld_out"),
    (lambda L: L.mxq_gemm_w4a4(FAKE, FAKE, None, FAKE, 8, 8, 64, FAKE, 8, None), "w_codes is NULL"),
    (lambda L: L.mxq_gemm_w4a4(FAKE_ODD, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 8, None), "a_codes must be 16"),
    (lambda L: L.mxq_gemm_w4a4(FAKE, FAKE, FAKE, FAKE, -8, 8, 64, FAKE, 8, None), "negative"),
    (lambda L: L.mxq_gemm_w4a8(FAKE, ctypes.c_float(float("nan")), FAKE, FAKE, 8, 8, 64, FAKE, 8, None), "finite"),
    (lambda L: L.mxq_gemm_w4a8(FAKE, ctypes.c_float(1.0), FAKE, FAKE, 8, 8, 64, None, 8, None), "out is NULL"),
    (lambda L: L.mxq_gemm_bf16(FAKE, FAKE_ODD, 8, 8, 64, FAKE, 8, None), "w must be 16"),
    (lambda L: L.mxq_sqnr(FAKE, FAKE, 4, 12, 12, 12, FAKE, 1 << 20, FAKE, None), "multiple of 8"),
    (lambda L: L.mxq_sqnr(FAKE, FAKE, 4, 16, 16, 16, FAKE, 8, FAKE, None), "workspace"),
    (lambda L: L.mxq_sqnr(FAKE, FAKE, 4, 16, 16, 16, FAKE, 1 << 20, None, None), "out3"),
    (lambda L: L.mxq_sqnr_noalloc(FAKE, FAKE, 4, 12, 12, 12, FAKE, None), "multiple of 8"),
    (lambda L: L.mxq_sqnr_noalloc(FAKE, FAKE, 4, 16, 8, 16, FAKE, None), "pitch below"),
    (lambda L: L.mxq_sqnr_noalloc(FAKE, FAKE, 4, 16, 16, 16, None, None), "out3"),
    (lambda L: L.mxq_sqnr_noalloc(FAKE_ODD, FAKE, 4, 16, 16, 16, FAKE, None), "16-byte"),
    (lambda L: L.mxq_dequantize(FAKE, 16, FAKE, 1, 4, 48, FAKE, 48, None), "multiple of 32"),
    (lambda L: L.mxq_dequantize_fp8(FAKE, 24, ctypes.c_float(1.0), 4, 24, FAKE, 24, None), "multiple of 16"),
    (lambda L: L.mxq_dequantize_fp8(FAKE, 16, ctypes.c_float(1.0), 4, 32, FAKE, 32, None), "pitch"),
    (lambda L: L.mxq_dequantize_fp8(FAKE, 32, ctypes.c_float(float("inf")), 4, 32, FAKE, 32, None), "finite"),
    (lambda L: L.mxq_dequantize_fp8(FAKE_ODD, 32, ctypes.c_float(1.0), 4, 32, FAKE, 32, None), "multiples of 16"),
    (lambda L: L.mxq_dequantize_fp8(FAKE, 32, ctypes.c_float(1.0), 4, 32, FAKE_ODD, 32, None), "16-byte"),
    (lambda L: L.mxq_dequantize_fp8(None, 32, ctypes.c_float(1.0), 4, 32, FAKE, 32, None), "NULL"),
    (lambda L: L.mxq_quantize_rule(FAKE, 1, 4, 48, 48, FAKE, 32, FAKE, 2, 1, None), "multiple of 32"),
    (lambda L: L.mxq_quantize_hadamard(FAKE, 1, 4, 96, 96, 64, 0, FAKE, 48, FAKE, 3, None), "multiple of block_n"),
    (lambda L: L.mxq_quantize_hadamard(FAKE, 1, 4, 64, 64, 64, 0, FAKE, 16, FAKE, 2, None), "ld_codes"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 48, FAKE, FAKE, 8, 8, 48, 0, FAKE, 8, None, 0, None), "multiple of 32"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 32, FAKE, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "ld_x"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 68, FAKE, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "aligned"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE_ODD, 1, 64, FAKE, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "aligned"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 0, 1 << 21, FAKE, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "row pitch"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 64, None, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "w_codes is NULL"),
    (lambda L: L.mxq_gemm_w4a4_fused(None, 1, 64, FAKE, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "NULL"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 64, FAKE, FAKE, 8, 8, 64, 0, FAKE, 4, None, 0, None), "ld_out"),
    # past the fused kernel's break-even, a workspace that is too small or misaligned
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 8192, FAKE, FAKE, 8, 1024, 8192, 0, FAKE, 1024, FAKE, 16, None),
     "workspace"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 8192, FAKE, FAKE, 8, 1024, 8192, 0, FAKE, 1024, FAKE_ODD, 1 << 20,
                                     None), "workspace"),
    (lambda L: L.mxq_mfma_ceiling(0, FAKE, FAKE, FAKE, FAKE, 8, 8, 48, 4, 1, FAKE, None), "multiple of 32"),
    (lambda L: L.mxq_mfma_ceiling(0, FAKE, FAKE, FAKE, FAKE, 0, 8, 64, 4, 1, FAKE, None), "M, N >= 1"),
    (lambda L: L.mxq_mfma_ceiling(0, FAKE, FAKE, FAKE, FAKE, 8, 8, 64, 6, 1, FAKE, None), "waves"),
    (lambda L: L.mxq_mfma_ceiling(0, FAKE, FAKE, FAKE, FAKE, 8, 8, 64, 4, 0, FAKE, None), "iters"),
    (lambda L: L.mxq_mfma_ceiling(0, FAKE, None, FAKE, FAKE, 8, 8, 64, 4, 1, FAKE, None), "a_scales is NULL"),
    (lambda L: L.mxq_mfma_ceiling(1, FAKE, None, FAKE, None, 8, 8, 64, 4, 1, FAKE, None), "w_scales is NULL"),
    (lambda L: L.mxq_mfma_ceiling(2, FAKE_ODD, None, FAKE, None, 8, 8, 64, 4, 1, FAKE, None), "aligned"),
    (lambda L: L.mxq_mfma_ceiling(2, FAKE, None, FAKE, None, 8, 8, 64, 4, 1, None, None), "sink"),
])
def test_invalid_arguments_are_rejected_before_launch(call, needle):
    st = call(mxq.lib)
    assert st == mxq.MXQ_ERR_INVALID_ARG, (st, _err())
    assert needle in _err()


def test_unknown_dtype_is_unsupported():
    st = mxq.lib.mxq_quantize(FAKE, 7, 4, 64, 64, FAKE, 32, FAKE, 2, None)
    assert st == mxq.MXQ_ERR_UNSUPPORTED and "dtype" in _err()


@pytest.mark.parametrize("call,needle", [
    (lambda L: L.mxq_quantize_rule(FAKE, 1, 4, 64, 64, FAKE, 32, FAKE, 2, 5, None), "scale rule"),
    (lambda L: L.mxq_quantize_hadamard(FAKE, 1, 4, 64, 64, 32, 0, FAKE, 32, FAKE, 2, None), "block_n"),
    (lambda L: L.mxq_quantize_hadamard(FAKE, 1, 4, 64, 64, 64, 3, FAKE, 32, FAKE, 2, None), "scale rule"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 1, 64, FAKE, FAKE, 8, 8, 64, 2, FAKE, 8, None, 0, None), "scale rule"),
    (lambda L: L.mxq_gemm_w4a4_fused(FAKE, 9, 64, FAKE, FAKE, 8, 8, 64, 0, FAKE, 8, None, 0, None), "dtype"),
    (lambda L: L.mxq_mfma_ceiling(3, FAKE, FAKE, FAKE, FAKE, 8, 8, 64, 4, 1, FAKE, None), "mode"),
])
def test_unknown_rule_or_block_is_unsupported(call, needle):
    st = call(mxq.lib)
    assert st == mxq.MXQ_ERR_UNSUPPORTED and needle in _err(), (st, _err())


def test_empty_problems_are_noops():
    assert mxq.lib.mxq_quantize(None, 1, 0, 64, 64, None, 32, None, 2, None) == mxq.MXQ_OK
    assert mxq.lib.mxq_gemm_w4a4(None, None, None, None, 0, 8, 64, None, 8, None) == mxq.MXQ_OK
    assert mxq.lib.mxq_gemm_w4a8(None, ctypes.c_float(1.0), None, None, 8, 0, 64, None, 0, None) == mxq.MXQ_OK
    assert mxq.lib.mxq_gemm_w4a4_fused(None, 1, 64, None, None, 0, 8, 64, 0, None, 8, None, 0, None) == mxq.MXQ_OK
    assert _err() == ""


@pytest.mark.parametrize("M,N,K,routes", [
    (75600, 5120, 13824, True), (75600, 768, 13824, False), (75600, 769, 13824, True),
    (57344, 12288, 3072, True), (57344, 256, 3072, False), (57344, 257, 3072, True),
    (57344, 768, 8192, False), (57344, 1024, 8192, True), (0, 4096, 8192, False), (8, 4096, 48, False)])
def test_fused_workspace_follows_the_break_even(M, N, K, routes):
    n = mxq.lib.mxq_gemm_w4a4_fused_workspace_bytes(M, N, K)
    assert mxq.fused_workspace_bytes(M, N, K) == n
    if routes:
        assert n == -(-(M * K // 2) // 16) * 16 + M * K // 32
    else:
        assert n == 0


def test_workspace_size_is_fixed_and_small():
    n = mxq.lib.mxq_sqnr_workspace_bytes(75600 * 5120)
    assert 0 < n <= 1 << 16 and n == mxq.lib.mxq_sqnr_workspace_bytes(16)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device failure path")
def test_launch_without_gpu_reports_hip_error():
    st = mxq.lib.mxq_quantize(FAKE, 1, 4, 64, 64, FAKE, 32, FAKE, 2, None)
    assert st == mxq.MXQ_ERR_HIP
    assert "HIP error" in _err()
    with pytest.raises(mxq.MxqError):
        mxq._check(st)


def _amax_set():
    rng = np.random.default_rng(6)
    return np.concatenate([rng.uniform(0.1, 1000, 300), rng.lognormal(0, 20, 300),
                           [448.0, 1.0, 3e-5, 7e20, 3.0e38, np.finfo(np.float32).max, 1.5e-36,
                            np.finfo(np.float32).tiny, 448.0 / np.finfo(np.float32).max * 1.0001]]).astype(np.float32)


def test_fp8_static_scales_match_the_oracle():
    """The library's static scales (a host computation, no GPU) equal the oracle's
    correctly rounded quotients on the oracle's pinned amax set and wider magnitudes."""
    for amax in _amax_set():
        if not (448.0 / np.float64(amax) <= np.finfo(np.float32).max):
            continue
        s_a, inv_s = ctypes.c_float(), ctypes.c_float()
        assert mxq.lib.mxq_fp8_static_scales(ctypes.c_float(amax), ctypes.byref(s_a), ctypes.byref(inv_s)) == 0
        rs, ri = oracle.fp8_static_scales(amax)
        assert np.float32(s_a.value) == rs and np.float32(inv_s.value) == ri, amax
        assert mxq.fp8_static_scales(float(amax)) == (float(rs), float(ri))


@pytest.mark.parametrize("amax", [0.0, -1.0, float("inf"), float("-inf"), float("nan"), 1e-40, 4e-45])
def test_fp8_static_scales_rejects_bad_amax(amax):
    s_a, inv_s = ctypes.c_float(-7.0), ctypes.c_float(-7.0)
    st = mxq.lib.mxq_fp8_static_scales(ctypes.c_float(amax), ctypes.byref(s_a), ctypes.byref(inv_s))
    assert st == mxq.MXQ_ERR_INVALID_ARG and "amax" in _err()
    assert s_a.value == -7.0 and inv_s.value == -7.0          # outputs untouched on error
    with pytest.raises(mxq.MxqError):
        mxq.fp8_static_scales(amax)


def test_fp8_static_scales_rejects_null_outputs():
    out = ctypes.c_float()
    assert mxq.lib.mxq_fp8_static_scales(ctypes.c_float(1.0), None, ctypes.byref(out)) == mxq.MXQ_ERR_INVALID_ARG
    assert mxq.lib.mxq_fp8_static_scales(ctypes.c_float(1.0), ctypes.byref(out), None) == mxq.MXQ_ERR_INVALID_ARG
