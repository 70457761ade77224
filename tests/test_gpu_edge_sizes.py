"""Degenerate sizes on every entry point, through the binding and the C ABI on the GPU:
empty row counts, empty column counts and K = 0.  Each call must succeed and be a no-op
(nothing written outside an empty output), except that a GEMM with K = 0 writes zeros
(an empty sum) and the SQNR of empty tensors is S = N = 0, dB = NaN (the 0/0 case of the
SQNR definition, as in the oracle)."""

import math

import numpy as np
import pytest
import torch

import oracle
from helpers import announce

pytestmark = pytest.mark.gpu


def _bf16(r, c):
    return torch.randn(r, c, device="cuda").to(torch.bfloat16)


def test_quantizers_on_empty_rows(gpu):
    announce("edge sizes: quantizers, 0 rows")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    for rule in ("ocp", "uos"):
        c, s = gpu.quantize(x, rule)
        assert c.shape == (0, 128) and s.shape == (0, 8)
    for n in (16, 64, 256):
        c, s = gpu.quantize_hadamard(x, n)
        assert c.shape == (0, 128) and s.shape == (0, 8)
    q = gpu.quantize_fp8(x, 1.0)
    assert q.shape == (0, 256)
    x32 = torch.empty(0, 256, dtype=torch.float32, device="cuda")
    c, s = gpu.quantize(x32)
    assert c.shape == (0, 128)
    torch.cuda.synchronize()


def test_dequantizers_on_empty_rows(gpu):
    announce("edge sizes: dequantizers, 0 rows")
    c = torch.empty(0, 128, dtype=torch.uint8, device="cuda")
    s = torch.empty(0, 8, dtype=torch.uint8, device="cuda")
    y = gpu.dequantize(c, s, 256)
    assert y.shape == (0, 256)
    y8 = gpu.dequantize_fp8(torch.empty(0, 256, dtype=torch.uint8, device="cuda"), 0.5)
    assert y8.shape == (0, 256)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N", [(0, 96), (80, 0), (0, 0)])
def test_gemms_on_empty_m_or_n(gpu, M, N):
    announce(f"edge sizes: GEMMs M={M} N={N}")
    K = 256
    a, w = _bf16(M, K), _bf16(N, K)
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    assert gpu.gemm_w4a4(ac, asc, wc, wsc).shape == (M, N)
    assert gpu.gemm_w4a4_fused(a, wc, wsc).shape == (M, N)
    assert gpu.gemm_w4a4_fused(a, wc, wsc, route=False).shape == (M, N)
    a8 = gpu.quantize_fp8(a, 1.0)
    assert gpu.gemm_w4a8(a8, 1.0, wc, wsc).shape == (M, N)
    assert gpu.gemm_bf16(a, w).shape == (M, N)
    torch.cuda.synchronize()


def test_gemms_with_k_zero_write_zeros(gpu):
    announce("edge sizes: GEMMs K=0")
    M, N = 37, 70
    a = torch.empty(M, 0, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(N, 0, dtype=torch.bfloat16, device="cuda")
    codes_a = torch.empty(M, 0, dtype=torch.uint8, device="cuda")
    codes_w = torch.empty(N, 0, dtype=torch.uint8, device="cuda")
    for name, call in (
        ("w4a8", lambda out: gpu.gemm_w4a8(codes_a, 1.0, codes_w, codes_w, out=out)),
        ("bf16", lambda out: gpu.gemm_bf16(a, w, out=out)),
        ("w4a4_fused", lambda out: gpu.gemm_w4a4_fused(a, codes_w, codes_w, out=out, route=False)),
    ):
        out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        call(out)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out.float()) == 0, name


def test_sqnr_of_empty_tensors_is_nan(gpu):
    announce("edge sizes: SQNR of 0 x 64")
    e = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    r = gpu.sqnr(e, e)
    torch.cuda.synchronize()
    s, n, db = (float(v) for v in r.cpu())
    assert s == 0.0 and n == 0.0 and math.isnan(db)
    rs, rn, rdb = oracle.sqnr_db(np.zeros((0, 64), np.uint16), np.zeros((0, 64), np.uint16))
    assert rs == 0.0 and rn == 0.0 and math.isnan(rdb)
