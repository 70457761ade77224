"""The scaled GEMMs on outputs of 17.2M elements (4252 x 4036: 17 x 16 tiles of 256 x 256
with ragged M and N, once with a last column tile wider than half a tile and once
narrower), against the oracle element by element, and the last m-tile's rows
bit-identical to the same GEMM run on those rows alone (a different launch shape and
tile order must not change a bit); for W4A4 also the fused entry point, which runs its
own kernel, bit-identical to quantize + GEMM.

W4A4 meets the bar on every output.  W4A8 (the Wan2.2 FFN-up activation model at its own
K = 5120) is held to what the hardware allows at this scale: the FP8 x FP4 MFMA's
alignment of each group of 8 products leaves a few outputs per million with heavy
cancellation above the bar, so at most 1 in 10^5 outputs may exceed it, by less than 3x
(measured here: 7 outside, at most 1.91x).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, to_np_bf16_bits

pytestmark = pytest.mark.gpu

SHAPES = [(4252, 4036), (4252, 3940)]


def _host_f32(t):
    from helpers import bf16_bits_to_f32
    return bf16_bits_to_f32(to_np_bf16_bits(t))


def _assert_tol(out, ref, tot, label):
    ok, err, bound = oracle.within_tolerance(to_np_bf16_bits(out), ref, tot)
    assert ok.all(), f"{label}: {int((~ok).sum())}/{ok.size} outside the bar"


def _last_rows(M):
    return (((M + 255) // 256) - 1) * 256


@pytest.mark.parametrize("M,N", SHAPES)
def test_w4a4_large_output(gpu, M, N):
    K = 512                      # the fast path needs scale rows of a multiple of 16 bytes
    a = workloads.activations(M, K, "lognormal_channels", seed=M + N, name="large", device="cuda")
    w = workloads.weights(N, K, 0.02, seed=N, name="large", device="cuda")
    announce(f"w4a4 large output M={M} N={N} K={K}")
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    out = gpu.gemm_w4a4(ac, asc, wc, wsc)
    r0 = _last_rows(M)
    sub = gpu.gemm_w4a4(ac[r0:].contiguous(), asc[r0:].contiguous(), wc, wsc)
    fused = gpu.gemm_w4a4_fused(a, wc, wsc, route=False)
    torch.cuda.synchronize()
    assert torch.equal(out[r0:].view(torch.int16), sub.view(torch.int16)), "the last m-tile differs when run alone"
    assert torch.equal(out.view(torch.int16), fused.view(torch.int16)), "the fused kernel differs from quantize + GEMM"
    rac, ras = oracle.quantize_mxfp4(_host_f32(a))
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w))
    ref, tot = oracle.gemm_w4a4(rac, ras, rwc, rws, K)
    _assert_tol(out, ref, tot, f"w4a4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N", SHAPES)
def test_w4a8_large_output(gpu, M, N):
    K = 5120                     # the Wan2.2 FFN-up activation model at its own K
    a = workloads.activations(M, K, "lognormal_channels", seed=M + N, name="large", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=N, name="large", device="cuda")
    announce(f"w4a8 large output M={M} N={N} K={K}")
    s_a, inv_s = gpu.fp8_static_scales(float(gpu.absmax(a).item()))
    q = gpu.quantize_fp8(a, inv_s)
    wc, wsc = gpu.quantize(w)
    out = gpu.gemm_w4a8(q, s_a, wc, wsc)
    r0 = _last_rows(M)
    sub = gpu.gemm_w4a8(q[r0:].contiguous(), s_a, wc, wsc)
    torch.cuda.synchronize()
    assert torch.equal(out[r0:].view(torch.int16), sub.view(torch.int16)), "the last m-tile differs when run alone"
    host = _host_f32(a)
    rs_a, rinv = oracle.fp8_static_scales(np.max(np.abs(host)))
    rq = oracle.quantize_fp8(host, rinv)
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w))
    ref, tot = oracle.gemm_w4a8(rq, rs_a, rwc, rws, K)
    ok, err, bound = oracle.within_tolerance(to_np_bf16_bits(out), ref, tot)
    outside, worst = int((~ok).sum()), float(np.max(err / bound))
    print(f"W4A8 {M}x{N}x{K} lognormal: {outside}/{ok.size} outside the bar, worst {worst:.3f}x", flush=True)
    assert np.isfinite(bound).all() and outside <= ok.size * 1e-5 and worst < 3.0
