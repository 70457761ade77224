"""GPU parity of the SQNR reduction (within 0.01 dB of the oracle; closed forms exact
to rounding) and of the whole W4A4 / W4A8 vs bf16 chain on a Wan2.2-shaped layer."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, bf16_from_bits, to_np_bf16_bits

pytestmark = pytest.mark.gpu


def _db(t):
    s, n, d = t.cpu().tolist()
    return s, n, d


@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 520), (2048, 5120), (75600, 64)])
def test_sqnr_matches_oracle(gpu, rows, cols):
    ref = workloads.activations(rows, cols, "student_t", seed=rows, name="sqnr_ref", device="cuda")
    noise = workloads.activations(rows, cols, "lognormal_channels", seed=cols, name="sqnr_n", device="cuda")
    test = (ref.float() + 0.05 * noise.float()).to(torch.bfloat16)
    announce(f"mxq_sqnr {rows}x{cols}")
    s, n, d = _db(gpu.sqnr(ref, test))
    rs, rn, rd = oracle.sqnr_db(to_np_bf16_bits(ref), to_np_bf16_bits(test))
    assert abs(d - rd) < 0.01 and abs(s - rs) <= 1e-6 * rs and abs(n - rn) <= 1e-5 * rn


def test_sqnr_closed_forms(gpu):
    ref = workloads.activations(300, 256, "student_t", seed=1, name="cf", device="cuda")
    half = (ref.float() / 2).to(torch.bfloat16)                 # exact: power of two
    assert abs(_db(gpu.sqnr(ref, half))[2] - 20 * math.log10(2)) < 1e-6
    assert abs(_db(gpu.sqnr(ref, torch.zeros_like(ref)))[2]) < 1e-6
    assert abs(_db(gpu.sqnr(ref, -ref))[2] + 20 * math.log10(2)) < 1e-6
    s, n, d = _db(gpu.sqnr(ref, ref))
    assert n == 0 and d == math.inf
    z = torch.zeros_like(ref)
    assert math.isnan(_db(gpu.sqnr(z, z))[2])


def test_sqnr_deterministic_and_strided(gpu):
    full = workloads.activations(1000, 1032, "student_t", seed=2, name="det", device="cuda")
    ref, test = full[:, :1024], full[:, 8:]
    r1 = gpu.sqnr(ref, test).clone()
    r2 = gpu.sqnr(ref, test).clone()
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    rs, rn, rd = oracle.sqnr_db(to_np_bf16_bits(ref), to_np_bf16_bits(test))
    assert abs(r1[2].item() - rd) < 0.01


@pytest.mark.parametrize("M", [2048])
def test_wan_down_chain_sqnr(gpu, M):
    """Wan2.2-shaped FFN down (K = 13824, N = 5120) at reduced M: quantize -> W4A4 / W4A8 ->
    SQNR against the bf16 reference, each side computing its own chain."""
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda", M=M)
    announce(f"chain sqnr M={M}")
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    s_a, inv_s = gpu.fp8_static_scales(float(gpu.absmax(a).item()))
    q8 = gpu.quantize_fp8(a, inv_s)
    ref = gpu.gemm_bf16(a, w)
    o44 = gpu.gemm_w4a4(ac, asc, wc, wsc)
    o48 = gpu.gemm_w4a8(q8, s_a, wc, wsc)
    d44 = _db(gpu.sqnr(ref, o44))[2]
    d48 = _db(gpu.sqnr(ref, o48))[2]
    torch.cuda.synchronize()
    ha, hw = bf16_bits_to_f32(to_np_bf16_bits(a)), bf16_bits_to_f32(to_np_bf16_bits(w))
    rac, ras = oracle.quantize_mxfp4(ha)
    rwc, rws = oracle.quantize_mxfp4(hw)
    rsa, rinv = oracle.fp8_static_scales(np.max(np.abs(ha)))
    rq = oracle.quantize_fp8(ha, rinv)
    r_ref = oracle.gemm.to_bf16(oracle.gemm_bf16(to_np_bf16_bits(a), to_np_bf16_bits(w))[0])
    r44 = oracle.gemm.to_bf16(oracle.gemm_w4a4(rac, ras, rwc, rws, wl.K)[0])
    r48 = oracle.gemm.to_bf16(oracle.gemm_w4a8(rq, rsa, rwc, rws, wl.K)[0])
    od44 = oracle.sqnr_db(r_ref, r44)[2]
    od48 = oracle.sqnr_db(r_ref, r48)[2]
    print(f"SQNR W4A4 gpu {d44:.4f} oracle {od44:.4f} | W4A8 gpu {d48:.4f} oracle {od48:.4f}", flush=True)
    assert abs(d44 - od44) < 0.01 and abs(d48 - od48) < 0.01
    assert d48 > d44            # FP8 activations keep more of the signal than MXFP4 ones


def test_sqnr_extreme_magnitudes(gpu):
    """Squares past binary32's range (|x| >= 2^64) and below its normal range (|x| <=
    2^-64) are formed in binary64: the dB matches the oracle."""
    rng = np.random.default_rng(44)
    for scale in (2.0 ** 100, 2.0 ** 120, 2.0 ** -100, 2.0 ** -126):
        ref = (rng.standard_normal((64, 256)) * scale).astype(np.float32)
        test = (ref * (1 + 0.01 * rng.standard_normal((64, 256)))).astype(np.float32)
        rb = oracle.f64_to_bf16_bits(ref.astype(np.float64))
        tb = oracle.f64_to_bf16_bits(test.astype(np.float64))
        announce(f"mxq_sqnr extreme scale 2^{math.log2(scale):.0f}")
        s, n, d = _db(gpu.sqnr(bf16_from_bits(rb), bf16_from_bits(tb)))
        rs, rn, rd = oracle.sqnr_db(rb, tb)
        assert math.isfinite(d) and abs(d - rd) < 1e-6, (scale, d, rd)
        assert abs(s - rs) <= 1e-12 * rs and abs(n - rn) <= 1e-12 * rn
