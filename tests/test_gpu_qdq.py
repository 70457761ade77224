"""GPU parity of the quantize-dequantize (QDQ) emulation path against the oracle.

"AMD Quark adds native W4A8 mixed-precision for Wan2.2 ...", section "Quark quantization
pipeline and mixed-precision selection": the W4A8 quality figures come from QDQ
emulation -- operands quantized, dequantized back to the compute type, then multiplied
by an ordinary bf16 GEMM -- not from native kernels.  The chains here:
    QDQ-W4A4: mxq_quantize (A, W) -> mxq_dequantize (A, W) -> mxq_gemm_bf16
    QDQ-W4A8: mxq_quantize_fp8 (A) -> mxq_dequantize_fp8 (A, x s_a); mxq_quantize ->
              mxq_dequantize (W) -> mxq_gemm_bf16
The dequantization steps are bit-exact against the oracle; the chain outputs are held to
the GEMM bar against the oracle's own chain (oracle quantize -> oracle dequantize ->
float64 GEMM of the dequantized bf16 operands).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, to_np_bf16_bits

pytestmark = pytest.mark.gpu


def _assert_tol(got_bits, out, tot, label):
    ok, err, bound = oracle.within_tolerance(got_bits, out, tot)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())}/{ok.size} outside tolerance; first at {i}: "
                             f"err {err[i]:.3e} bound {bound[i]:.3e}")


@pytest.mark.parametrize("s_a", [1.0, 0.0078125, 2.2321430606098147e-06, 0.3171, -0.5, 1e30, 2.0 ** -130])
def test_dequantize_fp8_every_code(gpu, s_a):
    codes = np.tile(np.arange(256, dtype=np.uint8), (3, 1))             # [3, 256]
    s = np.float32(s_a)
    announce(f"mxq_dequantize_fp8 exhaustive s_a={s_a}")
    y = gpu.dequantize_fp8(torch.from_numpy(codes).cuda(), float(s))
    torch.cuda.synchronize()
    got = to_np_bf16_bits(y)
    ref = oracle.dequantize_fp8(codes, s)
    nan = (codes & 0x7F) == 0x7F
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)   # NaN


def test_dequantize_fp8_workload_rows_ragged_and_strided(gpu):
    name = "wan_ffn_up_w4a8"
    a = workloads.activations(777, 5120 - 16, "lognormal_channels", seed=1, name=name, device="cpu")
    host = bf16_bits_to_f32(to_np_bf16_bits(a))
    s_a, inv_s = oracle.fp8_static_scales(np.max(np.abs(host)))
    q = oracle.quantize_fp8(host, inv_s)
    qg = torch.from_numpy(q).cuda()
    announce("mxq_dequantize_fp8 workload rows, strided output")
    y = gpu.dequantize_fp8(qg, float(s_a))
    full = torch.full((777, q.shape[1] + 48), 3.0, dtype=torch.bfloat16, device="cuda")
    gpu.dequantize_fp8(qg, float(s_a), out=full[:, :q.shape[1]])
    torch.cuda.synchronize()
    ref = oracle.dequantize_fp8(q, s_a)
    np.testing.assert_array_equal(to_np_bf16_bits(y), ref)
    np.testing.assert_array_equal(to_np_bf16_bits(full[:, :q.shape[1]]), ref)
    assert bool((full[:, q.shape[1]:] == 3.0).all())


def _mx_dq_bits(codes, scales, K):
    return oracle.f64_to_bf16_bits(oracle.dequantize_mxfp4(codes, scales, K))


def _qdq_w4a4(gpu, a, w):
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    K = a.shape[1]
    return gpu.gemm_bf16(gpu.dequantize(ac, asc, K), gpu.dequantize(wc, wsc, K))


def _qdq_w4a8(gpu, a, w):
    s_a, inv_s = gpu.fp8_static_scales(float(gpu.absmax(a).item()))
    q = gpu.quantize_fp8(a, inv_s)
    wc, wsc = gpu.quantize(w)
    return gpu.gemm_bf16(gpu.dequantize_fp8(q, s_a), gpu.dequantize(wc, wsc, a.shape[1])), s_a


def _oracle_w4a4(a_host, w_host, K):
    rac, ras = oracle.quantize_mxfp4(a_host)
    rwc, rws = oracle.quantize_mxfp4(w_host)
    return oracle.gemm_bf16(_mx_dq_bits(rac, ras, K), _mx_dq_bits(rwc, rws, K))


def _oracle_w4a8(a_host, w_host, K):
    rs_a, rinv = oracle.fp8_static_scales(np.max(np.abs(a_host)))
    rq = oracle.quantize_fp8(a_host, rinv)
    rwc, rws = oracle.quantize_mxfp4(w_host)
    return oracle.gemm_bf16(oracle.dequantize_fp8(rq, rs_a), _mx_dq_bits(rwc, rws, K)), rs_a


@pytest.mark.parametrize("M,N,K,dist", [(300, 520, 416, "lognormal_channels"), (513, 257, 1024, "student_t"),
                                        (64, 96, 96, "lognormal_channels"), (260, 300, 3072, "student_t")])
def test_qdq_chains_match_the_oracle_chain(gpu, M, N, K, dist):
    a = workloads.activations(M, K, dist, seed=M, name="qdq", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=N, name="qdq", device="cuda")
    announce(f"qdq chains {M}x{N}x{K} {dist}")
    o4 = _qdq_w4a4(gpu, a, w)
    o8, s_a = _qdq_w4a8(gpu, a, w)
    torch.cuda.synchronize()
    ah, wh = bf16_bits_to_f32(to_np_bf16_bits(a)), bf16_bits_to_f32(to_np_bf16_bits(w))
    ref4, tot4 = _oracle_w4a4(ah, wh, K)
    _assert_tol(to_np_bf16_bits(o4), ref4, tot4, "qdq-w4a4")
    (ref8, tot8), rs_a = _oracle_w4a8(ah, wh, K)
    assert np.float32(s_a) == rs_a
    _assert_tol(to_np_bf16_bits(o8), ref8, tot8, "qdq-w4a8")


def test_qdq_w4a4_equals_native_w4a4_within_the_bar(gpu):
    """MXFP4 values are exact in bf16 (2 significant bits, scales inside bf16's range), so
    the QDQ-W4A4 chain computes the native W4A4 sum: both are held to the same oracle."""
    M, N, K = 513, 300, 2048
    a = workloads.activations(M, K, "student_t", seed=9, name="qdq-native", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=9, name="qdq-native", device="cuda")
    announce("qdq w4a4 vs native")
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    native = gpu.gemm_w4a4(ac, asc, wc, wsc)
    qdq = gpu.gemm_bf16(gpu.dequantize(ac, asc, K), gpu.dequantize(wc, wsc, K))
    torch.cuda.synchronize()
    rac, ras = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(a)))
    rwc, rws = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(w)))
    ref, tot = oracle.gemm_w4a4(rac, ras, rwc, rws, K)
    _assert_tol(to_np_bf16_bits(native), ref, tot, "native")
    _assert_tol(to_np_bf16_bits(qdq), ref, tot, "qdq")


def test_qdq_full_size_sampled(gpu):
    """The Wan2.2 FFN-down workload at full size through both QDQ chains, sampled rows
    against the oracle chain (the static scale from the whole tensor's amax)."""
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda")
    announce("qdq full size")
    o4 = _qdq_w4a4(gpu, a, w)
    o8, s_a = _qdq_w4a8(gpu, a, w)
    amax = float(gpu.absmax(a).item())
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([rng.integers(0, wl.M, 24), [0, wl.M - 1]]))
    ri = torch.from_numpy(rows).cuda()
    ah = bf16_bits_to_f32(to_np_bf16_bits(a.index_select(0, ri)))
    wh = bf16_bits_to_f32(to_np_bf16_bits(w))
    rac, ras = oracle.quantize_mxfp4(ah)
    rwc, rws = oracle.quantize_mxfp4(wh)
    wdq = _mx_dq_bits(rwc, rws, wl.K)
    ref4, tot4 = oracle.gemm_bf16(_mx_dq_bits(rac, ras, wl.K), wdq)
    _assert_tol(to_np_bf16_bits(o4.index_select(0, ri)), ref4, tot4, "qdq-w4a4 full")
    rs_a, rinv = oracle.fp8_static_scales(amax)
    assert np.float32(s_a) == rs_a
    ref8, tot8 = oracle.gemm_bf16(oracle.dequantize_fp8(oracle.quantize_fp8(ah, rinv), rs_a), wdq)
    _assert_tol(to_np_bf16_bits(o8.index_select(0, ri)), ref8, tot8, "qdq-w4a8 full")
