"""GPU parity of the W4A4 GEMM with the activation quantization fused in (mxq_gemm_w4a4_fused).

The fused call must equal mxq_quantize_rule followed by mxq_gemm_w4a4, bit for bit, and
therefore the oracle's chain (quantize_mxfp4, gemm_w4a4) within the GEMM bar.

* identity weights make every output one dequantized activation code: with W = I (codes
  of 1.0) the output is exactly e2m1(code) * 2^(s_a - 127) * 2^(s_w - 127), so the fused
  quantizer is checked element by element against the oracle's quantizer -- every
  finite bf16 pattern as a block maximum (fast bf16 path and generic bf16 path), binary32
  over a wide range (generic binary32 path), both scale rules; two weight scales keep
  every product normal and finite in one of the runs;
* bit-identity with the unfused chain on tile-spanning shapes with ragged M / N tails,
  2 to 54 K-windows, row-strided activations and outputs, K off the fast path, binary32
  activations, both rules, the Wan2.2 FFN-down workload at reduced size and the Wan2.2
  FFN-down and FLUX FFN-up / FFN-down workloads at full size;
* the oracle chain within the bar on the tiny workload (binary32) and sampled outputs;
* the call with a workspace, on both sides of the break-even where it routes to the
  separate quantization pass: the same bits as the fused kernel and the chain.

The tests of the fused kernel itself call it with route=False (no workspace).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, bf16_from_bits, to_np_bf16_bits, u8_to_gpu

pytestmark = pytest.mark.gpu


def _identity_weights(K, s_w):
    """W = I (N = K): element n of row n is the E2M1 code of 1.0 (0x2), all scales s_w."""
    codes = np.zeros((K, K // 2), np.uint8)
    n = np.arange(K)
    codes[n, n // 2] = np.where(n % 2 == 0, 0x02, 0x20).astype(np.uint8)
    scales = np.full((K, K // 32), s_w, np.uint8)
    return u8_to_gpu(codes), u8_to_gpu(scales)


def _check_identity(mxq, a_gpu, a_host_f32, rule, label):
    """Fused output against the oracle's dequantized codes, exactly, with W = I."""
    M, K = a_gpu.shape
    rc, rs = oracle.quantize_mxfp4(a_host_f32, rule)
    deq = oracle.dequantize_mxfp4(rc, rs, K).astype(np.float64)
    covered = np.zeros(deq.shape, bool)
    for s_w in (191, 63):                      # x 2^64 and x 2^-64
        wc, wsc = _identity_weights(K, s_w)
        announce(f"fused identity {label} {rule} s_w={s_w} M={M} K={K} {a_gpu.dtype}")
        out = mxq.gemm_w4a4_fused(a_gpu, wc, wsc, rule, route=False)
        torch.cuda.synchronize()
        got = bf16_bits_to_f32(to_np_bf16_bits(out)).astype(np.float64)
        want = deq * 2.0 ** (s_w - 127)
        exact = (want == 0) | ((np.abs(want) >= 2.0 ** -126) & (np.abs(want) < 2.0 ** 128))
        bad = np.nonzero(exact & (got != want))
        assert bad[0].size == 0, (f"{label} s_w={s_w}: {bad[0].size} mismatches, first at "
                                  f"{bad[0][0]},{bad[1][0]}: got {got[bad[0][0], bad[1][0]]!r} "
                                  f"want {want[bad[0][0], bad[1][0]]!r}")
        covered |= exact
    assert covered.all()


def _bf16_maxima_rows(K, seed):
    """Every finite non-negative bf16 pattern as a 32-element block maximum (random
    sign), with a random body of smaller magnitude, as rows of K elements."""
    rng = np.random.default_rng(seed)
    pats = np.arange(0, 0x7F80, dtype=np.uint32)
    n = pats.size
    anchor = (pats | (rng.integers(0, 2, n, dtype=np.uint32) << 15)).astype(np.uint16)
    body_mag = (rng.random((n, 31)) * (pats[:, None].astype(np.float64) + 1)).astype(np.uint32)
    body = (body_mag | (rng.integers(0, 2, (n, 31), dtype=np.uint32) << 15)).astype(np.uint16)
    blocks = np.concatenate([anchor[:, None], body], axis=1)
    blocks = np.take_along_axis(blocks, rng.permuted(np.tile(np.arange(32), (n, 1)), axis=1), axis=1)
    per_row = K // 32
    pad = (-n) % per_row
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.uint16)])
    return blocks.reshape(-1, K)


@pytest.mark.parametrize("K", [512, 768])            # fast path, generic bf16 path
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_fused_quantizer_every_bf16_maximum_through_identity(gpu, K, rule):
    bits = _bf16_maxima_rows(K, 51 + K)
    _check_identity(gpu, bf16_from_bits(bits), bf16_bits_to_f32(bits), rule, f"bf16 maxima K={K}")


@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_fused_quantizer_binary32_through_identity(gpu, rule):
    rng = np.random.default_rng(52)
    M, K = 512, 256
    m = rng.uniform(1, 2, (M, K)) * rng.choice([-1, 1], (M, K))
    e = rng.integers(-140, 120, (M, K // 32)).repeat(32, axis=1) + rng.integers(-8, 1, (M, K))
    x = np.ldexp(m, e).astype(np.float32)
    x[rng.random((M, K)) < 0.02] = 0.0
    _check_identity(gpu, torch.from_numpy(x).cuda(), x, rule, "binary32")


def _chain(mxq, a, wc, wsc, rule):
    ac, asc = mxq.quantize(a, rule=rule)
    return mxq.gemm_w4a4(ac, asc, wc, wsc)


def _assert_same(got, want, label):
    g, w = to_np_bf16_bits(got), to_np_bf16_bits(want)
    bad = np.nonzero(g != w)
    assert bad[0].size == 0, f"{label}: {bad[0].size} outputs differ, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (513, 257, 1024), (260, 300, 1536), (256, 512, 2048),
                                   (64, 96, 768), (1, 1, 32), (130, 70, 288)])
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_fused_bit_identical_to_quantize_then_gemm(gpu, M, N, K, rule):
    g = torch.Generator(device="cuda").manual_seed(M * 7 + N * 3 + K)
    a = (torch.randn(M, K, device="cuda", generator=g) * torch.exp(torch.randn(1, K, device="cuda", generator=g)))
    a = a.to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    wc, wsc = gpu.quantize(w)
    announce(f"fused vs chain {rule} M={M} N={N} K={K}")
    out = gpu.gemm_w4a4_fused(a, wc, wsc, rule, route=False)
    ref = _chain(gpu, a, wc, wsc, rule)
    torch.cuda.synchronize()
    _assert_same(out, ref, f"{M}x{N}x{K} {rule}")


def test_fused_strided_activations_and_output(gpu):
    M, N, K = 300, 260, 1024
    g = torch.Generator(device="cuda").manual_seed(5)
    full = (torch.randn(M, K + 64, device="cuda", generator=g) * 3).to(torch.bfloat16)
    a = full[:, :K]
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    wc, wsc = gpu.quantize(w)
    out_full = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    announce("fused strided A and out")
    gpu.gemm_w4a4_fused(a, wc, wsc, out=out_full[:, :N], route=False)
    ref = _chain(gpu, a.contiguous(), wc, wsc, "ocp")
    torch.cuda.synchronize()
    _assert_same(out_full[:, :N], ref, "strided")
    assert bool((out_full[:, N:] == 7.0).all()), "fused call wrote past the output columns"


def test_fused_binary32_activations(gpu):
    M, N, K = 200, 130, 640
    g = torch.Generator(device="cuda").manual_seed(6)
    a = torch.randn(M, K, device="cuda", generator=g) * 4
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    wc, wsc = gpu.quantize(w)
    announce("fused binary32 activations")
    out = gpu.gemm_w4a4_fused(a, wc, wsc, route=False)
    ref = _chain(gpu, a, wc, wsc, "ocp")
    torch.cuda.synchronize()
    _assert_same(out, ref, "binary32")


def test_fused_tiny_workload_against_oracle(gpu):
    a, w = workloads.tiny_inputs(0)
    ta, tw = torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda()
    wc, wsc = gpu.quantize(tw)
    announce("fused tiny workload")
    out = gpu.gemm_w4a4_fused(ta, wc, wsc, route=False)
    torch.cuda.synchronize()
    rac, ras = oracle.quantize_mxfp4(a)
    rwc, rws = oracle.quantize_mxfp4(w)
    ref, tot = oracle.gemm_w4a4(rac, ras, rwc, rws, a.shape[1])
    ok, _, _ = oracle.within_tolerance(to_np_bf16_bits(out), ref, tot)
    assert ok.all()


@pytest.mark.parametrize("name,M", [("wan_ffn_down_sqnr", 1024), ("flux_qkv_w4a4", None)])
def test_fused_workload_bitwise_and_oracle(gpu, name, M):
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda", M=M)
    wc, wsc = gpu.quantize(w)
    announce(f"fused workload {name} {tuple(a.shape)}")
    out = gpu.gemm_w4a4_fused(a, wc, wsc, route=False)
    ref = _chain(gpu, a, wc, wsc, "ocp")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name}: fused differs from the chain"
    rng = np.random.default_rng(53)
    rows = np.unique(np.concatenate([rng.integers(0, a.shape[0], 24), [0, a.shape[0] - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, wl.N, 32), [0, wl.N - 1]]))
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    rac, ras = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(a.index_select(0, ri))))
    rwc, rws = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(w.index_select(0, ci))))
    r, tot = oracle.gemm_w4a4(rac, ras, rwc, rws, wl.K)
    ok, _, _ = oracle.within_tolerance(to_np_bf16_bits(out.index_select(0, ri).index_select(1, ci)), r, tot)
    assert ok.all()


@pytest.mark.parametrize("name", ["wan_ffn_down_sqnr", "flux_ffn_up_w4a4", "flux_ffn_down_w4a4"])
def test_fused_full_size_bitwise(gpu, name):
    a, w = workloads.workload_inputs(name, device="cuda")
    wc, wsc = gpu.quantize(w)
    announce(f"fused full size {name} {tuple(a.shape)}")
    out = gpu.gemm_w4a4_fused(a, wc, wsc, route=False)
    ref = _chain(gpu, a, wc, wsc, "ocp")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name}: full-size fused output differs from the chain"
    # past the break-even the call with a workspace quantizes in a pass of its own
    assert gpu.fused_workspace_bytes(*a.shape[:1], w.shape[0], a.shape[1]) > 0
    routed = gpu.gemm_w4a4_fused(a, wc, wsc)
    torch.cuda.synchronize()
    assert torch.equal(routed.view(torch.int16), ref.view(torch.int16)), f"{name}: routed call differs from the chain"


@pytest.mark.parametrize("M,N,K", [(300, 256, 3072), (300, 520, 3072), (200, 768, 8192), (200, 1030, 8192),
                                   (97, 900, 8224)])
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_routed_call_equals_fused_kernel(gpu, M, N, K, rule):
    g = torch.Generator(device="cuda").manual_seed(M + N + K)
    a = (torch.randn(M, K, device="cuda", generator=g) * torch.exp(torch.randn(1, K, device="cuda", generator=g)))
    a = a.to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    wc, wsc = gpu.quantize(w)
    routes = gpu.fused_workspace_bytes(M, N, K) > 0
    assert routes == ((N + 255) // 256 > (3 if K >= 8192 else 1))
    announce(f"routed vs fused {rule} M={M} N={N} K={K} routes={routes}")
    fused = gpu.gemm_w4a4_fused(a, wc, wsc, rule, route=False)
    routed = gpu.gemm_w4a4_fused(a, wc, wsc, rule)
    ref = _chain(gpu, a, wc, wsc, rule)
    torch.cuda.synchronize()
    _assert_same(routed, fused, f"routed {M}x{N}x{K} {rule}")
    _assert_same(routed, ref, f"chain {M}x{N}x{K} {rule}")
