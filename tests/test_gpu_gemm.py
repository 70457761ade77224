"""GPU parity of the W4A4 / W4A8 / bf16 GEMMs against the float64 oracle.

Bar, per element: |gpu - oracle| <= 1e-5 * sum_k |a_k w_k| + 1 bf16 ulp(oracle), with the
oracle computed from its own quantization of the same seeded inputs.  Cases: the tiny
workload, shapes spanning several 256 x 256 tiles with ragged M / N / K tails (including
scale rows that are not 4-byte multiples), random codes over the full E2M1 range,
outputs sampled at the full workload sizes in the launch configuration the benchmark
times, exact metamorphic properties (power-of-two scaling, zero input) and determinism.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, to_np_bf16_bits, to_np_u8, u8_to_gpu

pytestmark = pytest.mark.gpu


def _assert_tol(got_bits, out, tot, label):
    ok, err, bound = oracle.within_tolerance(got_bits, out, tot)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{label}: {int((~ok).sum())}/{ok.size} outside tolerance; first at {tuple(i)}: "
                             f"err {err[tuple(i)]:.3e} bound {bound[tuple(i)]:.3e} oracle {out[tuple(i)]:.6e}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def _host_absmax(t, chunk=4096):
    """max |x| of a GPU bf16 tensor, reduced on the host chunk by chunk."""
    m = 0.0
    for r0 in range(0, t.shape[0], chunk):
        m = max(m, float(np.max(np.abs(bf16_bits_to_f32(to_np_bf16_bits(t[r0:r0 + chunk]))))))
    return m


def _host_f32(t):
    return bf16_bits_to_f32(to_np_bf16_bits(t)) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _w4a4_case(mxq, a, w, label):
    """a: [M,K], w: [N,K] GPU tensors (bf16 or fp32).  GPU quantize + GEMM vs oracle."""
    announce(f"w4a4 {label} M={a.shape[0]} N={w.shape[0]} K={a.shape[1]}")
    ac, asc = mxq.quantize(a)
    wc, wsc = mxq.quantize(w)
    out = mxq.gemm_w4a4(ac, asc, wc, wsc)
    torch.cuda.synchronize()
    K = a.shape[1]
    rac, ras = oracle.quantize_mxfp4(_host_f32(a))
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w))
    ref, tot = oracle.gemm_w4a4(rac, ras, rwc, rws, K)
    return _assert_tol(to_np_bf16_bits(out), ref, tot, label)


def test_w4a4_tiny_workload(gpu):
    a, w = workloads.tiny_inputs(0)
    _w4a4_case(gpu, torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda(), "tiny")


@pytest.mark.parametrize("M,N,K", [(300, 520, 416), (513, 257, 1024), (64, 96, 96), (256, 256, 256),
                                   (700, 384, 288), (1, 1, 32), (260, 300, 3072), (300, 520, 8704)])
def test_w4a4_tiles_and_ragged_tails(gpu, M, N, K):
    """K = 8704 takes the fast path with ordinary output stores (K above 8192); the other
    whole-window shapes take it with non-temporal ones."""
    a = workloads.activations(M, K, "lognormal_channels", seed=M, name="ragged", device="cuda")
    w = workloads.weights(N, K, 0.02, seed=N, name="ragged", device="cuda")
    _w4a4_case(gpu, a, w, f"ragged{M}x{N}x{K}")


def test_w4a4_random_codes_full_e2m1_range(gpu):
    rng = np.random.default_rng(21)
    M, N, K = 320, 288, 512
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wsc = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    announce("w4a4 random codes")
    out = gpu.gemm_w4a4(u8_to_gpu(ac), u8_to_gpu(asc), u8_to_gpu(wc), u8_to_gpu(wsc))
    torch.cuda.synchronize()
    ref, tot = oracle.gemm_w4a4(ac, asc, wc, wsc, K)
    _assert_tol(to_np_bf16_bits(out), ref, tot, "random-codes")


def test_w4a4_power_of_two_scaling_and_zero_are_exact(gpu):
    rng = np.random.default_rng(22)
    M, N, K = 300, 260, 768
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = rng.integers(115, 135, (M, K // 32), dtype=np.uint8)
    wsc = rng.integers(115, 135, (N, K // 32), dtype=np.uint8)
    g = [u8_to_gpu(x) for x in (ac, asc, wc, wsc)]
    announce("w4a4 metamorphic")
    o1 = gpu.gemm_w4a4(*g)
    o2 = gpu.gemm_w4a4(g[0], u8_to_gpu(asc + 5), g[2], g[3])
    o3 = gpu.gemm_w4a4(torch.zeros_like(g[0]), g[1], g[2], g[3])
    o4 = gpu.gemm_w4a4(u8_to_gpu(ac ^ 0x88), g[1], g[2], g[3])   # negate A
    torch.cuda.synchronize()
    # a power-of-two scale commutes with every rounding step: exact
    assert torch.equal(o2.float(), o1.float() * 32)
    assert torch.count_nonzero(o3.float()) == 0
    # negation is not bit-exact (the MFMA's internal accumulation is not sign-symmetric):
    # the negated product is checked against the oracle like any other
    ref, tot = oracle.gemm_w4a4(ac ^ 0x88, asc, wc, wsc, K)
    _assert_tol(to_np_bf16_bits(o4), ref, tot, "negated-A")


def test_w4a4_deterministic(gpu):
    a = workloads.activations(600, 1536, "student_t", seed=3, name="det", device="cuda")
    w = workloads.weights(520, 1536, 0.015, seed=3, name="det", device="cuda")
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    o1 = gpu.gemm_w4a4(ac, asc, wc, wsc)
    o2 = gpu.gemm_w4a4(ac, asc, wc, wsc)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_w4a4_k_zero_writes_zeros(gpu):
    out = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    e = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    f = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    gpu.gemm_w4a4(e, e, f, f, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0


def _sample_rows_cols(M, N, seed, nr=40, nc=48):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.integers(0, M, nr), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, N, nc), [0, N - 1]]))
    return rows, cols


@pytest.mark.parametrize("name", ["wan_ffn_down_sqnr", "flux_ffn_up_w4a4", "flux_ffn_down_w4a4", "flux_qkv_w4a4"])
def test_w4a4_full_size_sampled(gpu, name):
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda")
    announce(f"w4a4 full {name}")
    ac, asc = gpu.quantize(a)
    wc, wsc = gpu.quantize(w)
    out = gpu.gemm_w4a4(ac, asc, wc, wsc)
    torch.cuda.synchronize()
    rows, cols = _sample_rows_cols(wl.M, wl.N, 5)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    rac, ras = oracle.quantize_mxfp4(_host_f32(a.index_select(0, ri)))
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w.index_select(0, ci)))
    ref, tot = oracle.gemm_w4a4(rac, ras, rwc, rws, wl.K)
    got = to_np_bf16_bits(out.index_select(0, ri).index_select(1, ci))
    _assert_tol(got, ref, tot, name)


# ---------------------------------------------------------------------------- W4A8

def _w4a8_case(mxq, a, w, label):
    announce(f"w4a8 {label} M={a.shape[0]} N={w.shape[0]} K={a.shape[1]}")
    amax = float(mxq.absmax(a).item())
    s_a, inv_s = mxq.fp8_static_scales(amax)
    q = mxq.quantize_fp8(a, inv_s)
    wc, wsc = mxq.quantize(w)
    out = mxq.gemm_w4a8(q, s_a, wc, wsc)
    torch.cuda.synchronize()
    host = _host_f32(a)
    rs_a, rinv = oracle.fp8_static_scales(np.max(np.abs(host)))
    rq = oracle.quantize_fp8(host, rinv)
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w))
    ref, tot = oracle.gemm_w4a8(rq, rs_a, rwc, rws, a.shape[1])
    return _assert_tol(to_np_bf16_bits(out), ref, tot, label)


_W4A8_TILES = [(300, 520, 1056), (513, 257, 1024), (260, 300, 5120), (700, 384, 5024), (256, 256, 3104),
               (1, 1, 1024), (64, 96, 2080), (300, 520, 8704)]


@pytest.mark.parametrize("dist", ["lognormal_channels", "student_t"])
@pytest.mark.parametrize("M,N,K", _W4A8_TILES)
def test_w4a8_tiles_and_ragged_tails(gpu, M, N, K, dist):
    """Tiles and ragged M / N / K tails (K off the 128-element window for 1056, 5024,
    3104, 2080) on the W4A8 workloads' own activation models -- N(0,1) times a
    LogNormal(0,1) per-channel scale (Wan2.2 FFN up, K = 5120) and Student-t(3) (FFN
    down, K = 13824) -- statically scaled from each tensor's amax, at the unchanged bar,
    for K >= 1024 (at these sizes no output meets the few-per-million excess recorded
    below)."""
    a = workloads.activations(M, K, dist, seed=M, name="w4a8", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=N, name="w4a8", device="cuda")
    _w4a8_case(gpu, a, w, f"ragged{M}x{N}x{K}-{dist}")


@pytest.mark.parametrize("M,N,K", [(300, 520, 416), (64, 96, 96), (1, 1, 32), (700, 384, 288), (256, 256, 256)])
def test_w4a8_short_k_student_t(gpu, M, N, K):
    """Short reductions (one to four 128-element windows) on the Student-t activation
    model, at the unchanged bar."""
    a = workloads.activations(M, K, "student_t", seed=M, name="w4a8", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=N, name="w4a8", device="cuda")
    _w4a8_case(gpu, a, w, f"short{M}x{N}x{K}")


def _enc8(v):
    return int(oracle.e4m3_encode(np.array([v], np.float64))[0])


def test_w4a8_fp8_mfma_group_alignment(gpu):
    """The hardware fact behind the W4A8 domain, pinned: the FP8 x FP4 scaled MFMA adds
    each group of 8 consecutive K products on a fixed-point grid whose last bit is
    2^(E - 13), E the exponent of the group's largest product; smaller products (or
    their low bits) are dropped.  With +448 and -448 in a group (E = 8) a lone 2^-5
    survives and a lone 2^-6 vanishes; with 62 copies of 2^-6, exactly the 6 that share
    the pair's group of 8 vanish; with +-16 (E = 4) even 2^-9 survives.  W4A4 products
    never span enough binades to reach this."""
    M, N, K = 32, 32, 64
    wc = u8_to_gpu(np.full((N, K // 2), 0x22, np.uint8))        # every weight 1.0
    ws = u8_to_gpu(np.full((N, K // 32), 127, np.uint8))
    cases = []

    def row(big, small_e, count, start=2):
        a = np.zeros((M, K), np.uint8)
        a[:, 0], a[:, 1] = _enc8(big), _enc8(-big)
        a[:, start:start + count] = _enc8(2.0 ** -small_e)
        return a

    cases = [(row(448.0, 5, 1), 2.0 ** -5), (row(448.0, 6, 1), 0.0), (row(448.0, 6, 62), 56 * 2.0 ** -6),
             (row(16.0, 9, 1), 2.0 ** -9), (row(64.0, 7, 62), 62 * 2.0 ** -7), (row(64.0, 8, 62), 56 * 2.0 ** -8)]
    announce("w4a8 MFMA group alignment")
    for a8, expect in cases:
        out = gpu.gemm_w4a8(u8_to_gpu(a8), 1.0, wc, ws)
        torch.cuda.synchronize()
        got = oracle.bf16_bits_to_f64(to_np_bf16_bits(out))
        assert np.all(got == expect), (got[0, 0], expect)


def test_w4a8_rare_excess_over_a_large_output(gpu):
    """The same hardware effect over 17.2M outputs (4252 x 4036, lognormal-channel
    activations, K = 1024): a few outputs per million with heavy cancellation exceed the
    bar.  Recorded, not hidden: at most 1 in 10^5 outputs outside, none beyond 3x
    (measured with these seeds: 26 outside, at most 1.68x; with another seed stream 84,
    at most 2.85x)."""
    M, N, K = 4252, 4036, 1024
    a = workloads.activations(M, K, "lognormal_channels", seed=M + N, name="large", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=N, name="large", device="cuda")
    announce(f"w4a8 large output lognormal {M}x{N}x{K}")
    s_a, inv_s = gpu.fp8_static_scales(float(gpu.absmax(a).item()))
    out = gpu.gemm_w4a8(gpu.quantize_fp8(a, inv_s), s_a, *gpu.quantize(w))
    torch.cuda.synchronize()
    host = _host_f32(a)
    rs_a, rinv = oracle.fp8_static_scales(np.max(np.abs(host)))
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w))
    ref, tot = oracle.gemm_w4a8(oracle.quantize_fp8(host, rinv), rs_a, rwc, rws, K)
    ok, err, bound = oracle.within_tolerance(to_np_bf16_bits(out), ref, tot)
    outside, worst = int((~ok).sum()), float(np.max(err / bound))
    print(f"W4A8 {M}x{N}x{K} lognormal: {outside}/{ok.size} outside the bar, worst {worst:.3f}x", flush=True)
    assert outside <= ok.size * 1e-5 and worst < 3.0


def test_w4a8_short_k_lognormal_outside_the_domain(gpu):
    """At short K -- reductions of a few hundred elements on the
    lognormal-channel model, where per-channel scales put E4M3 subnormals next to values
    near 448 inside one group of 8 -- the dropped products can exceed the bar on rare
    outputs with heavy cancellation.  Recorded, not hidden: at most 1 in 10^4 outputs
    outside the bar, none beyond 1.5x it (measured: 5 of ~425k, at most 1.31x)."""
    worst, outside, total = 0.0, 0, 0
    for M, N, K in [(300, 520, 416), (700, 384, 288), (64, 96, 96), (256, 256, 256)]:
        a = workloads.activations(M, K, "lognormal_channels", seed=M, name="w4a8", device="cuda")
        w = workloads.weights(N, K, 0.015, seed=N, name="w4a8", device="cuda")
        announce(f"w4a8 short-K lognormal {M}x{N}x{K}")
        amax = float(gpu.absmax(a).item())
        s_a, inv_s = gpu.fp8_static_scales(amax)
        out = gpu.gemm_w4a8(gpu.quantize_fp8(a, inv_s), s_a, *gpu.quantize(w))
        torch.cuda.synchronize()
        host = _host_f32(a)
        rs_a, rinv = oracle.fp8_static_scales(np.max(np.abs(host)))
        rwc, rws = oracle.quantize_mxfp4(_host_f32(w))
        ref, tot = oracle.gemm_w4a8(oracle.quantize_fp8(host, rinv), rs_a, rwc, rws, K)
        ok, err, bound = oracle.within_tolerance(to_np_bf16_bits(out), ref, tot)
        worst = max(worst, float(np.max(err / bound)))
        outside += int((~ok).sum())
        total += ok.size
    print(f"W4A8 short-K lognormal: {outside}/{total} outside the bar, worst {worst:.3f}x", flush=True)
    assert outside <= total * 1e-4 and worst < 1.5


def test_w4a8_random_codes(gpu):
    """Random E4M3 codes over a 2^8 magnitude window (exponent fields 6..14, the spread of
    statically scaled activations) and random MXFP4 weights with random scales."""
    rng = np.random.default_rng(23)
    M, N, K = 320, 288, 512
    e = rng.integers(6, 15, (M, K))
    a8 = ((rng.integers(0, 2, (M, K)) << 7) | (e << 3) | rng.integers(0, 8, (M, K))).astype(np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    wsc = rng.integers(115, 140, (N, K // 32), dtype=np.uint8)
    s_a = np.float32(0.0123)
    announce("w4a8 random codes")
    out = gpu.gemm_w4a8(u8_to_gpu(a8), float(s_a), u8_to_gpu(wc), u8_to_gpu(wsc))
    torch.cuda.synchronize()
    ref, tot = oracle.gemm_w4a8(a8, s_a, wc, wsc, K)
    _assert_tol(to_np_bf16_bits(out), ref, tot, "w4a8-random")


def test_w4a8_accumulation_precision_characterization(gpu):
    """The FP8 x FP4 block-scaled MFMA does not sum its 64 products exactly: with E4M3
    codes spanning the whole format (2^-9 .. 448) inside one block its error reaches
    ~1e-4 * sum|a*b| for a single instruction (K = 64), shrinking as K grows.  This is
    recorded, not hidden: the error beyond bf16 rounding must stay under 2.5e-4 * sum|a*b|
    here, while the workload-size tests hold the 1e-5 bar."""
    rng = np.random.default_rng(24)
    worst = {}
    for K in (64, 512, 4096):
        M, N = 256, 256
        a8 = rng.integers(0, 256, (M, K), dtype=np.uint8)
        a8[(a8 & 0x7F) == 0x7F] = 0x40
        wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        wsc = rng.integers(115, 140, (N, K // 32), dtype=np.uint8)
        announce(f"w4a8 precision K={K}")
        out = gpu.gemm_w4a8(u8_to_gpu(a8), 1.0, u8_to_gpu(wc), u8_to_gpu(wsc))
        torch.cuda.synchronize()
        ref, tot = oracle.gemm_w4a8(a8, np.float32(1.0), wc, wsc, K)
        got = oracle.bf16_bits_to_f64(to_np_bf16_bits(out))
        excess = np.maximum(np.abs(got - ref) - 0.5 * oracle.bf16_ulp(ref), 0) / tot
        worst[K] = float(excess.max())
    print("W4A8 max error beyond bf16 rounding / sum|ab|:", worst, flush=True)
    assert max(worst.values()) < 2.5e-4


@pytest.mark.parametrize("name", ["wan_ffn_up_w4a8", "wan_ffn_down_sqnr"])
def test_w4a8_full_size_sampled(gpu, name):
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda")
    announce(f"w4a8 full {name}")
    amax = float(gpu.absmax(a).item())
    s_a, inv_s = gpu.fp8_static_scales(amax)
    q = gpu.quantize_fp8(a, inv_s)
    wc, wsc = gpu.quantize(w)
    out = gpu.gemm_w4a8(q, s_a, wc, wsc)
    torch.cuda.synchronize()
    rows, cols = _sample_rows_cols(wl.M, wl.N, 6, nr=96, nc=wl.N)   # ~100 full output rows
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    # the static scale is a whole-tensor statistic: the host takes the max over all of A
    amax_host = _host_absmax(a)
    assert amax == amax_host
    rs_a, rinv = oracle.fp8_static_scales(amax_host)
    assert (float(rs_a), float(rinv)) == (s_a, inv_s)
    rq = oracle.quantize_fp8(_host_f32(a.index_select(0, ri)), rinv)
    rwc, rws = oracle.quantize_mxfp4(_host_f32(w.index_select(0, ci)))
    ref, tot = oracle.gemm_w4a8(rq, rs_a, rwc, rws, wl.K)
    got = to_np_bf16_bits(out.index_select(0, ri).index_select(1, ci))
    _assert_tol(got, ref, tot, name)


# ---------------------------------------------------------------------------- bf16 reference

@pytest.mark.parametrize("M,N,K", [(300, 520, 416), (64, 96, 96), (513, 257, 2048)])
def test_bf16_reference_gemm(gpu, M, N, K):
    a = workloads.activations(M, K, "student_t", seed=M, name="bf16", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=N, name="bf16", device="cuda")
    announce(f"bf16 gemm {M}x{N}x{K}")
    out = gpu.gemm_bf16(a, w)
    torch.cuda.synchronize()
    ref, tot = oracle.gemm_bf16(to_np_bf16_bits(a), to_np_bf16_bits(w))
    _assert_tol(to_np_bf16_bits(out), ref, tot, f"bf16-{M}x{N}x{K}")


def test_bf16_reference_full_size_sampled(gpu):
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda")
    announce("bf16 gemm full")
    out = gpu.gemm_bf16(a, w)
    torch.cuda.synchronize()
    rows, cols = _sample_rows_cols(wl.M, wl.N, 7)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ref, tot = oracle.gemm_bf16(to_np_bf16_bits(a.index_select(0, ri)), to_np_bf16_bits(w.index_select(0, ci)))
    _assert_tol(to_np_bf16_bits(out.index_select(0, ri).index_select(1, ci)), ref, tot, "bf16-full")
