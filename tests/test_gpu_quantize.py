"""GPU parity of the quantization kernels against the oracle: bit-exact bytes.

* MXFP4: an exhaustive anchor sweep (every finite bf16 pattern under every scale byte
  it can meet), random binary32 patterns under random scales, the tiny workload (fp32),
  the FLUX-shaped activations and weights in full, rows sampled from the Wan2.2-shaped
  activations at full size, ragged / strided layouts, and determinism.
* FP8 E4M3 (static): every bf16 pattern under several multipliers, workload shapes, binary32
  and strided inputs and outputs with a partial last pass.
* Dequantization: every code byte under every scale byte.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, bf16_from_bits, to_np_bf16_bits, to_np_u8

pytestmark = pytest.mark.gpu


def _check_mx(mxq, x_gpu, x_host_f32, label):
    announce(f"mxq_quantize {label} {tuple(x_gpu.shape)} {x_gpu.dtype}")
    codes, scales = mxq.quantize(x_gpu)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_mxfp4(x_host_f32)
    gc, gs = to_np_u8(codes), to_np_u8(scales)
    bad_s = np.nonzero(gs != rs)
    bad_c = np.nonzero(gc != rc)
    assert bad_s[0].size == 0, f"{label}: {bad_s[0].size} scale mismatches, first at {bad_s[0][0]},{bad_s[1][0]}"
    assert bad_c[0].size == 0, f"{label}: {bad_c[0].size} code mismatches, first at {bad_c[0][0]},{bad_c[1][0]}"
    return codes, scales


def _anchor_blocks_bf16(seed=0):
    """Blocks of 32 bf16 patterns: element 0 is an anchor of magnitude 2^(s-125), which
    fixes the scale byte at s; the other 31 are every finite pattern whose exponent field
    is <= s + 2 (so the scale cannot move), both signs."""
    rng = np.random.default_rng(seed)
    rows, expect = [], []
    for s in range(0, 253):
        top = min((s + 3) << 7, 0x7F80)
        mags = np.arange(0, top, dtype=np.uint32)
        pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        nb = -(-len(pats) // 31)
        pad = np.zeros(nb * 31 - len(pats), np.uint16)
        body = np.concatenate([pats, pad]).reshape(nb, 31)
        anchor = np.full((nb, 1), (s + 2) << 7, np.uint16) | (rng.integers(0, 2, (nb, 1)).astype(np.uint16) << 15)
        rows.append(np.concatenate([anchor, body], axis=1))
        expect.append(np.full(nb, s, np.uint8))
    blocks = np.concatenate(rows)
    exp_s = np.concatenate(expect)
    n = -(-len(blocks) // 32) * 32
    pad_blocks = np.zeros((n - len(blocks), 32), np.uint16)
    blocks = np.concatenate([blocks, pad_blocks])
    return blocks.reshape(-1, 32 * 32), exp_s


def test_mxfp4_exhaustive_bf16_anchor_sweep(gpu):
    bits, exp_s = _anchor_blocks_bf16()
    x = bf16_from_bits(bits)
    codes, scales = _check_mx(gpu, x, bf16_bits_to_f32(bits), "anchor-sweep")
    got = to_np_u8(scales).reshape(-1)[: len(exp_s)]
    np.testing.assert_array_equal(got, exp_s)       # construction check: the anchor fixed the scale


def test_mxfp4_random_binary32_patterns(gpu):
    rng = np.random.default_rng(1)
    nblk = 1 << 17
    s = rng.integers(0, 253, nblk)
    e = (rng.random((nblk, 31)) * (s[:, None] + 3)).astype(np.uint32)          # exponent field <= s + 2
    man = rng.integers(0, 1 << 23, (nblk, 31), dtype=np.uint32)
    sign = rng.integers(0, 2, (nblk, 31), dtype=np.uint32) << 31
    body = sign | (e << 23) | man
    anchor = ((s.astype(np.uint32) + 2) << 23)[:, None] | (rng.integers(0, 2, (nblk, 1), dtype=np.uint32) << 31)
    u = np.concatenate([anchor, body], axis=1)
    perm = rng.permuted(np.tile(np.arange(32), (nblk, 1)), axis=1)            # anchor at a random position
    u = np.take_along_axis(u, perm, axis=1).reshape(-1, 1024)
    x32 = u.view(np.float32)
    _check_mx(gpu, torch.from_numpy(x32).cuda(), x32, "random-fp32")


def test_mxfp4_tiny_workload_fp32(gpu):
    a, w = workloads.tiny_inputs(0)
    _check_mx(gpu, torch.from_numpy(a).cuda(), a, "tiny A")
    _check_mx(gpu, torch.from_numpy(w).cuda(), w, "tiny W")


@pytest.mark.parametrize("name", ["flux_qkv_w4a4"])
def test_mxfp4_flux_shapes_full(gpu, name):
    a, w = workloads.workload_inputs(name, device="cuda")
    _check_mx(gpu, a, bf16_bits_to_f32(to_np_bf16_bits(a)), f"{name} A")
    _check_mx(gpu, w, bf16_bits_to_f32(to_np_bf16_bits(w)), f"{name} W")


@pytest.mark.parametrize("name", ["wan_ffn_down_sqnr", "flux_ffn_down_w4a4"])
def test_mxfp4_full_size_sampled_rows(gpu, name):
    wl = workloads.WORKLOADS[name]
    a = workloads.activations(wl.M, wl.K, wl.act, seed=0, name=name, device="cuda")
    announce(f"mxq_quantize full {name} {tuple(a.shape)}")
    codes, scales = gpu.quantize(a)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(2).integers(0, wl.M, 48), [0, wl.M - 1]]))
    idx = torch.from_numpy(rows).cuda()
    xa = bf16_bits_to_f32(to_np_bf16_bits(a.index_select(0, idx)))
    rc, rs = oracle.quantize_mxfp4(xa)
    np.testing.assert_array_equal(to_np_u8(scales.index_select(0, idx)), rs)
    np.testing.assert_array_equal(to_np_u8(codes.index_select(0, idx)), rc)


@pytest.mark.parametrize("rows,cols,pad", [(1, 32, 0), (37, 96, 32), (5, 4096, 64), (129, 160, 8)])
def test_mxfp4_ragged_and_strided(gpu, rows, cols, pad):
    g = torch.Generator(device="cuda").manual_seed(rows * 1000 + cols)
    full = torch.randn(rows, cols + pad, device="cuda", generator=g).mul_(3.0).to(torch.bfloat16)
    x = full[:, :cols]
    ld_c, ld_s = cols // 2 + 16, cols // 32 + 3
    codes_buf = torch.full((rows, ld_c), 0xAB, dtype=torch.uint8, device="cuda")
    scales_buf = torch.full((rows, ld_s), 0xCD, dtype=torch.uint8, device="cuda")
    announce(f"mxq_quantize strided {rows}x{cols} ld_x={cols + pad}")
    gpu.quantize_into(x, codes_buf[:, : cols // 2], scales_buf[:, : cols // 32])
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(x)))
    cb, sb = to_np_u8(codes_buf), to_np_u8(scales_buf)
    np.testing.assert_array_equal(cb[:, : cols // 2], rc)
    np.testing.assert_array_equal(sb[:, : cols // 32], rs)
    assert np.all(cb[:, cols // 2:] == 0xAB) and np.all(sb[:, cols // 32:] == 0xCD)   # no writes past the rows


def test_mxfp4_zero_and_empty(gpu):
    x = torch.zeros(3, 64, dtype=torch.bfloat16, device="cuda")
    x[1] = -0.0
    c, s = gpu.quantize(x)
    torch.cuda.synchronize()
    assert to_np_u8(s).max() == 0
    np.testing.assert_array_equal(to_np_u8(c)[0], 0)
    np.testing.assert_array_equal(to_np_u8(c)[1], 0x88)
    c, s = gpu.quantize(torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"))
    assert c.shape == (0, 32) and s.shape == (0, 2)


def test_mxfp4_deterministic(gpu):
    a = workloads.activations(1000, 3072, "student_t", seed=4, name="det", device="cuda")
    c1, s1 = gpu.quantize(a)
    c2, s2 = gpu.quantize(a)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_nonfinite_blocks_get_the_nan_scale(gpu, dtype, rule):
    """Outside the contract (finite input), but defined: a block holding +-inf or NaN gets
    scale byte 0xFF; every other block is quantized as if the bad blocks were absent."""
    rng = np.random.default_rng(71)
    x = rng.standard_t(3, (8, 256)).astype(np.float32)
    bad = {(0, 0): [(0, 5, np.inf)], (1, 1): [(1, 40, -np.inf)], (2, 3): [(2, 100, np.nan)],
           (3, 6): [(3, 200, np.inf), (3, 201, np.nan)], (5, 7): [(5, 255, -np.inf), (5, 224, np.inf)]}
    for hits in bad.values():
        for r, c, v in hits:
            x[r, c] = v
    if dtype == "bf16":
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)     # truncation keeps inf / NaN
        xt, host = bf16_from_bits(bits), bf16_bits_to_f32(bits)
    else:
        xt, host = torch.from_numpy(x).cuda(), x.copy()
    announce(f"mxq_quantize non-finite blocks {dtype} {rule}")
    codes, scales = gpu.quantize(xt, rule)
    torch.cuda.synchronize()
    gs, gc = to_np_u8(scales), to_np_u8(codes)
    clean = host.copy()
    for (r, b) in bad:
        assert gs[r, b] == 0xFF, (r, b, hex(gs[r, b]))
        clean[r, 32 * b: 32 * b + 32] = 0.0
    rc, rs = oracle.quantize_mxfp4(clean, rule)
    good = np.ones_like(gs, dtype=bool)
    for (r, b) in bad:
        good[r, b] = False
    np.testing.assert_array_equal(gs[good], rs[good])
    gcb, rcb = gc.reshape(8, 8, 16), rc.reshape(8, 8, 16)
    np.testing.assert_array_equal(gcb[good], rcb[good])


# ---------------------------------------------------------------------------------- FP8

@pytest.mark.parametrize("inv_s", [1.0, 448.0 / 3.7, 1e-3, 2.0 ** 20, 0.75])
def test_fp8_every_bf16_pattern(gpu, inv_s):
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].copy()               # finite only
    bits = np.concatenate([bits, np.zeros((-len(bits)) % 256, np.uint16)]).reshape(-1, 256)
    x = bf16_from_bits(bits)
    announce(f"mxq_quantize_fp8 all-bf16 inv_s={inv_s}")
    q = gpu.quantize_fp8(x, inv_s)
    torch.cuda.synchronize()
    ref = oracle.quantize_fp8(bf16_bits_to_f32(bits), np.float32(inv_s))
    got = to_np_u8(q)
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, (bad[0].size, bits[bad][:4], got[bad][:4], ref[bad][:4])


def test_fp8_static_scale_workload_rows(gpu):
    name = "wan_ffn_up_w4a8"
    wl = workloads.WORKLOADS[name]
    a = workloads.activations(4096, wl.K, wl.act, seed=0, name=name, device="cuda")
    amax_gpu = gpu.absmax(a)
    torch.cuda.synchronize()
    host = bf16_bits_to_f32(to_np_bf16_bits(a))
    assert float(amax_gpu.item()) == float(np.max(np.abs(host)))
    s_a, inv_s = oracle.fp8_static_scales(np.max(np.abs(host)))
    assert gpu.fp8_static_scales(float(amax_gpu.item())) == (float(s_a), float(inv_s))
    q = gpu.quantize_fp8(a, float(inv_s))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np_u8(q), oracle.quantize_fp8(host, inv_s))
    assert (to_np_u8(q) & 0x7F).max() == 0x7E          # the tensor maximum maps onto 448


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pad_in,pad_out", [(0, 0), (48, 32)])
def test_fp8_input_types_strided_and_ragged(gpu, dtype, pad_in, pad_out):
    """Binary32 and bf16 input, packed or row-strided input and output, 37 x 784: 3626
    8-element units, so the kernel's last pass is partial and strided units cross rows."""
    rng = np.random.default_rng(61 + pad_in)
    rows, cols = 37, 784
    m = rng.standard_t(3, (rows, cols + pad_in)) * np.ldexp(1.0, rng.integers(-12, 12, (rows, 1)))
    full32 = m.astype(np.float32)
    if dtype == "bf16":
        bits = (full32.view(np.uint32) >> 16).astype(np.uint16)
        full = bf16_from_bits(bits)
        host = bf16_bits_to_f32(bits[:, :cols])
    else:
        full = torch.from_numpy(full32).cuda()
        host = full32[:, :cols]
    x = full[:, :cols]
    inv_s = float(oracle.fp8_static_scales(np.max(np.abs(host)))[1])
    qfull = torch.full((rows, cols + pad_out), 0xA5, dtype=torch.uint8, device="cuda")
    announce(f"mxq_quantize_fp8 {dtype} pad_in={pad_in} pad_out={pad_out} {rows}x{cols}")
    q = gpu.quantize_fp8(x, inv_s, out=qfull[:, :cols])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np_u8(q), oracle.quantize_fp8(np.ascontiguousarray(host), np.float32(inv_s)))
    if pad_out:
        assert (to_np_u8(qfull[:, cols:]) == 0xA5).all()      # nothing past the viewed columns


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_infinities_saturate(gpu, dtype):
    x = np.array([[np.inf, -np.inf, 1.0, -2.0] * 4], dtype=np.float32)
    xt = bf16_from_bits((x.view(np.uint32) >> 16).astype(np.uint16)) if dtype == "bf16" else torch.from_numpy(x).cuda()
    q = to_np_u8(gpu.quantize_fp8(xt, 3.0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q[0, 0::4], 0x7E)        # +448
    np.testing.assert_array_equal(q[0, 1::4], 0xFE)        # -448
    np.testing.assert_array_equal(q[0, 2::4], oracle.quantize_fp8(np.float32([[3.0]]), np.float32(1.0))[0, 0])
    np.testing.assert_array_equal(q[0, 3::4], oracle.quantize_fp8(np.float32([[-6.0]]), np.float32(1.0))[0, 0])


def test_absmax_fp32_and_strided(gpu):
    g = torch.Generator(device="cuda").manual_seed(9)
    full = torch.randn(300, 136, device="cuda", generator=g)
    full[17, 130] = 1e6          # outside the viewed columns: must be ignored
    x = full[:, :128]
    m = gpu.absmax(x)
    torch.cuda.synchronize()
    assert float(m.item()) == float(np.max(np.abs(x.cpu().numpy())))


# ---------------------------------------------------------------------------- dequantize

def test_dequantize_every_code_and_scale(gpu):
    """Every code byte under every scale byte (one scale per row), bit for bit: products
    past the largest bf16 round to +-inf, and scale byte 0xFF (the E8M0 NaN) gives NaN."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # [256, 256] -> K = 512
    scales = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, 16))  # one scale byte per row
    cg, sg = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    announce("mxq_dequantize exhaustive")
    y = gpu.dequantize(cg, sg, 512)
    torch.cuda.synchronize()
    ref = oracle.dequantize_mxfp4(codes, scales, 512)
    nan = np.isnan(ref)
    assert nan.sum() == 512 and nan[255].all()                           # exactly the 0xFF row
    ref_bits = oracle.f64_to_bf16_bits(np.where(nan, 0.0, ref))
    got = to_np_bf16_bits(y)
    np.testing.assert_array_equal(got[~nan], ref_bits[~nan])
    assert (np.abs(ref[~nan]) >= 2.0 ** 128).any()                        # the overflow cases are in
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_dequantize_workload_rows_and_strided_output(gpu):
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a = workloads.activations(2048, wl.K, wl.act, seed=0, name=name, device="cpu")
    rc, rs = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(a)))     # the oracle's codes
    codes, scales = torch.from_numpy(rc).cuda(), torch.from_numpy(rs).cuda()
    announce("mxq_dequantize workload rows, strided output")
    y = gpu.dequantize(codes, scales, wl.K)
    full = torch.full((2048, wl.K + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    gpu.dequantize(codes, scales, wl.K, out=full[:, :wl.K])
    torch.cuda.synchronize()
    ref_bits = oracle.f64_to_bf16_bits(oracle.dequantize_mxfp4(rc, rs, wl.K))
    np.testing.assert_array_equal(to_np_bf16_bits(y), ref_bits)
    np.testing.assert_array_equal(to_np_bf16_bits(full[:, :wl.K]), ref_bits)
    assert bool((full[:, wl.K:] == 3.0).all())
