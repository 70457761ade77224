"""GPU parity of the fused block-Hadamard rotation + MXFP4 quantizer (mxq_quantize_hadamard)
against the oracle: bit-exact codes and scales.

* bf16 inputs: heavy-tailed values and values spread over the whole exponent range
  (subnormal binary32 intermediates included), every block size and both scale rules;
* binary32 inputs over a wide exponent range;
* row-strided input and ragged row counts, partial 64-block spans for both input types;
* rows of the Wan2.2-shaped activations at full size;
* the W4A4 chain with both operands rotated, on the Wan2.2 FFN-down shape at reduced M:
  SQNR against the unrotated bf16 reference, GPU chain vs oracle chain within 0.01 dB,
  printed beside the unrotated chain (the gain is measured, not pinned).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, bf16_from_bits, to_np_bf16_bits, to_np_u8

pytestmark = pytest.mark.gpu
SIZES = (16, 64, 256)


def _check(mxq, x_gpu, x_host_f32, n, rule, label):
    announce(f"mxq_quantize_hadamard n={n} {rule} {label} {tuple(x_gpu.shape)} {x_gpu.dtype}")
    codes, scales = mxq.quantize_hadamard(x_gpu, n, rule)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_mxfp4_rotated(x_host_f32, n, rule)
    gs, gc = to_np_u8(scales), to_np_u8(codes)
    bad = np.nonzero(gs != rs)
    assert bad[0].size == 0, f"{label}: {bad[0].size} scale mismatches, first at {bad[0][0]},{bad[1][0]}"
    bad = np.nonzero(gc != rc)
    assert bad[0].size == 0, f"{label}: {bad[0].size} code mismatches, first at {bad[0][0]},{bad[1][0]}"


def _bf16_bits(rng, shape):
    """bf16 patterns: half heavy-tailed values, half uniform over bit patterns up to 2^118
    (sums of 256 of them stay finite: overflow is outside the contract)."""
    t = rng.standard_t(3, shape).astype(np.float32)
    tb = (t.view(np.uint32) >> 16).astype(np.uint16)
    ub = rng.integers(0, 0x7A80, shape).astype(np.uint16) | (rng.integers(0, 2, shape).astype(np.uint16) << 15)
    rows = rng.random(shape[0]) < 0.5
    return np.where(rows[:, None], tb, ub)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_hadamard_bf16_random(gpu, n, rule):
    rng = np.random.default_rng(31 + n)
    bits = _bf16_bits(rng, (256, 1024))
    _check(gpu, bf16_from_bits(bits), bf16_bits_to_f32(bits), n, rule, "bf16 random")


@pytest.mark.parametrize("n", SIZES)
def test_hadamard_fp32_wide_range(gpu, n):
    rng = np.random.default_rng(41 + n)
    m = rng.uniform(1, 2, (128, 2048)) * rng.choice([-1, 1], (128, 2048))
    e = rng.integers(-140, 120, (128, 1))            # one exponent range per row
    x = np.ldexp(m, e + rng.integers(-6, 7, (128, 2048))).astype(np.float32)
    _check(gpu, torch.from_numpy(x).cuda(), x, n, "ocp", "fp32 wide")


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_hadamard_tiny_block_boundary(gpu, n, rule):
    """Blocks whose rotated, normalised maximum lies around 2^-121, with full 24-bit
    significands reaching down into the subnormal range: the binary32 product by
    1/sqrt(n) then rounds on the subnormal grid, next to FP4 rounding boundaries of the
    smallest scales (2^-127 .. 2^-119), and some blocks are all zero."""
    rng = np.random.default_rng(53 + n)
    rows, cols = 96, 2048
    L = {16: 2, 64: 3, 256: 4}[n]
    m = rng.uniform(1, 2, (rows, cols)) * rng.choice([-1, 1], (rows, cols))
    top = -121 + L + rng.integers(-8, 9, (rows, 1))   # maximum exponent of each row
    x = np.ldexp(m, top - rng.integers(0, 30, (rows, cols))).astype(np.float32)
    x[::7, ::5] = 0.0                                  # some zeros, a few all-zero blocks
    x[5, :256] = 0.0
    _check(gpu, torch.from_numpy(x).cuda(), x, n, rule, "fp32 near 2^-121")


@pytest.mark.parametrize("rows,cols,pad,n", [(1, 256, 0, 256), (37, 512, 64, 64), (129, 768, 16, 16)])
def test_hadamard_strided_and_ragged(gpu, rows, cols, pad, n):
    g = torch.Generator(device="cuda").manual_seed(rows + cols)
    full = torch.randn(rows, cols + pad, device="cuda", generator=g).mul_(5.0).to(torch.bfloat16)
    x = full[:, :cols]
    _check(gpu, x, bf16_bits_to_f32(to_np_bf16_bits(x)), n, "ocp", "strided")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("pad", [0, 32])
def test_hadamard_partial_spans(gpu, dtype, n, pad):
    """45 x 768: 1080 blocks, so the last 64-block span of a wave is partial (56 blocks);
    packed rows and row-strided rows (spans cross row ends), both input types, both rules."""
    rng = np.random.default_rng(51 + n + pad)
    rows, cols = 45, 768
    m = rng.standard_t(3, (rows, cols + pad)) * np.ldexp(1.0, rng.integers(-20, 20, (rows, 1)))
    full32 = m.astype(np.float32)
    if dtype == "bf16":
        bits = (full32.view(np.uint32) >> 16).astype(np.uint16)
        full = bf16_from_bits(bits)
        host = bf16_bits_to_f32(bits[:, :cols])
    else:
        full = torch.from_numpy(full32).cuda()
        host = full32[:, :cols]
    x = full[:, :cols]
    for rule in ("ocp", "uos"):
        _check(gpu, x, np.ascontiguousarray(host), n, rule, f"partial spans {dtype} pad={pad}")


@pytest.mark.parametrize("n", SIZES)
def test_hadamard_nonfinite_runs_get_the_nan_scale(gpu, n):
    """Outside the contract, but defined: an infinity or NaN reaches every element of its
    run of n, so every block of that run gets scale byte 0xFF; other runs are unaffected."""
    rng = np.random.default_rng(81 + n)
    x = rng.standard_t(3, (4, 512)).astype(np.float32)
    x[0, 5] = np.nan
    x[1, 300] = np.inf
    x[3, 511] = -np.inf
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    host = bf16_bits_to_f32(bits)
    announce(f"mxq_quantize_hadamard non-finite n={n}")
    codes, scales = gpu.quantize_hadamard(bf16_from_bits(bits), n)
    torch.cuda.synchronize()
    gs, gc = to_np_u8(scales), to_np_u8(codes)
    bad = np.zeros_like(gs, dtype=bool)
    clean = host.copy()
    for r, c in ((0, 5), (1, 300), (3, 511)):
        run = (c // n) * n
        bad[r, run // 32: (run + n + 31) // 32] = True
        clean[r, run: run + n] = 0.0
    assert (gs[bad] == 0xFF).all()
    rc, rs = oracle.quantize_mxfp4_rotated(clean, n)
    np.testing.assert_array_equal(gs[~bad], rs[~bad])
    np.testing.assert_array_equal(gc.reshape(4, 16, 16)[~bad], rc.reshape(4, 16, 16)[~bad])


def test_hadamard_workload_rows(gpu):
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a = workloads.activations(wl.M, wl.K, wl.act, seed=0, name=name, device="cuda")
    for n in SIZES:
        announce(f"mxq_quantize_hadamard full {name} n={n}")
        codes, scales = gpu.quantize_hadamard(a, n)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.random.default_rng(32 + n).integers(0, wl.M, 16), [0, wl.M - 1]]))
        idx = torch.from_numpy(rows).cuda()
        rc, rs = oracle.quantize_mxfp4_rotated(bf16_bits_to_f32(to_np_bf16_bits(a.index_select(0, idx))), n)
        np.testing.assert_array_equal(to_np_u8(scales.index_select(0, idx)), rs)
        np.testing.assert_array_equal(to_np_u8(codes.index_select(0, idx)), rc)


def test_hadamard_rejects_bad_block(gpu):
    x = torch.zeros(2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.MxqError):
        gpu.quantize_hadamard(x, 32)
    with pytest.raises(gpu.MxqError):
        gpu.quantize_hadamard(torch.zeros(2, 96, dtype=torch.bfloat16, device="cuda"), 64)


@pytest.mark.parametrize("n", [64, 256])
def test_hadamard_chain_sqnr_against_oracle(gpu, n):
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a, w = workloads.workload_inputs(name, device="cuda", M=512)
    announce(f"hadamard chain sqnr n={n} {tuple(a.shape)}")
    ref = gpu.gemm_bf16(a, w)
    ac, asc = gpu.quantize_hadamard(a, n)
    wc, wsc = gpu.quantize_hadamard(w, n)
    d_rot = float(gpu.sqnr(ref, gpu.gemm_w4a4(ac, asc, wc, wsc))[2].item())
    pc, psc = gpu.quantize(a)
    qc, qsc = gpu.quantize(w)
    d_plain = float(gpu.sqnr(ref, gpu.gemm_w4a4(pc, psc, qc, qsc))[2].item())
    torch.cuda.synchronize()
    ab, wb = to_np_bf16_bits(a), to_np_bf16_bits(w)
    ha, hw = bf16_bits_to_f32(ab), bf16_bits_to_f32(wb)
    rac, ras = oracle.quantize_mxfp4_rotated(ha, n)
    rwc, rws = oracle.quantize_mxfp4_rotated(hw, n)
    r_ref = oracle.gemm.to_bf16(oracle.gemm_bf16(ab, wb)[0])
    r_rot = oracle.gemm.to_bf16(oracle.gemm_w4a4(rac, ras, rwc, rws, wl.K)[0])
    o_rot = oracle.sqnr_db(r_ref, r_rot)[2]
    print(f"n={n}: W4A4 SQNR rotated gpu {d_rot:.4f} oracle {o_rot:.4f} | unrotated gpu {d_plain:.4f}", flush=True)
    assert abs(d_rot - o_rot) < 0.01
