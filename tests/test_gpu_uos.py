"""GPU parity of the UOS scale rule (mxq_quantize_rule) against the oracle: bit-exact bytes.

* every finite bf16 pattern as a block maximum (the rule depends only on amax), with a
  random body below it;
* random binary32 blocks with maxima around the 1.8125 significand boundary (fp32 input);
* rows of the Wan2.2-shaped activations at full size;
* the W4A4 chain on the tiny workload and the Wan2.2 FFN-down shape at reduced M: SQNR
  against the bf16 reference with UOS-quantized operands, GPU chain vs oracle chain
  within 0.01 dB, printed beside the OCP chain (the comparison of the two rules is a
  measurement, not a pinned value).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, bf16_from_bits, to_np_bf16_bits, to_np_u8

pytestmark = pytest.mark.gpu


def _check(mxq, x_gpu, x_host_f32, label, rule="uos"):
    announce(f"mxq_quantize_rule {rule} {label} {tuple(x_gpu.shape)} {x_gpu.dtype}")
    codes, scales = mxq.quantize(x_gpu, rule=rule)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_mxfp4(x_host_f32, rule)
    gs, gc = to_np_u8(scales), to_np_u8(codes)
    bad = np.nonzero(gs != rs)
    assert bad[0].size == 0, f"{label}: {bad[0].size} scale mismatches, first at {bad[0][0]},{bad[1][0]}"
    bad = np.nonzero(gc != rc)
    assert bad[0].size == 0, f"{label}: {bad[0].size} code mismatches, first at {bad[0][0]},{bad[1][0]}"
    return codes, scales


def test_uos_every_bf16_pattern_as_block_maximum(gpu):
    rng = np.random.default_rng(21)
    pats = np.arange(0, 0x7F80, dtype=np.uint32)               # every finite non-negative bf16
    n = pats.size
    anchor = (pats | (rng.integers(0, 2, n, dtype=np.uint32) << 15)).astype(np.uint16)
    # body: magnitudes at most the anchor's (random patterns below it), random signs
    body_mag = (rng.random((n, 31)) * (pats[:, None].astype(np.float64) + 1)).astype(np.uint32)
    body = (body_mag | (rng.integers(0, 2, (n, 31), dtype=np.uint32) << 15)).astype(np.uint16)
    blocks = np.concatenate([anchor[:, None], body], axis=1)
    pad = (-n) % 32
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.uint16)])
    bits = blocks.reshape(-1, 32 * 32)
    _check(gpu, bf16_from_bits(bits), bf16_bits_to_f32(bits), "bf16 maxima")


def test_uos_random_binary32_around_the_boundary(gpu):
    rng = np.random.default_rng(22)
    nblk = 1 << 16
    e = rng.integers(1, 254, nblk).astype(np.uint32)
    # fraction fields clustered at 0x680000 (significand 1.8125) and spread over the rest
    frac = np.where(rng.random(nblk) < 0.5, 0x680000 + rng.integers(-3, 4, nblk),
                    rng.integers(0, 1 << 23, nblk)).astype(np.uint32) & 0x7FFFFF
    amax_bits = (e << 23) | frac
    body = rng.random((nblk, 31)) * amax_bits.view(np.float32)[:, None]
    sign = rng.integers(0, 2, (nblk, 32)).astype(bool)
    x = np.concatenate([amax_bits.view(np.float32)[:, None], body.astype(np.float32)], axis=1)
    x = np.where(sign, -x, x).astype(np.float32)
    x = np.take_along_axis(x, rng.permuted(np.tile(np.arange(32), (nblk, 1)), axis=1), axis=1)
    x = x.reshape(-1, 1024)
    _check(gpu, torch.from_numpy(x).cuda(), x, "fp32 boundary")


def test_uos_workload_rows(gpu):
    name = "wan_ffn_down_sqnr"
    wl = workloads.WORKLOADS[name]
    a = workloads.activations(wl.M, wl.K, wl.act, seed=0, name=name, device="cuda")
    announce(f"mxq_quantize_rule uos full {name}")
    codes, scales = gpu.quantize(a, rule="uos")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(23).integers(0, wl.M, 32), [0, wl.M - 1]]))
    idx = torch.from_numpy(rows).cuda()
    rc, rs = oracle.quantize_mxfp4(bf16_bits_to_f32(to_np_bf16_bits(a.index_select(0, idx))), "uos")
    np.testing.assert_array_equal(to_np_u8(scales.index_select(0, idx)), rs)
    np.testing.assert_array_equal(to_np_u8(codes.index_select(0, idx)), rc)


def test_uos_bad_rule_is_rejected(gpu):
    x = torch.zeros(1, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gpu.quantize(x, rule="nvfp4")
    c = torch.empty(1, 16, dtype=torch.uint8, device="cuda")
    s = torch.empty(1, 1, dtype=torch.uint8, device="cuda")
    st = gpu.lib.mxq_quantize_rule(gpu._p(x), 1, 1, 32, 32, gpu._p(c), 16, gpu._p(s), 1, 7, gpu._stream())
    assert st == 2       # MXQ_ERR_UNSUPPORTED


def _chain_db(gpu, a, w, rule):
    ac, asc = gpu.quantize(a, rule=rule)
    wc, wsc = gpu.quantize(w, rule=rule)
    ref = gpu.gemm_bf16(a, w)
    out = gpu.gemm_w4a4(ac, asc, wc, wsc)
    return float(gpu.sqnr(ref, out)[2].item())


def _oracle_chain_db(a_bits, w_bits, K, rule):
    ha, hw = bf16_bits_to_f32(a_bits), bf16_bits_to_f32(w_bits)
    rac, ras = oracle.quantize_mxfp4(ha, rule)
    rwc, rws = oracle.quantize_mxfp4(hw, rule)
    r_ref = oracle.gemm.to_bf16(oracle.gemm_bf16(a_bits, w_bits)[0])
    r44 = oracle.gemm.to_bf16(oracle.gemm_w4a4(rac, ras, rwc, rws, K)[0])
    return oracle.sqnr_db(r_ref, r44)[2]


@pytest.mark.parametrize("name,M", [("tiny_w4a4", None), ("wan_ffn_down_sqnr", 1024)])
def test_uos_chain_sqnr_against_oracle(gpu, name, M):
    if name == "tiny_w4a4":
        a32, w32 = workloads.tiny_inputs(0)
        a = torch.from_numpy(a32).cuda().to(torch.bfloat16)
        w = torch.from_numpy(w32).cuda().to(torch.bfloat16)
    else:
        a, w = workloads.workload_inputs(name, device="cuda", M=M)
    K = a.shape[1]
    announce(f"uos chain sqnr {name} {tuple(a.shape)} x {tuple(w.shape)}")
    d_uos = _chain_db(gpu, a, w, "uos")
    d_ocp = _chain_db(gpu, a, w, "ocp")
    torch.cuda.synchronize()
    ab, wb = to_np_bf16_bits(a), to_np_bf16_bits(w)
    o_uos = _oracle_chain_db(ab, wb, K, "uos")
    o_ocp = _oracle_chain_db(ab, wb, K, "ocp")
    print(f"{name}: W4A4 SQNR  UOS gpu {d_uos:.4f} oracle {o_uos:.4f} | OCP gpu {d_ocp:.4f} oracle {o_ocp:.4f}",
          flush=True)
    assert abs(d_uos - o_uos) < 0.01 and abs(d_ocp - o_ocp) < 0.01
