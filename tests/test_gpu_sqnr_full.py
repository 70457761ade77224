"""Whole-output SQNR parity at full size on the Wan2.2 FFN-down workload (75600 x 13824
activations, 5120 x 13824 weights): W4A4 and W4A8 against the bf16 reference, the GPU
chain (mxq_quantize / mxq_quantize_fp8 -> GEMMs -> mxq_sqnr) against the oracle chain
(its own quantization, float64 GEMMs, float64 SQNR) over every one of the 387M outputs,
to 0.01 dB ("AMD Quark adds native W4A8 mixed-precision for Wan2.2 ...", section "Quark
quantization pipeline and mixed-precision selection": blocks are scored by the SQNR of
their whole output against BF16).

The host work (about 32 TFLOP of float64 GEMMs) is split into row chunks, one test
each, so progress shows as the chunks finish.  Each chunk's SQNR is checked on its own
against the GPU's SQNR of the same rows; the last test sums the chunks' signal and noise
powers and checks the whole-output dB the benchmark reports.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, bf16_bits_to_f32, to_np_bf16_bits

pytestmark = pytest.mark.gpu

NAME = "wan_ffn_down_sqnr"
WL = workloads.WORKLOADS[NAME]
CHUNKS = 8
BOUNDS = [WL.M * i // CHUNKS for i in range(CHUNKS + 1)]
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
_partial = {}


def _db(s, n):
    if n == 0.0:
        return math.nan if s == 0.0 else math.inf
    return 10.0 * math.log10(s / n)


@pytest.fixture(scope="module")
def chain(gpu):
    a, w = workloads.workload_inputs(NAME, device="cuda")
    announce("full-size chain: quantize, GEMMs, SQNR")
    wc, wsc = gpu.quantize(w)
    amax = float(gpu.absmax(a).item())
    s_a, inv_s = gpu.fp8_static_scales(amax)
    ac, asc = gpu.quantize(a)
    a8 = gpu.quantize_fp8(a, inv_s)
    o44 = gpu.gemm_w4a4(ac, asc, wc, wsc)
    o48 = gpu.gemm_w4a8(a8, s_a, wc, wsc)
    ref = gpu.gemm_bf16(a, w)
    r44 = gpu.sqnr(ref, o44).cpu().tolist()
    r48 = gpu.sqnr(ref, o48).cpu().tolist()
    del ac, asc, a8
    # the oracle's own operands: weights quantized from the host copy, the static scale
    # from the host maximum over the whole tensor
    host_amax = 0.0
    for r0 in range(0, WL.M, 8192):
        host_amax = max(host_amax, float(np.max(np.abs(bf16_bits_to_f32(to_np_bf16_bits(a[r0:r0 + 8192]))))))
    assert host_amax == amax
    rs_a, rinv = oracle.fp8_static_scales(host_amax)
    assert (float(rs_a), float(rinv)) == (s_a, inv_s)
    w_bits = to_np_bf16_bits(w)
    rwc, rws = oracle.quantize_mxfp4(bf16_bits_to_f32(w_bits))
    torch.cuda.synchronize()
    return {"a": a, "ref": ref, "o44": o44, "o48": o48, "r44": r44, "r48": r48, "w_bits": w_bits,
            "rwc": rwc, "rws": rws, "rs_a": rs_a, "rinv": rinv}


def _oracle_chunk(c, r0, r1):
    """Oracle (S, N) of W4A4 and W4A8 over rows r0..r1: quantization in parallel row
    slices, then the float64 GEMMs and float64 sums."""
    a_bits = to_np_bf16_bits(c["a"][r0:r1])
    a_f32 = bf16_bits_to_f32(a_bits)
    edges = np.linspace(0, r1 - r0, THREADS + 1).astype(int)
    parts = [(edges[i], edges[i + 1]) for i in range(THREADS) if edges[i + 1] > edges[i]]
    with ThreadPoolExecutor(len(parts)) as ex:
        q4 = list(ex.map(lambda p: oracle.quantize_mxfp4(a_f32[p[0]:p[1]]), parts))
        q8 = list(ex.map(lambda p: oracle.quantize_fp8(a_f32[p[0]:p[1]], c["rinv"]), parts))
    ac = np.concatenate([q[0] for q in q4])
    asc = np.concatenate([q[1] for q in q4])
    a8 = np.concatenate(q8)
    ref, _ = oracle.gemm_bf16(a_bits, c["w_bits"], total=False)
    refb = oracle.gemm.to_bf16(ref)
    o44, _ = oracle.gemm_w4a4(ac, asc, c["rwc"], c["rws"], WL.K, total=False)
    s4, n4, _ = oracle.sqnr_db(refb, oracle.gemm.to_bf16(o44))
    del o44
    o48, _ = oracle.gemm_w4a8(a8, c["rs_a"], c["rwc"], c["rws"], WL.K, total=False)
    s8, n8, _ = oracle.sqnr_db(refb, oracle.gemm.to_bf16(o48))
    return (s4, n4), (s8, n8)


def _ensure(c, i):
    if i not in _partial:
        _partial[i] = _oracle_chunk(c, BOUNDS[i], BOUNDS[i + 1])
    return _partial[i]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("i", range(CHUNKS))
def test_full_size_sqnr_row_chunk(gpu, chain, i):
    r0, r1 = BOUNDS[i], BOUNDS[i + 1]
    (s4, n4), (s8, n8) = _ensure(chain, i)
    ref = chain["ref"][r0:r1]
    g4 = gpu.sqnr(ref, chain["o44"][r0:r1]).cpu().tolist()
    g8 = gpu.sqnr(ref, chain["o48"][r0:r1]).cpu().tolist()
    print(f"rows {r0}..{r1}: W4A4 {g4[2]:.4f} dB (oracle {_db(s4, n4):.4f}), "
          f"W4A8 {g8[2]:.4f} dB (oracle {_db(s8, n8):.4f})", flush=True)
    assert abs(g4[2] - _db(s4, n4)) < 0.01
    assert abs(g8[2] - _db(s8, n8)) < 0.01


@pytest.mark.timeout(900)
def test_full_size_sqnr_whole_output(gpu, chain):
    parts = [_ensure(chain, i) for i in range(CHUNKS)]
    s4 = sum(p[0][0] for p in parts)
    n4 = sum(p[0][1] for p in parts)
    s8 = sum(p[1][0] for p in parts)
    n8 = sum(p[1][1] for p in parts)
    d4, d8 = _db(s4, n4), _db(s8, n8)
    print(f"whole output: W4A4 {chain['r44'][2]:.4f} dB (oracle {d4:.4f}), "
          f"W4A8 {chain['r48'][2]:.4f} dB (oracle {d8:.4f})", flush=True)
    assert abs(chain["r44"][2] - d4) < 0.01
    assert abs(chain["r48"][2] - d8) < 0.01
    # the reference's signal power is common to both modes, and the GPU's matches
    assert abs(chain["r44"][0] - s4) <= 1e-4 * s4 and chain["r44"][0] == chain["r48"][0]
