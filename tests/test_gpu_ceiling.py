"""The MFMA ceiling measurement (mxq_mfma_ceiling) runs on real operand planes of every
GEMM mode, deterministically, and never reports more than the dense peak.

It is a measurement aid with no numeric result to compare: the checks are that the work
is done (the per-lane sink is finite and reproducible bit for bit, since fragments are
gathered from fixed pseudo-random positions) and that the rate is physically possible.
"""

import pytest
import torch

import workloads
from helpers import announce

pytestmark = pytest.mark.gpu

PEAK_TFLOPS = {"w4a4": 10100.0, "w4a8": 5000.0, "bf16": 2500.0}


@pytest.mark.parametrize("mode", ["w4a4", "w4a8", "bf16"])
def test_mfma_ceiling_runs_on_workload_operands(gpu, mode):
    a, w = workloads.workload_inputs("wan_ffn_down_sqnr", device="cuda", M=2048)
    if mode == "w4a4":
        ac, asc = gpu.quantize(a)
        wc, wsc = gpu.quantize(w)
        ops = (ac, asc, wc, wsc)
    elif mode == "w4a8":
        s_a, inv_s = gpu.fp8_static_scales(float(gpu.absmax(a).item()))
        wc, wsc = gpu.quantize(w)
        ops = (gpu.quantize_fp8(a, inv_s), None, wc, wsc)
    else:
        ops = (a, None, w, None)
    waves, iters = 2048, 200
    s1 = torch.full((waves * 64,), float("nan"), device="cuda")
    s2 = torch.full_like(s1, float("nan"))
    announce(f"mfma ceiling {mode}")
    gpu.mfma_ceiling(mode, *ops, waves=waves, iters=iters, sink=s1)     # warm-up, and the reference sink
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flop = gpu.mfma_ceiling(mode, *ops, waves=waves, iters=iters, sink=s2)
    e1.record()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(s1).all()), "sink not fully written"
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), "ceiling loop is not deterministic"
    tflops = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 0.05 * PEAK_TFLOPS[mode] < tflops <= 1.02 * PEAK_TFLOPS[mode], tflops
