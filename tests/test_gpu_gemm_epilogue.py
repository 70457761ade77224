"""Output layouts of the three GEMMs.

The epilogue picks its store width from the output pitch and base address: 16-byte row
segments staged through LDS (pitch a multiple of 8 elements, 16-byte aligned base), 8-byte
stores (pitch a multiple of 4, 8-byte aligned base) or single elements.  Writing into a
row-strided view must give the same bits as a contiguous output, on a shape with partial
tiles in both M and N, and leave every element outside the view untouched.
"""

import pytest
import torch

import workloads
from helpers import announce

pytestmark = pytest.mark.gpu

M, N = 300, 520
SENTINEL = 0x7FC1          # a bf16 NaN pattern no GEMM output can take


def _operands(gpu, mode, K):
    a = workloads.activations(M, K, "student_t", seed=K, name="epilogue", device="cuda")
    w = workloads.weights(N, K, 0.015, seed=K + 1, name="epilogue", device="cuda")
    if mode == "w4a4":
        ac, asc = gpu.quantize(a)
        wc, wsc = gpu.quantize(w)
        return lambda out=None: gpu.gemm_w4a4(ac, asc, wc, wsc, out=out)
    if mode == "w4a8":
        s_a, inv_s = gpu.fp8_static_scales(float(gpu.absmax(a).item()))
        a8 = gpu.quantize_fp8(a, inv_s)
        wc, wsc = gpu.quantize(w)
        return lambda out=None: gpu.gemm_w4a8(a8, s_a, wc, wsc, out=out)
    return lambda out=None: gpu.gemm_bf16(a, w, out=out)


# (pitch padding, column offset of the view): 16-byte path, 8-byte path, element path
# (odd pitch), element path (base 2 bytes past a 16-byte boundary)
LAYOUTS = [(8, 0), (4, 0), (1, 0), (8, 1)]


@pytest.mark.parametrize("mode", ["w4a4", "w4a8", "bf16"])
# fast path with non-temporal staged stores (K <= 8192), with ordinary ones (K > 8192);
# generic path (K % 64 != 0)
@pytest.mark.parametrize("K", [1024, 8704, 480])
def test_strided_outputs_match_contiguous(gpu, mode, K):
    run = _operands(gpu, mode, K)
    announce(f"epilogue {mode} {M}x{N}x{K} contiguous")
    ref = run().view(torch.int16)
    torch.cuda.synchronize()
    for pad, off in LAYOUTS:
        full = torch.full((M, N + pad + off), SENTINEL, dtype=torch.int16, device="cuda")
        view = full.view(torch.bfloat16)[:, off:off + N]
        announce(f"epilogue {mode} K={K} pitch {N + pad + off} offset {off}")
        run(out=view)
        torch.cuda.synchronize()
        assert torch.equal(full[:, off:off + N], ref), f"{mode} K={K} pad={pad} off={off}: values differ"
        outside = torch.cat([full[:, :off], full[:, off + N:]], dim=1)
        assert bool((outside == SENTINEL).all()), f"{mode} K={K} pad={pad} off={off}: wrote outside the view"
