"""The allocation-free SQNR entry point (mxq_sqnr_noalloc), called through the C ABI,
against the workspace entry point (mxq_sqnr) on the same inputs: the same kernels and
partition, so the three doubles must agree bit for bit, and both within 0.01 dB of the
oracle.  Two calls in a row on one GPU, the second on a smaller input, check that no
state carries over in the shared scratch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import announce, to_np_bf16_bits

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("shapes", [[(2048, 5120), (37, 520)], [(75600, 64), (1, 8)]])
def test_sqnr_noalloc_matches_sqnr_twice(gpu, shapes):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for rows, cols in shapes:
        ref = workloads.activations(rows, cols, "student_t", seed=rows, name="noalloc_ref", device="cuda")
        noise = workloads.activations(rows, cols, "lognormal_channels", seed=cols, name="noalloc_n", device="cuda")
        test = (ref.float() + 0.05 * noise.float()).to(torch.bfloat16)
        nb = gpu.lib.mxq_sqnr_workspace_bytes(rows * cols)
        ws = torch.empty(nb // 8, dtype=torch.float64, device="cuda")
        out_ws = torch.full((3,), -1.0, dtype=torch.float64, device="cuda")
        out_na = torch.full((3,), -2.0, dtype=torch.float64, device="cuda")
        announce(f"mxq_sqnr_noalloc {rows}x{cols}")
        st = gpu.lib.mxq_sqnr(_ptr(ref), _ptr(test), rows, cols, cols, cols, _ptr(ws), nb, _ptr(out_ws), stream)
        assert st == 0, gpu.lib.mxq_last_error()
        st = gpu.lib.mxq_sqnr_noalloc(_ptr(ref), _ptr(test), rows, cols, cols, cols, _ptr(out_na), stream)
        assert st == 0, gpu.lib.mxq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), (out_na.tolist(), out_ws.tolist())
        rs, rn, rd = oracle.sqnr_db(to_np_bf16_bits(ref), to_np_bf16_bits(test))
        assert abs(out_na[2].item() - rd) < 0.01


def test_sqnr_noalloc_binding_and_strided_views(gpu):
    full = workloads.activations(600, 1032, "student_t", seed=2, name="noalloc_det", device="cuda")
    ref, test = full[:, :1024], full[:, 8:]
    out = torch.empty(3, dtype=torch.float64, device="cuda")
    announce("mxq_sqnr_noalloc strided")
    gpu.sqnr_noalloc(ref, test, out)
    expect = gpu.sqnr(ref, test)
    torch.cuda.synchronize()
    assert torch.equal(out, expect)


def test_sqnr_noalloc_rejects_bad_arguments(gpu):
    out = torch.empty(3, dtype=torch.float64, device="cuda")
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda")
    st = gpu.lib.mxq_sqnr_noalloc(_ptr(x), _ptr(x), 4, 12, 12, 12, _ptr(out), None)
    assert st == gpu.MXQ_ERR_INVALID_ARG and b"multiple of 8" in gpu.lib.mxq_last_error()
    st = gpu.lib.mxq_sqnr_noalloc(_ptr(x), _ptr(x), 4, 8, 12, 12, None, None)
    assert st == gpu.MXQ_ERR_INVALID_ARG
