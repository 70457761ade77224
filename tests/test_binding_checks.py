"""The binding's buffer checks (CPU): every tensor handed to the library -- inputs and
caller-supplied outputs or scratch -- is checked for device, dtype and shape before any
C call, so a host tensor or a short buffer never reaches a kernel.  Exercised on CPU and
meta tensors, with ``is_gpu`` standing them in for device tensors where needed."""

import pytest
import torch

import mxfp4_microscaled_quantization_amd as mxq

DEV = lambda t: True   # noqa: E731  (treat any tensor as a GPU tensor)


def test_check_buffer_accepts_matching_buffers():
    t = torch.empty((4, 16), dtype=torch.uint8, device="meta")
    assert mxq.check_buffer(t, "t", torch.uint8, (4, 16), is_gpu=DEV) == 16
    wide = torch.empty((4, 32), dtype=torch.bfloat16, device="meta")[:, :16]
    assert mxq.check_buffer(wide, "w", torch.bfloat16, (4, 16), is_gpu=DEV) == 32
    flat = torch.empty(10, dtype=torch.float64, device="meta")
    assert mxq.check_buffer(flat, "ws", torch.float64, min_numel=3, is_gpu=DEV) is None


@pytest.mark.parametrize("make,kw,needle", [
    (lambda: torch.empty((4, 16), dtype=torch.uint8), {}, "GPU tensor"),
    (lambda: "not a tensor", {}, "torch tensor"),
    (lambda: torch.empty((4, 16), dtype=torch.int8, device="meta"), {"is_gpu": DEV}, "torch.uint8"),
    (lambda: torch.empty((3, 16), dtype=torch.uint8, device="meta"), {"is_gpu": DEV}, "shape"),
    (lambda: torch.empty((4, 16), dtype=torch.uint8, device="meta"), {"is_gpu": DEV, "device": torch.device("cpu")},
     "expected cpu"),
    (lambda: torch.empty((16, 4), dtype=torch.uint8, device="meta").t(), {"is_gpu": DEV}, "contiguous rows"),
])
def test_check_buffer_rejects(make, kw, needle):
    with pytest.raises(ValueError, match=needle):
        mxq.check_buffer(make(), "buf", torch.uint8, (4, 16), **kw)


def test_check_buffer_flat_scratch():
    short = torch.empty(2, dtype=torch.float64, device="meta")
    with pytest.raises(ValueError, match="at least 3"):
        mxq.check_buffer(short, "out3", torch.float64, min_numel=3, is_gpu=DEV)
    strided = torch.empty(8, dtype=torch.float64, device="meta")[::2]
    with pytest.raises(ValueError, match="contiguous"):
        mxq.check_buffer(strided, "out3", torch.float64, min_numel=3, is_gpu=DEV)


@pytest.mark.parametrize("call", [
    lambda: mxq.quantize(torch.zeros(4, 64, dtype=torch.bfloat16)),
    lambda: mxq.quantize_into(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 32, dtype=torch.uint8),
                              torch.zeros(4, 2, dtype=torch.uint8)),
    lambda: mxq.quantize_fp8(torch.zeros(4, 64, dtype=torch.bfloat16), 1.0),
    lambda: mxq.gemm_w4a4(*(torch.zeros(s, dtype=torch.uint8) for s in ((4, 32), (4, 2), (8, 32), (8, 2)))),
    lambda: mxq.gemm_w4a8(torch.zeros(4, 64, dtype=torch.uint8), 1.0, torch.zeros(8, 32, dtype=torch.uint8),
                          torch.zeros(8, 2, dtype=torch.uint8)),
    lambda: mxq.gemm_bf16(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(8, 64, dtype=torch.bfloat16)),
    lambda: mxq.sqnr(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 64, dtype=torch.bfloat16)),
    lambda: mxq.dequantize(torch.zeros(4, 32, dtype=torch.uint8), torch.zeros(4, 2, dtype=torch.uint8), 64),
    lambda: mxq.dequantize_fp8(torch.zeros(4, 64, dtype=torch.uint8), 1.0),
])
def test_host_tensors_are_rejected_before_the_library(call):
    with pytest.raises(ValueError, match="GPU tensor"):
        call()
