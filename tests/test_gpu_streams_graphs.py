"""The library on several streams and inside a captured HIP graph.

Every entry point only enqueues work on the caller's stream, allocates nothing and keeps
no state between calls, so:
* two streams running the path concurrently on different inputs give the same bits as
  running it on one stream;
* the whole step (MXFP4 and FP8 quantization, the W4A4 / W4A8 / bf16 GEMMs, both SQNRs,
  and the fused W4A4) captured in one graph and replayed several times, with eager work
  between the replays, reproduces the eager results bit for bit on every replay.
"""

import numpy as np
import pytest
import torch

from helpers import announce

pytestmark = pytest.mark.gpu

M, K, N = 1024, 3072, 1280


def _inputs(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    a = (torch.randn(M, K, device="cuda", generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    return a, w


class _Step:
    """Preallocated buffers and one pass of the path on the current stream."""

    def __init__(self, mxq, a, w):
        self.mxq, self.a, self.w = mxq, a, w
        self.wc, self.wsc = mxq.quantize(w)
        amax = float(mxq.absmax(a).item())
        self.s_a, self.inv_s = mxq.fp8_static_scales(amax)
        dev = a.device
        self.ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        self.asc = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        self.a8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
        self.o44 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.o48 = torch.empty_like(self.o44)
        self.ref = torch.empty_like(self.o44)
        self.of = torch.empty_like(self.o44)
        self.ws1 = torch.empty(mxq.sqnr_workspace_bytes(M * N) // 8, dtype=torch.float64, device=dev)
        self.ws2 = torch.empty_like(self.ws1)
        self.r44 = torch.empty(3, dtype=torch.float64, device=dev)
        self.r48 = torch.empty(3, dtype=torch.float64, device=dev)

    def run(self):
        m = self.mxq
        m.quantize_into(self.a, self.ac, self.asc)
        m.quantize_fp8(self.a, self.inv_s, out=self.a8)
        m.gemm_w4a4(self.ac, self.asc, self.wc, self.wsc, out=self.o44)
        m.gemm_w4a8(self.a8, self.s_a, self.wc, self.wsc, out=self.o48)
        m.gemm_bf16(self.a, self.w, out=self.ref)
        m.sqnr(self.ref, self.o44, workspace=self.ws1, out3=self.r44)
        m.sqnr(self.ref, self.o48, workspace=self.ws2, out3=self.r48)
        m.gemm_w4a4_fused(self.a, self.wc, self.wsc, out=self.of, route=False)

    def outputs(self):
        return [t.clone() for t in (self.ac, self.asc, self.a8, self.o44, self.o48, self.ref, self.of,
                                    self.r44, self.r48)]

    def clear(self):
        for t in (self.ac, self.asc, self.a8):
            t.fill_(0x55)
        for t in (self.o44, self.o48, self.ref, self.of):
            t.fill_(-3.0)
        self.r44.fill_(-1.0)
        self.r48.fill_(-1.0)


def _same(xs, ys):
    """Index of the first output that differs bit for bit, or -1."""
    bits = {torch.bfloat16: torch.int16, torch.float64: torch.int64}
    for i, (x, y) in enumerate(zip(xs, ys)):
        if x.dtype in bits:
            x, y = x.view(bits[x.dtype]), y.view(bits[y.dtype])
        if not torch.equal(x, y):
            return i
    return -1


def test_two_streams_concurrently(gpu):
    s1, s2 = _Step(gpu, *_inputs(1)), _Step(gpu, *_inputs(2))
    announce("two streams: sequential reference")
    s1.run()
    s2.run()
    torch.cuda.synchronize()
    ref1, ref2 = s1.outputs(), s2.outputs()
    s1.clear()
    s2.clear()
    torch.cuda.synchronize()
    st1, st2 = torch.cuda.Stream(), torch.cuda.Stream()
    announce("two streams: concurrent")
    for _ in range(3):
        with torch.cuda.stream(st1):
            s1.run()
        with torch.cuda.stream(st2):
            s2.run()
    torch.cuda.synchronize()
    assert _same(s1.outputs(), ref1) == -1 and _same(s2.outputs(), ref2) == -1


def test_captured_graph_replays_match_eager(gpu):
    step = _Step(gpu, *_inputs(3))
    announce("graph: eager reference")
    step.run()
    torch.cuda.synchronize()
    eager = step.outputs()
    # warm up on a side stream, as graph capture expects, then capture one pass
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    announce("graph: capture")
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()
    other = _Step(gpu, *_inputs(4))
    for r in range(3):
        step.clear()
        torch.cuda.synchronize()
        announce(f"graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        bad = _same(step.outputs(), eager)
        assert bad == -1, f"replay {r}: output {bad} differs from the eager pass"
        other.run()                      # eager work between replays
        torch.cuda.synchronize()
    assert np.isfinite(float(step.r44[2].item()))
