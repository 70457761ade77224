"""The seeded generators are deterministic and have the stated shapes/statistics."""

import numpy as np
import torch

import workloads


def test_tiny_inputs_deterministic_and_shaped():
    a1, w1 = workloads.tiny_inputs(0)
    a2, w2 = workloads.tiny_inputs(0)
    assert a1.shape == (128, 256) and w1.shape == (128, 256)
    assert a1.dtype == np.float32 and w1.dtype == np.float32
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(w1, w2)
    assert 5.0 < np.max(np.abs(a1)) < 200.0          # outliers present
    assert 0.015 < np.std(w1) < 0.025


def test_generators_deterministic():
    x1 = workloads.activations(64, 96, "lognormal_channels", seed=3, name="t")
    x2 = workloads.activations(64, 96, "lognormal_channels", seed=3, name="t")
    assert x1.dtype == torch.bfloat16 and x1.shape == (64, 96)
    assert torch.equal(x1, x2)
    t = workloads.activations(256, 256, "student_t", seed=1, name="t", dtype=torch.float32)
    assert torch.isfinite(t).all()
    w = workloads.weights(300, 64, 0.015, seed=1, name="t", dtype=torch.float32)
    assert abs(w.std().item() - 0.015) < 0.001


def test_workload_table():
    for w in workloads.WORKLOADS.values():
        assert w.K % 32 == 0
    assert workloads.WORKLOADS["wan_ffn_down_sqnr"].modes == ("w4a4", "w4a8", "bf16")


def test_host_draw_is_device_and_thread_independent(monkeypatch):
    a1 = workloads.activations(3000, 64, "student_t", seed=5, name="thr")
    monkeypatch.setattr(workloads, "_THREADS", 1)
    a2 = workloads.activations(3000, 64, "student_t", seed=5, name="thr")
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    # a reduced-M draw is the first rows of the full draw
    a3 = workloads.activations(1500, 64, "student_t", seed=5, name="thr")
    assert torch.equal(a3.view(torch.int16), a1[:1500].view(torch.int16))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8 - 2 ** -20, 3.0e38], np.float32)
    got = workloads._bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
