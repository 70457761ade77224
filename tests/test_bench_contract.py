"""Host-side pieces of bench.py: the one-GPU refusal, the CPU oracle baseline record and
the rule that HBM traffic is only taken from a counter summary of the current source."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_record():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((16, 256)).astype(np.float32)
    a = ((a.view(np.uint32) >> 16) << 16).view(np.float32)          # bf16-representable rows
    w = rng.standard_normal((64, 256)).astype(np.float32) * 0.02
    w_bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    rec = bench.cpu_baseline("tiny", 16, a, w_bits)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["seconds"] > 0
    assert isinstance(rec["cores"], int) and rec["cores"] >= 1
    assert "16 activation rows" in rec["sample"]


def test_traffic_only_from_a_summary_of_the_same_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "pmc_k_wl.txt").write_text(
        "kernel: k\nsource_sha256_16: 0123456789abcdef\nhbm_bytes_per_launch: 1.5000e+09\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic_from_profile("k_wl", "0123456789abcdef") == 1.5e9
    assert bench._traffic_from_profile("k_wl", "fedcba9876543210") is None   # kernel changed since
    assert bench._traffic_from_profile("other_wl", "0123456789abcdef") is None


def test_committed_summaries_name_their_kernel_and_command():
    prof = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(prof))
    assert any(n.startswith("kernel_trace_") for n in names)
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "command" in text, n
        if n.startswith("pmc_"):
            assert "source_sha256_16:" in text and "hbm_bytes_per_launch:" in text, n
