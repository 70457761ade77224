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


class _FakeStep:
    """The host-side fields cpu_baseline reads from a step (CPU tensors)."""

    def __init__(self, modes):
        import torch
        import workloads
        self.wl = workloads.GemmShape("tiny_bench", 16, 256, 64, modes, "normal", 0.02)
        self.a = [workloads.activations(16, 256, "normal", seed=7, name="tb")]
        self.w = workloads.weights(64, 256, 0.02, seed=7, name="tb")
        self.s_a, self.inv_s = 0.01, 100.0
        self.torch = torch


def test_cpu_baseline_record():
    import torch
    st = _FakeStep(("w4a4",))
    rec = bench.cpu_baseline(None, torch, st, 16)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["seconds"] > 0
    assert isinstance(rec["cores"], int) and rec["cores"] >= 1
    assert "first 16 of 16 activation rows" in rec["sample"] and "extrapolated" in rec["sample"]
    rec8 = bench.cpu_baseline(None, torch, _FakeStep(("w4a8",)), 16)
    assert "W4A8" in rec8["sample"] and rec8["value"] > 0


def test_traffic_only_from_a_summary_of_the_same_source(tmp_path, monkeypatch):
    h = bench._src_hash(*bench.SRC_OF["mxq_gemm_w4a4"])
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "pmc_mxq_gemm_w4a4_wl.txt").write_text(
        f"kernel: k\nsource_sha256_16: {h}\nhbm_bytes_per_launch: 1.5000e+09\n")
    (tmp_path / "profiles" / "pmc_mxq_gemm_w4a8_wl.txt").write_text(
        "kernel: k\nsource_sha256_16: 0123456789abcdef\nhbm_bytes_per_launch: 1.5000e+09\n")
    src = tmp_path / "mxfp4_microscaled_quantization_amd" / "csrc"
    src.mkdir(parents=True)
    for name in ("gemm.hip", "gemm_scaled.hip"):
        (src / name).write_bytes(open(os.path.join(ROOT, "mxfp4_microscaled_quantization_amd", "csrc", name),
                                      "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic_from_profile("mxq_gemm_w4a4", "wl") == 1.5e9
    assert bench._traffic_from_profile("mxq_gemm_w4a8", "wl") is None    # kernel changed since
    assert bench._traffic_from_profile("mxq_gemm_bf16", "wl") is None    # no summary


def _write_csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_matches_step_order(tmp_path):
    import workloads
    wl = workloads.WORKLOADS["wan_ffn_down_sqnr"]
    seq = []
    for label, n in bench.step_kernels(wl):
        seq += [label] * n
    names = {"mxq_gemm_bf16": "gemm_bf16_kernel", "mxq_quantize": "mx_quantize_kernel<false, false>",
             "mxq_gemm_w4a4": "gemm_fast_kernel<0>", "mxq_quantize_fp8": "fp8_quantize_kernel<false>",
             "mxq_gemm_w4a8": "gemm_fast_kernel<1>", "mxq_sqnr_w4a4": "sqnr_partial_kernel",
             "mxq_sqnr_w4a8": "sqnr_partial_kernel"}
    rows, t, did = [], 0, 0
    for k in ["mx_quantize_kernel<false, false>", "at::native::elementwise_kernel"]:   # setup launches
        did += 1
        rows.append([did, f"mxq::(anonymous namespace)::{k}(int)" if "mxq" not in k and "at::" not in k else k, t, t + 5000])
        t += 10000
    for step in range(3):
        for label in seq:
            did += 1
            dur = 1000 * (1 + seq.index(label))
            rows.append([did, f"mxq::(anonymous namespace)::{names[label]}(mxq::Params)", t, t + dur])
            t += dur + 10
    _write_csv(tmp_path / "prof" / "x_kernel_trace.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                                          "End_Timestamp"], rows)
    out = tmp_path / "trace.txt"
    sys.argv = ["bench.py", "--summarize", "trace", "--input", str(tmp_path / "prof"), "--workload",
                "wan_ffn_down_sqnr", "--out", str(out), "--command", "rocprofv3 ... -- python bench.py --steps 2"]
    bench.main()
    text = out.read_text()
    w4a4 = [ln for ln in text.splitlines() if ln.startswith("mxq_gemm_w4a4")][0]
    assert "gemm_fast_kernel<0>" in w4a4 and " 2 " in w4a4          # the last two steps only
    assert "command: rocprofv3" in text


def test_stats_summary_groups_by_kernel_and_grid(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]
    q = "void mxq::(anonymous namespace)::mx_quantize_kernel<false, false, true>(void const*, long)"
    rows = [[1, q, 0, 400000, 1024, 1024 * 16384], [2, q, 500000, 910000, 1024, 1024 * 16384],
            [3, q, 1000000, 1034000, 1024, 1024 * 2160], [4, "at::native::copy", 0, 10, 256, 256]]
    _write_csv(tmp_path / "prof" / "x_kernel_trace.csv", hdr, rows)
    out = tmp_path / "stats.txt"
    sys.argv = ["bench.py", "--summarize", "stats", "--input", str(tmp_path / "prof"), "--workload",
                "wan_ffn_down_sqnr", "--out", str(out), "--command", "rocprofv3 --kernel-trace -- python bench.py"]
    bench.main()
    lines = [ln.split() for ln in out.read_text().splitlines() if not ln.startswith("#")]
    assert [(ln[0], ln[1], ln[2]) for ln in lines] == [("2", "16384", "405.0"), ("1", "2160", "34.0")]
    assert all("mx_quantize_kernel<false," in " ".join(ln) for ln in lines)   # torch's kernels left out


def test_waves_summary_gives_fractions_of_wave_cycles(tmp_path):
    import workloads
    wl = workloads.WORKLOADS["flux_ffn_up_w4a4"]
    seq = []
    for label, n in bench.step_kernels(wl):
        seq += [label] * n
    names = {"mxq_quantize": "mx_quantize_kernel<false, false, true>", "mxq_gemm_w4a4": "gemm_fast_kernel<0, true>"}
    ctr = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 150.0, "SQ_WAIT_INST_ANY": 450.0, "SQ_ACTIVE_INST_ANY": 400.0,
           "SQ_ACTIVE_INST_LDS": 60.0, "SQ_ACTIVE_INST_VMEM": 40.0, "SQ_LDS_BANK_CONFLICT": 25.0,
           "SQ_LDS_IDX_ACTIVE": 100.0}
    rows, did = [], 0
    for step in range(2):
        for label in seq:
            did += 1
            for c, v in ctr.items():   # two shader engines' halves of each counter
                rows += [[did, f"void mxq::(anonymous namespace)::{names[label]}(mxq::Params)", c, v / 2]] * 2
    _write_csv(tmp_path / "prof" / "x_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                                                "Counter_Value"], rows)
    out = tmp_path / "waves.txt"
    sys.argv = ["bench.py", "--summarize", "waves", "--input", str(tmp_path / "prof"), "--workload",
                "flux_ffn_up_w4a4", "--out", str(out), "--command", "rocprofv3 --pmc ... -- python bench.py --steps 2"]
    bench.main()
    g = [ln for ln in out.read_text().splitlines() if ln.startswith("mxq_gemm_w4a4")][0]
    assert "wait 0.150 issue_wait 0.450 active 0.400 lds 0.060 vmem 0.040 lds_conflict 0.250" in g


def test_committed_summaries_name_their_kernel_and_command():
    prof = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(prof))
    assert any(n.startswith("kernel_trace_") for n in names)
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "command" in text, n
        if n.startswith("pmc_"):
            assert "source_sha256_16:" in text and "hbm_bytes_per_launch:" in text, n
