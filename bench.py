"""Benchmark of the MXFP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-extras] [--no-configs]
    python bench.py --summarize {trace,pmc,mfma,stats} --input DIR --workload NAME [--out FILE]
    python bench.py --copy-calibration

A step is one pass of the whole hot path over one batch of synthetic activations already
resident in HBM (weights are quantized once, offline, as in deployment; the static FP8
scale is calibrated once, before timing).  On the Wan2.2 FFN-down workload (the default,
the one configuration that holds every step) a step is, in this order:

  1. mxq_gemm_bf16      bf16 reference (the SQNR baseline)
  2. mxq_quantize       dynamic MXFP4 activations (bf16 -> codes + E8M0 scales)
  3. mxq_gemm_w4a4      MXFP4 x MXFP4 -> bf16
  4. mxq_quantize_fp8   static FP8 E4M3 activations
  5. mxq_gemm_w4a8      FP8 x MXFP4 -> bf16
  6. mxq_sqnr x 2       whole-output SQNR of W4A4 and W4A8 against the reference

Other workloads run only their own modes (W4A4: steps 2-3; W4A8: steps 4-5).  Steps
alternate between two copies of the activations, so no step re-reads lines the previous
one left in the caches.

Prints ONE JSON line.  `value` is the W4A4 GEMM's throughput (TFLOP/s) on the step's
workload, from its mean HIP-event time on the stream the kernels run on; `metric_values`
gives W4A4 and W4A8 beside each other; `roofline` is the W4A4 GEMM against the dense
MXFP4 peak.  `kernels` gives every step kernel's rate (mean, median, standard deviation,
coefficient of variation) against its own roofline.  Unless --no-extras: `configs` times
the other workloads' own kernels the same way (not with --no-configs), `mfma_ceiling` the
power-limited MFMA ceiling on the step's operand bits, `next` the follow-on paths (fused
W4A4, QDQ emulation, Hadamard rotation, UOS scales).  `cpu_baseline` times the CPU oracle on a
bounded row sample of the same workload and checks its SQNR against the GPU's on the
same rows.

--summarize turns rocprofv3 CSV output (run on `bench.py --workload NAME --no-extras
--no-cpu-baseline`; for `stats`, a whole run with --no-configs) into the text summaries
kept under profiles/.
"""

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
PEAK = {"hbm_GBps": 8000.0, "fp4_TFLOPs": 10100.0, "fp8_TFLOPs": 5000.0, "bf16_TFLOPs": 2500.0}
DEFAULT_WORKLOAD = "wan_ffn_down_sqnr"
OTHER_CONFIGS = ("flux_qkv_w4a4", "flux_ffn_up_w4a4", "flux_ffn_down_w4a4", "wan_ffn_up_w4a8")
METRIC = "W4A4/W4A8 GEMM TFLOP/s (% of MXFP4/FP8 peak); quantize GB/s (% of HBM)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="time the step only (for profiling)")
    p.add_argument("--no-configs", action="store_true", help="skip the other workloads' section")
    p.add_argument("--cpu-rows", type=int, default=2048, help="activation rows in the CPU oracle sample")
    p.add_argument("--config-reps", type=int, default=10, help="timed launches per kernel in the configs section")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of known size (for HBM counter scaling)")
    p.add_argument("--summarize", choices=("trace", "pmc", "mfma", "stats", "waves"),
                   help="summarize rocprofv3 CSV output")
    p.add_argument("--input", help="rocprofv3 output directory (--summarize; pmc: FETCH_DIR,WRITE_DIR)")
    p.add_argument("--copy-input", help="--copy-calibration counter directories COPY_FETCH_DIR,COPY_WRITE_DIR (pmc)")
    p.add_argument("--out", help="summary file to write (--summarize; pmc: a directory); stdout if absent")
    p.add_argument("--command", default="", help="the profiling command(s), recorded in the summary (' ;; '-separated)")
    return p.parse_args()


# ---------------------------------------------------------------------------- step definition

def step_kernels(wl):
    """Ordered (label, launches per call) of one step of workload `wl`."""
    modes = wl.modes
    seq = []
    if "bf16" in modes:
        seq.append(("mxq_gemm_bf16", 1))
    if "w4a4" in modes:
        seq += [("mxq_quantize", 1), ("mxq_gemm_w4a4", 1)]
    if "w4a8" in modes:
        seq += [("mxq_quantize_fp8", 1), ("mxq_gemm_w4a8", 1)]
    if "bf16" in modes:
        if "w4a4" in modes:
            seq.append(("mxq_sqnr_w4a4", 2))
        if "w4a8" in modes:
            seq.append(("mxq_sqnr_w4a8", 2))
    return seq


def work_table(wl):
    """Algorithmic units per launch: (amount, unit, peak, bound)."""
    M, K, N = wl.M, wl.K, wl.N
    flop = 2.0 * M * N * K
    return {
        "mxq_quantize": (M * K * (2 + 0.5 + 1 / 32), "GB/s", PEAK["hbm_GBps"], "hbm"),
        "mxq_quantize_fp8": (M * K * 3.0, "GB/s", PEAK["hbm_GBps"], "hbm"),
        "mxq_gemm_w4a4": (flop, "TFLOP/s", PEAK["fp4_TFLOPs"], "mfma"),
        "mxq_gemm_w4a8": (flop, "TFLOP/s", PEAK["fp8_TFLOPs"], "mfma"),
        "mxq_gemm_bf16": (flop, "TFLOP/s", PEAK["bf16_TFLOPs"], "mfma"),
        "mxq_sqnr_w4a4": (M * N * 4.0, "GB/s", PEAK["hbm_GBps"], "hbm"),
        "mxq_sqnr_w4a8": (M * N * 4.0, "GB/s", PEAK["hbm_GBps"], "hbm"),
    }


def algorithmic_bytes(wl, label):
    """Bytes the step itself must move per launch (inputs read once, outputs written once)."""
    M, K, N = wl.M, wl.K, wl.N
    mx = lambda r: r * (K // 2 + K // 32)   # noqa: E731  (codes + scales)
    return {"mxq_quantize": M * K * (2 + 0.5 + 1 / 32), "mxq_quantize_fp8": M * K * 3.0,
            "mxq_gemm_w4a4": mx(M) + mx(N) + 2.0 * M * N, "mxq_gemm_w4a8": M * K + mx(N) + 2.0 * M * N,
            "mxq_gemm_bf16": 2.0 * (M * K + N * K + M * N), "mxq_sqnr_w4a4": 4.0 * M * N,
            "mxq_sqnr_w4a8": 4.0 * M * N}[label]


SRC_OF = {"mxq_quantize": ("quantize.hip",), "mxq_quantize_fp8": ("quantize.hip",), "mxq_gemm_w4a4": ("gemm.hip", "gemm_scaled.hip"),
          "mxq_gemm_w4a8": ("gemm.hip", "gemm_scaled.hip"), "mxq_gemm_bf16": ("gemm.hip",), "mxq_sqnr_w4a4": ("sqnr.hip",),
          "mxq_sqnr_w4a8": ("sqnr.hip",)}


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp4_microscaled_quantization_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_from_profile(label: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it matches the source."""
    key = "mxq_sqnr" if label.startswith("mxq_sqnr") else label
    path = os.path.join(ROOT, "profiles", f"pmc_{key}_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != _src_hash(*SRC_OF[label]):
        return None
    return float(m_val.group(1))


def _rate(amount, unit, ms):
    return amount / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)


def _kinfo(label, samples_ms, wl, workload):
    import numpy as np
    amount, unit, peak, bound = work_table(wl)[label]
    t = np.asarray(samples_ms)
    ms = float(np.mean(t))
    rate = _rate(amount, unit, ms)
    return {"ms": round(ms, 4), "median_ms": round(float(np.median(t)), 4), "std_ms": round(float(np.std(t)), 4),
            "cv": round(float(np.std(t) / ms), 4), "achieved": round(rate, 2), "unit": unit, "peak": peak,
            "frac": round(rate / peak, 4), "bound": bound, "traffic": _traffic_from_profile(label, workload)}


# ---------------------------------------------------------------------------- GPU side

class Step:
    """Buffers and kernel closures of one workload's step (two activation copies)."""

    def __init__(self, mxq, workloads, torch, name, dev):
        self.wl = wl = workloads.WORKLOADS[name]
        M, K, N = wl.M, wl.K, wl.N
        a, w = workloads.workload_inputs(name, device=dev)
        self.a = [a, a.clone()]                       # rotated between steps
        self.w = w
        self.wc, self.wsc = mxq.quantize(w)           # offline weight preparation
        amax = float(mxq.absmax(a).item())            # static calibration
        self.s_a, self.inv_s = mxq.fp8_static_scales(amax)
        modes = wl.modes
        self.ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if "w4a4" in modes else None
        self.asc = torch.empty((M, K // 32), dtype=torch.uint8, device=dev) if "w4a4" in modes else None
        self.a8 = torch.empty((M, K), dtype=torch.uint8, device=dev) if "w4a8" in modes else None
        out = lambda: torch.empty((M, N), dtype=torch.bfloat16, device=dev)   # noqa: E731
        self.o44 = out() if "w4a4" in modes else None
        self.o48 = out() if "w4a8" in modes else None
        self.ref = out() if "bf16" in modes else None
        self.r44 = torch.zeros(3, dtype=torch.float64, device=dev)
        self.r48 = torch.zeros(3, dtype=torch.float64, device=dev)
        self.ws = torch.empty(mxq.sqnr_workspace_bytes(M * N) // 8, dtype=torch.float64, device=dev)
        s = self
        self.fns = {
            "mxq_gemm_bf16": lambda i: mxq.gemm_bf16(s.a[i], s.w, out=s.ref),
            "mxq_quantize": lambda i: mxq.quantize_into(s.a[i], s.ac, s.asc),
            "mxq_gemm_w4a4": lambda i: mxq.gemm_w4a4(s.ac, s.asc, s.wc, s.wsc, out=s.o44),
            "mxq_quantize_fp8": lambda i: mxq.quantize_fp8(s.a[i], s.inv_s, out=s.a8),
            "mxq_gemm_w4a8": lambda i: mxq.gemm_w4a8(s.a8, s.s_a, s.wc, s.wsc, out=s.o48),
            "mxq_sqnr_w4a4": lambda i: mxq.sqnr(s.ref, s.o44, workspace=s.ws, out3=s.r44),
            "mxq_sqnr_w4a8": lambda i: mxq.sqnr(s.ref, s.o48, workspace=s.ws, out3=s.r48),
        }
        self.seq = [label for label, _ in step_kernels(wl)]

    def run(self, i, stream=None, events=None):
        for j, label in enumerate(self.seq):
            self.fns[label](i & 1)
            if events is not None:
                events[j + 1].record(stream)


def time_steps(torch, st, steps, warmup):
    """Warm up, then time exactly `steps` steps (events around every kernel)."""
    import numpy as np
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        st.run(i)
    torch.cuda.synchronize()
    n = len(st.seq)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        st.run(s, stream, ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    samples = {label: [ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(steps)] for j, label in enumerate(st.seq)}
    step_ms = float(np.mean([ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]))
    return samples, wall, step_ms


def time_fn(torch, fn, n=10):
    stream = torch.cuda.current_stream()
    fn(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i + 1)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def copy_calibration():
    import torch
    n = 1 << 30                       # 1 GiB read + 1 GiB written per launch
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 5}))


def warm_up(torch, st, min_ms=200.0, min_steps=20):
    """Untimed steps until the GPU has run this step for `min_ms` (at least `min_steps`).

    The clock settles over tens of milliseconds of sustained work; this section follows the
    CPU-oracle baseline, during which the GPU idles, and its steps are short (FLUX FFN-up:
    ~1.2 ms), so a few warm-up steps leave the timed ones on the ramp."""
    t0 = time.perf_counter()
    i = 0
    while i < min_steps or (time.perf_counter() - t0) * 1e3 < min_ms:
        st.run(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def configs_section(mxq, workloads, torch, dev, reps):
    """Each other workload's own kernels, timed like the step (rotated activations)."""
    out = {}
    for name in OTHER_CONFIGS:
        st = Step(mxq, workloads, torch, name, dev)
        warm = warm_up(torch, st)
        samples, _, step_ms = time_steps(torch, st, reps, 0)
        wl = st.wl
        kern = {label: _kinfo(label, samples[label], wl, name) for label in st.seq}
        out[name] = {"shape": f"{wl.M}x{wl.K} @ {wl.K}x{wl.N}", "activations": wl.act, "step_ms": round(step_ms, 4),
                     "warmup_steps": warm, "kernels": kern}
        del st
        torch.cuda.empty_cache()
    return out


def extras(mxq, torch, st, res, dev):
    """Outside the timed step: MFMA ceilings, fused W4A4, QDQ emulation, Hadamard, UOS."""
    wl = st.wl
    M, K, N = wl.M, wl.K, wl.N
    flop = 2.0 * M * N * K
    a = st.a[0]
    kin = res["kernels"]
    # the power-limited MFMA ceiling on the step's own operand bits
    waves = 4096
    sink = torch.empty(waves * 64, dtype=torch.float32, device=dev)
    ceiling = {"what": "register-only loop of the GEMM's MFMA instruction on fragments of the step's operands"}
    st.fns["mxq_quantize"](0)
    st.fns["mxq_quantize_fp8"](0)
    for name, mode, ops, iters in (("mxq_gemm_w4a4", "w4a4", (st.ac, st.asc, st.wc, st.wsc), 1500),
                                   ("mxq_gemm_w4a8", "w4a8", (st.a8, None, st.wc, st.wsc), 1000),
                                   ("mxq_gemm_bf16", "bf16", (a, None, st.w, None), 3000)):
        ms_c = time_fn(torch, lambda i: mxq.mfma_ceiling(mode, *ops, waves=waves, iters=iters, sink=sink), n=3)
        rate_c = waves * iters * 16 * mxq.MFMA_FLOP[mode] / (ms_c * 1e-3) / 1e12
        peak = work_table(wl)[name][2]
        ceiling[name] = {"achieved": round(rate_c, 2), "unit": "TFLOP/s", "peak": peak,
                         "frac_of_peak": round(rate_c / peak, 4),
                         "gemm_frac_of_ceiling": round(kin[name]["achieved"] / rate_c, 4)}
    res["mfma_ceiling"] = ceiling
    del sink

    def gb(amount, ms):
        r = amount / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "achieved": round(r, 2), "unit": "GB/s", "peak": PEAK["hbm_GBps"],
                "frac": round(r / PEAK["hbm_GBps"], 4)}

    def tf(ms, peak):
        r = flop / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "achieved": round(r, 2), "unit": "TFLOP/s", "peak": peak, "frac": round(r / peak, 4)}

    q_amount = work_table(wl)["mxq_quantize"][0]
    db = lambda t: round(float(t[2].item()), 4)   # noqa: E731
    # W4A4 with the activation quantization fused into the GEMM, checked bit for bit: the
    # fused kernel itself (no workspace) and the call with a workspace, which past the
    # kernel's break-even quantizes in a pass of its own
    o_f = torch.empty_like(st.o44)
    o_r = torch.empty_like(st.o44)
    ws_bytes = mxq.fused_workspace_bytes(M, wl.N, K)
    ms_f = time_fn(torch, lambda i: mxq.gemm_w4a4_fused(st.a[i & 1], st.wc, st.wsc, out=o_f, route=False))
    ms_r = time_fn(torch, lambda i: mxq.gemm_w4a4_fused(st.a[i & 1], st.wc, st.wsc, out=o_r))
    st.fns["mxq_quantize"](0)
    st.fns["mxq_gemm_w4a4"](0)
    torch.cuda.synchronize()
    fused = {"mxq_gemm_w4a4_fused": tf(ms_f, PEAK["fp4_TFLOPs"]),
             "with_workspace": dict(tf(ms_r, PEAK["fp4_TFLOPs"]), routed=ws_bytes > 0, workspace_bytes=ws_bytes),
             "quantize_plus_w4a4_ms": round(kin["mxq_quantize"]["ms"] + kin["mxq_gemm_w4a4"]["ms"], 4),
             "bit_identical_to_quantize_then_w4a4": bool(torch.equal(o_f.view(torch.int16), st.o44.view(torch.int16))
                                                         and torch.equal(o_r.view(torch.int16),
                                                                         st.o44.view(torch.int16)))}
    del o_f, o_r
    # QDQ emulation (how the pages measured W4A8 quality): dequantize to bf16, bf16 GEMM
    y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    wdq = mxq.dequantize(st.wc, st.wsc, K)
    o_q = torch.empty_like(st.o44)
    st.fns["mxq_quantize"](0)
    ms_dq = time_fn(torch, lambda i: mxq.dequantize(st.ac, st.asc, K, out=y))
    mxq.gemm_bf16(y, wdq, out=o_q)
    r_q44 = mxq.sqnr(st.ref, o_q).clone()
    st.fns["mxq_quantize_fp8"](0)
    ms_dq8 = time_fn(torch, lambda i: mxq.dequantize_fp8(st.a8, st.s_a, out=y))
    ms_qg = time_fn(torch, lambda i: mxq.gemm_bf16(y, wdq, out=o_q), n=5)
    r_q48 = mxq.sqnr(st.ref, o_q).clone()
    torch.cuda.synchronize()
    qdq = {"mxq_dequantize": gb(M * K * (0.5 + 1 / 32 + 2), ms_dq),
           "mxq_dequantize_fp8": gb(M * K * 3.0, ms_dq8),
           "qdq_gemm_bf16": tf(ms_qg, PEAK["bf16_TFLOPs"]),
           "qdq_chain_ms": {"w4a4": round(kin["mxq_quantize"]["ms"] + ms_dq + ms_qg, 4),
                            "w4a8": round(kin["mxq_quantize_fp8"]["ms"] + ms_dq8 + ms_qg, 4)},
           "native_chain_ms": {"w4a4": round(kin["mxq_quantize"]["ms"] + kin["mxq_gemm_w4a4"]["ms"], 4),
                               "w4a8": round(kin["mxq_quantize_fp8"]["ms"] + kin["mxq_gemm_w4a8"]["ms"], 4)},
           "sqnr_db": {"qdq_w4a4": db(r_q44), "native_w4a4": res["sqnr_db"]["w4a4"],
                       "qdq_w4a8": db(r_q48), "native_w4a8": res["sqnr_db"]["w4a8"]}}
    del y, wdq, o_q
    # block-Hadamard rotation + MXFP4 of both operands (weights offline), n = 64 and 256
    hada = {}
    o_h = torch.empty_like(st.o44)
    for n in (64, 256):
        ms_h = time_fn(torch, lambda i: mxq.quantize_hadamard(st.a[i & 1], n))
        rwc, rwsc = mxq.quantize_hadamard(st.w, n)
        rac, rasc = mxq.quantize_hadamard(a, n)
        mxq.gemm_w4a4(rac, rasc, rwc, rwsc, out=o_h)
        hada[f"n{n}"] = {"mxq_quantize_hadamard": gb(q_amount, ms_h), "sqnr_db_w4a4": db(mxq.sqnr(st.ref, o_h))}
        del rwc, rwsc, rac, rasc
    # the UOS scale rule (both operands)
    ms_uos = time_fn(torch, lambda i: mxq.quantize_into(st.a[i & 1], st.ac, st.asc, rule="uos"))
    wc_u, wsc_u = mxq.quantize(st.w, rule="uos")
    mxq.quantize_into(a, st.ac, st.asc, rule="uos")
    mxq.gemm_w4a4(st.ac, st.asc, wc_u, wsc_u, out=o_h)
    uos = {"mxq_quantize_uos": gb(q_amount, ms_uos),
           "sqnr_db_w4a4": {"ocp": res["sqnr_db"]["w4a4"], "uos": db(mxq.sqnr(st.ref, o_h))}}
    del o_h, wc_u, wsc_u
    res["next"] = {"fused_activation_quant": fused, "qdq_emulation": qdq, "hadamard_rotation": hada,
                   "uos_scale_rule": uos}


def cpu_baseline(mxq, torch, st, rows):
    """The oracle as it stands on the first `rows` activation rows of the step's workload:
    its path for the headline GEMM (MXFP4 quantization + float64 W4A4 GEMM; FP8 + W4A8 on
    a W4A8-only workload) timed as the rate, then the rest of its chain (FP8, W4A8, bf16
    reference, SQNRs) with the SQNR of the same rows from the GPU beside it."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    wl = st.wl
    K, N = wl.K, wl.N
    a_bits = st.a[0][:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    w_bits = st.w.view(torch.int16).cpu().numpy().view(np.uint16)
    a32 = (a_bits.astype(np.uint32) << 16).view(np.float32)
    wc, ws = oracle.quantize_mxfp4((w_bits.astype(np.uint32) << 16).view(np.float32))   # offline: untimed
    s_a, inv_s = np.float32(st.s_a), np.float32(st.inv_s)        # the whole tensor's static scale
    t0 = time.perf_counter()
    if "w4a4" in wl.modes:
        ac, asc = oracle.quantize_mxfp4(a32)
        o44, _ = oracle.gemm_w4a4(ac, asc, wc, ws, K)
        what = "MXFP4 quantization + float64 W4A4 GEMM"
    else:
        o48, _ = oracle.gemm_w4a8(oracle.quantize_fp8(a32, inv_s), s_a, wc, ws, K)
        what = "FP8 quantization + float64 W4A8 GEMM"
    t_head = time.perf_counter() - t0
    res = {"value": round(2.0 * rows * N * K / t_head / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle", "seconds": round(t_head, 3),
           "sample": f"first {rows} of {wl.M} activation rows of {wl.name}: oracle {what} (with its "
                     f"tolerance sums), weights quantized beforehand; the full workload is extrapolated at "
                     f"{round(t_head * wl.M / rows, 1)} s"}
    if "w4a8" in wl.modes and "bf16" in wl.modes:
        t1 = time.perf_counter()
        o48, _ = oracle.gemm_w4a8(oracle.quantize_fp8(a32, inv_s), s_a, wc, ws, K)
        ref, _ = oracle.gemm_bf16(a_bits, w_bits)
        rb = oracle.gemm.to_bf16(ref)
        d44 = oracle.sqnr_db(rb, oracle.gemm.to_bf16(o44))[2]
        d48 = oracle.sqnr_db(rb, oracle.gemm.to_bf16(o48))[2]
        res["chain_seconds"] = round(t_head + time.perf_counter() - t1, 3)
        st.fns["mxq_quantize"](0)
        st.fns["mxq_gemm_w4a4"](0)
        st.fns["mxq_quantize_fp8"](0)
        st.fns["mxq_gemm_w4a8"](0)
        st.fns["mxq_gemm_bf16"](0)
        g44 = mxq.sqnr(st.ref[:rows], st.o44[:rows])[2].item()
        g48 = mxq.sqnr(st.ref[:rows], st.o48[:rows])[2].item()
        res["sqnr_db_sample_rows"] = {"oracle": {"w4a4": round(d44, 4), "w4a8": round(d48, 4)},
                                      "gpu": {"w4a4": round(g44, 4), "w4a8": round(g48, 4)}}
    return res


def main_bench(args):
    import numpy as np
    import torch

    import mxfp4_microscaled_quantization_amd as mxq
    import workloads

    dev = torch.device("cuda")
    st = Step(mxq, workloads, torch, args.workload, dev)
    wl = st.wl
    samples, wall, step_ms = time_steps(torch, st, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    kinfo = {label: _kinfo(label, samples[label], wl, args.workload) for label in st.seq}
    head = "mxq_gemm_w4a4" if "w4a4" in wl.modes else "mxq_gemm_w4a8"
    d = kinfo[head]
    res = {
        "metric": METRIC,
        "value": d["achieved"],
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4 x mxfp4 (w4a4), fp8 e4m3 x mxfp4 (w4a8); fp32 accumulate, bf16 out",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: A {wl.M}x{wl.K} bf16 ({wl.act}), W {wl.N}x{wl.K} bf16 "
                               f"N(0,{wl.w_std}); step: " + ", ".join(st.seq),
                   "M": wl.M, "K": wl.K, "N": wl.N, "parallelism": "single GPU"},
        "metric_values": {m: kinfo[f"mxq_gemm_{m}"]["achieved"] for m in ("w4a4", "w4a8") if m in wl.modes},
        "roofline": {"kernel": head, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
                     "unit": d["unit"], "frac": d["frac"], "traffic": d["traffic"]},
        "kernels": kinfo,
        "event_step_ms": round(step_ms, 4),
        "device": torch.cuda.get_device_name(0),
    }
    if "bf16" in wl.modes:
        torch.cuda.synchronize()
        res["sqnr_db"] = {"w4a4": round(float(st.r44[2].item()), 4), "w4a8": round(float(st.r48[2].item()), 4)}
    if not args.no_extras:
        if "bf16" in wl.modes:
            extras(mxq, torch, st, res, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(mxq, torch, st, min(args.cpu_rows, wl.M))
    if not args.no_extras and not args.no_configs and args.workload == DEFAULT_WORKLOAD:
        del st
        torch.cuda.empty_cache()
        res["configs"] = configs_section(mxq, workloads, torch, dev, args.config_reps)
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------- rocprofv3 summaries

def _read_csvs(d, suffix):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _short_name(name):
    """Kernel name without namespaces or argument list."""
    return re.sub(r"\(.*$", "", name.replace("(anonymous namespace)::", "").replace("mxq::", ""))


def _is_mxq(name):
    return "mxq::" in name


def _step_dispatches(events, wl, steps):
    """The last `steps` steps' dispatches of the library's kernels, labelled by position:
    events are (dispatch id, kernel name, payload) of every library kernel, in order."""
    per_step = []
    for label, n in step_kernels(wl):
        per_step += [label] * n
    need = steps * len(per_step)
    lib = [e for e in events if _is_mxq(e[1])]
    if len(lib) < need:
        raise ValueError(f"found {len(lib)} library dispatches, need {need}")
    tail = lib[-need:]
    out = {}
    for i, e in enumerate(tail):
        out.setdefault(per_step[i % len(per_step)], []).append(e)
    return out


def _pmc_dispatches(d, wl, steps):
    rows = _read_csvs(d, "counter_collection.csv")
    per = {}
    for r in rows:
        did = int(_col(r, "Dispatch_Id", "Correlation_Id"))
        e = per.setdefault(did, {"name": _col(r, "Kernel_Name"), "ctr": {}, "dur": None})
        name = _col(r, "Counter_Name")
        e["ctr"][name] = e["ctr"].get(name, 0.0) + float(_col(r, "Counter_Value"))
        if r.get("End_Timestamp"):
            e["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    ev = sorted((did, e["name"], e) for did, e in per.items())
    return _step_dispatches(ev, wl, steps)


def _copy_kib(d, counter):
    import numpy as np
    vals = [float(_col(r, "Counter_Value")) for r in _read_csvs(d, "counter_collection.csv")
            if _col(r, "Counter_Name") == counter and "copy" in _col(r, "Kernel_Name").lower()]
    return float(np.mean(vals))


def write_pmc_summaries(args, wl, steps):
    """HBM traffic per launch from two counter runs (FETCH_SIZE, then WRITE_SIZE; --input
    FETCH_DIR,WRITE_DIR), each scaled by what the same counter reads for a 1 GiB device
    copy (--copy-input COPY_FETCH_DIR,COPY_WRITE_DIR); one file per step kernel,
    profiles/pmc_<kernel>_<workload>.txt (--out is the directory)."""
    import numpy as np
    dirs = args.input.split(",")
    cdirs = args.copy_input.split(",")
    runs = {c: _pmc_dispatches(d, wl, steps) for c, d in zip(("FETCH_SIZE", "WRITE_SIZE"), dirs)}
    gib_kib = (1 << 30) / 1024.0
    scale = {c: gib_kib / _copy_kib(d, c) for c, d in zip(("FETCH_SIZE", "WRITE_SIZE"), cdirs)}
    cmds = args.command.split(" ;; ")
    done = set()
    for label, _ in step_kernels(wl):
        key = "mxq_sqnr" if label.startswith("mxq_sqnr") else label
        if key in done:
            continue
        done.add(key)
        kib = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            evs = runs[c][label]
            evs = evs[0::2] if label.startswith("mxq_sqnr") else evs
            kib[c] = (float(np.mean([e[2]["ctr"].get(c, 0.0) for e in evs])), len(evs))
        hbm = sum(kib[c][0] * 1024 * scale[c] for c in kib)
        alg = algorithmic_bytes(wl, label)
        kname = _short_name(runs["FETCH_SIZE"][label][0][1])
        text = "\n".join([
            f"# HBM traffic per launch: {key}, workload {args.workload}, MI355X (gfx950)",
            *[f"# command: {c}" for c in cmds],
            f"kernel: {kname}",
            f"source_sha256_16: {_src_hash(*SRC_OF[label])}",
            f"FETCH_SIZE_KiB_mean: {kib['FETCH_SIZE'][0]:.1f}   (launches: {kib['FETCH_SIZE'][1]})",
            f"WRITE_SIZE_KiB_mean: {kib['WRITE_SIZE'][0]:.1f}",
            f"scale_factors (1 GiB device copy): fetch x{scale['FETCH_SIZE']:.4f}, write x{scale['WRITE_SIZE']:.4f}",
            f"hbm_bytes_per_launch: {hbm:.4e}",
            f"algorithmic_bytes_per_launch: {alg:.4e}",
            f"traffic_over_algorithmic: {hbm / alg:.3f}", ""])
        path = os.path.join(args.out or ".", f"pmc_{key}_{args.workload}.txt")
        with open(path, "w") as f:
            f.write(text)
        print(text, end="")


def summarize(args):
    import numpy as np
    import workloads
    wl = workloads.WORKLOADS[args.workload]
    steps = int(re.search(r"--steps (\d+)", args.command).group(1)) if "--steps" in args.command else 5
    work = work_table(wl)
    lines = []
    if args.summarize == "trace":
        rows = _read_csvs(args.input, "kernel_trace.csv")
        ev = []
        for r in rows:
            ev.append((int(_col(r, "Dispatch_Id", "Correlation_Id")), _col(r, "Kernel_Name"),
                       (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3))
        ev.sort()
        by = _step_dispatches(ev, wl, steps)
        lines.append(f"# Kernel durations, workload {args.workload} ({wl.M}x{wl.K} @ {wl.K}x{wl.N}), MI355X (gfx950)")
        lines.append(f"# command: {args.command}")
        lines.append(f"# the last {steps} steps' launches, matched to the step's kernel order")
        lines.append(f"# {'kernel':24s} {'launches':>8s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}   rate   kernel name")
        for label, _ in step_kernels(wl):
            evs = by[label]
            if label.startswith("mxq_sqnr"):
                evs = evs[0::2]                           # the partial-sum kernel (the final pass is ~4 us)
            us = np.array([e[2] for e in evs])
            amount, unit, peak, _ = work[label]
            rate = _rate(amount, unit, us.mean() / 1e3)
            kname = _short_name(evs[0][1])
            lines.append(f"{label:26s} {len(us):8d} {us.mean():9.1f} {us.min():9.1f} {us.max():9.1f}   "
                         f"{rate:8.1f} {unit} ({rate / peak:.3f} of peak)   {kname}")
    elif args.summarize == "pmc":
        write_pmc_summaries(args, wl, steps)
        return
    elif args.summarize == "waves":
        # where the step kernels' waves spend their time: SQ wave-cycle counters of one
        # --pmc run, as fractions of the waves' lifetime (SQ_WAVE_CYCLES, the same units)
        by = _pmc_dispatches(args.input, wl, steps)
        lines.append(f"# Wave time breakdown per kernel, workload {args.workload}, MI355X (gfx950)")
        lines.append(f"# command: {args.command}")
        lines.append("# fractions of SQ_WAVE_CYCLES: wait = SQ_WAIT_ANY (s_waitcnt and barrier waits), "
                     "issue_wait = SQ_WAIT_INST_ANY (waiting to issue), active = SQ_ACTIVE_INST_ANY, "
                     "lds / vmem = SQ_ACTIVE_INST_LDS / _VMEM; lds_conflict = SQ_LDS_BANK_CONFLICT / "
                     "SQ_LDS_IDX_ACTIVE")
        for label, _ in step_kernels(wl):
            evs = by[label][0::2] if label.startswith("mxq_sqnr") else by[label]
            tot = lambda c: float(np.sum([e[2]["ctr"].get(c, 0.0) for e in evs]))
            wc = max(tot("SQ_WAVE_CYCLES"), 1.0)
            idx = max(tot("SQ_LDS_IDX_ACTIVE"), 1.0)
            lines.append(f"{label:26s} launches {len(evs):3d} wait {tot('SQ_WAIT_ANY') / wc:.3f} "
                         f"issue_wait {tot('SQ_WAIT_INST_ANY') / wc:.3f} active {tot('SQ_ACTIVE_INST_ANY') / wc:.3f} "
                         f"lds {tot('SQ_ACTIVE_INST_LDS') / wc:.3f} vmem {tot('SQ_ACTIVE_INST_VMEM') / wc:.3f} "
                         f"lds_conflict {tot('SQ_LDS_BANK_CONFLICT') / idx:.3f}")
    elif args.summarize == "stats":
        # every library kernel of the run (step, MFMA ceilings and the follow-on rows), one
        # line per kernel and launch grid (a grid stands for one shape), heaviest first
        groups = {}
        for r in _read_csvs(args.input, "kernel_trace.csv"):
            name = _col(r, "Kernel_Name")
            if not _is_mxq(name):
                continue
            key = (_short_name(name), int(_col(r, "Grid_Size_X")) // int(_col(r, "Workgroup_Size_X")))
            groups.setdefault(key, []).append((int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3)
        lines.append(f"# Every library kernel of one bench.py run on workload {args.workload} "
                     f"({wl.M}x{wl.K} @ {wl.K}x{wl.N}), MI355X (gfx950)")
        lines.append(f"# command: {args.command}")
        lines.append("# durations over all launches with that grid (warm-up launches included)")
        lines.append(f"# {'calls':>6s} {'workgroups':>10s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}   kernel")
        for (kname, wgs), us in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            u = np.array(us)
            lines.append(f"{len(u):8d} {wgs:10d} {u.mean():10.1f} {u.min():10.1f} {u.max():10.1f}   {kname}")
    else:
        by = _pmc_dispatches(args.input, wl, steps)
        if True:
            lines.append(f"# Matrix-core busy fraction and clock per kernel, workload {args.workload}, MI355X (gfx950)")
            lines.append(f"# command: {args.command}")
            lines.append("# clock = GRBM_GUI_ACTIVE / 8 XCDs / kernel duration; "
                         "mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8)")
            for label, _ in step_kernels(wl):
                evs = by[label][0::2] if label.startswith("mxq_sqnr") else by[label]
                gui = np.array([e[2]["ctr"].get("GRBM_GUI_ACTIVE", 0.0) for e in evs])
                busy = np.array([e[2]["ctr"].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for e in evs])
                dur = np.array([e[2]["dur"] or math.nan for e in evs])
                clock = gui / 8 / (dur * 1e3)
                frac = busy / (1024 * gui / 8)
                lines.append(f"{label:26s} launches {len(evs):3d} avg_us {np.nanmean(dur):9.1f} clock_GHz "
                             f"{np.nanmean(clock):5.2f} mfma_busy {np.mean(frac):.3f}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, end="")


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    main_bench(args)


if __name__ == "__main__":
    main()
