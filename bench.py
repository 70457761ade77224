"""Benchmark of the MXFP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic activations
already resident in HBM (weights are quantized once, offline, as in deployment; the
static FP8 scale is calibrated once, before timing):

  1. mxq_quantize       dynamic MXFP4 activations (bf16 -> codes + E8M0 scales)
  2. mxq_quantize_fp8   static FP8 E4M3 activations
  3. mxq_gemm_w4a4      MXFP4 x MXFP4 -> bf16
  4. mxq_gemm_w4a8      FP8 x MXFP4 -> bf16
  5. mxq_gemm_bf16      bf16 reference
  6. mxq_sqnr x 2       whole-output SQNR of W4A4 and W4A8 against the reference

Prints ONE JSON line.  `value` is the step's GEMM throughput (all GEMM FLOPs of the step
divided by the step time, TFLOP/s).  `roofline` describes the kernel that takes the most
time; `kernels` gives every kernel's achieved rate (from its mean time over the steps;
median, standard deviation and coefficient of variation beside it) against its own
roofline, all timed with HIP events on the stream the kernels run on.  `cpu_baseline` times the CPU oracle
on a bounded row sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
PEAK = {"hbm_GBps": 8000.0, "fp4_TFLOPs": 10100.0, "fp8_TFLOPs": 5000.0, "bf16_TFLOPs": 2500.0}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="wan_ffn_down_sqnr")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=6144, help="activation rows in the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of known size (for HBM counter scaling)")
    return p.parse_args()


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp4_microscaled_quantization_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_from_profile(kernel_key: str, src_hash: str):
    """HBM bytes per launch from a committed counter summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel_key}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != src_hash:
        return None
    return float(m_val.group(1))


def copy_calibration():
    import torch
    n = 1 << 30                       # 1 GiB read + 1 GiB written per launch
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 5}))


def cpu_baseline(name, rows, a_host_rows, w_bits):
    """The oracle as it stands, on `rows` activation rows of the workload (its static FP8
    scale is calibrated on the sample itself)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    wl_K = a_host_rows.shape[1]
    w_f32 = (w_bits.astype(np.uint32) << 16).view(np.float32)
    wc, ws = oracle.quantize_mxfp4(w_f32)                 # offline weight prep: not timed
    s_a, inv_s = oracle.fp8_static_scales(np.max(np.abs(a_host_rows)))
    t0 = time.perf_counter()
    ac, asc = oracle.quantize_mxfp4(a_host_rows)
    q8 = oracle.quantize_fp8(a_host_rows, inv_s)
    a_bits = (a_host_rows.view(np.uint32) >> 16).astype(np.uint16)
    ref, _ = oracle.gemm_bf16(a_bits, w_bits)
    o44, _ = oracle.gemm_w4a4(ac, asc, wc, ws, wl_K)
    o48, _ = oracle.gemm_w4a8(q8, s_a, wc, ws, wl_K)
    rb = oracle.gemm.to_bf16(ref)
    oracle.sqnr_db(rb, oracle.gemm.to_bf16(o44))
    oracle.sqnr_db(rb, oracle.gemm.to_bf16(o48))
    dt = time.perf_counter() - t0
    N = w_bits.shape[0]
    flops = 3 * 2.0 * rows * N * wl_K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{rows} activation rows of {name} through the whole oracle chain "
                      f"(MXFP4 + FP8 quantize, W4A4/W4A8/bf16 GEMMs in float64, 2x SQNR); "
                      f"weights quantized beforehand, untimed"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mxfp4_microscaled_quantization_amd as mxq
    import workloads

    if args.copy_calibration:
        copy_calibration()
        return

    wl = workloads.WORKLOADS[args.workload]
    M, K, N = wl.M, wl.K, wl.N
    dev = torch.device("cuda")

    # ---- inputs resident in HBM; offline weight prep and static calibration ----
    a, w = workloads.workload_inputs(args.workload, device=dev)
    wc, wsc = mxq.quantize(w)
    amax = float(mxq.absmax(a).item())
    s_a, inv_s = mxq.fp8_static_scales(amax)
    ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    asc = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    a8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    o44 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    o48 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws1 = torch.empty(mxq.sqnr_workspace_bytes(M * N) // 8, dtype=torch.float64, device=dev)
    ws2 = torch.empty_like(ws1)
    r44 = torch.empty(3, dtype=torch.float64, device=dev)
    r48 = torch.empty(3, dtype=torch.float64, device=dev)

    kernels = [
        ("mxq_quantize", lambda: mxq.quantize_into(a, ac, asc)),
        ("mxq_quantize_fp8", lambda: mxq.quantize_fp8(a, inv_s, out=a8)),
        ("mxq_gemm_w4a4", lambda: mxq.gemm_w4a4(ac, asc, wc, wsc, out=o44)),
        ("mxq_gemm_w4a8", lambda: mxq.gemm_w4a8(a8, s_a, wc, wsc, out=o48)),
        ("mxq_gemm_bf16", lambda: mxq.gemm_bf16(a, w, out=ref)),
        ("mxq_sqnr_w4a4", lambda: mxq.sqnr(ref, o44, workspace=ws1, out3=r44)),
        ("mxq_sqnr_w4a8", lambda: mxq.sqnr(ref, o48, workspace=ws2, out3=r48)),
    ]
    flop = 2.0 * M * N * K
    work = {  # algorithmic units per launch: (amount, unit, peak, bound)
        "mxq_quantize": (M * K * (2 + 0.5 + 1 / 32), "GB/s", PEAK["hbm_GBps"], "hbm"),
        "mxq_quantize_fp8": (M * K * 3.0, "GB/s", PEAK["hbm_GBps"], "hbm"),
        "mxq_gemm_w4a4": (flop, "TFLOP/s", PEAK["fp4_TFLOPs"], "mfma"),
        "mxq_gemm_w4a8": (flop, "TFLOP/s", PEAK["fp8_TFLOPs"], "mfma"),
        "mxq_gemm_bf16": (flop, "TFLOP/s", PEAK["bf16_TFLOPs"], "mfma"),
        "mxq_sqnr_w4a4": (M * N * 4.0, "GB/s", PEAK["hbm_GBps"], "hbm"),
        "mxq_sqnr_w4a8": (M * N * 4.0, "GB/s", PEAK["hbm_GBps"], "hbm"),
    }

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, (_, fn) in enumerate(kernels):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    samples = {name: np.array([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)])
               for i, (name, _) in enumerate(kernels)}
    per_kernel_ms = {name: float(np.mean(t)) for name, t in samples.items()}
    step_ms = float(np.mean([ev[s][0].elapsed_time(ev[s][-1]) for s in range(args.steps)]))
    ms_per_step = wall * 1e3 / args.steps

    src_keys = {"mxq_quantize": ("quantize.hip",), "mxq_quantize_fp8": ("quantize.hip",),
                "mxq_gemm_w4a4": ("gemm.hip",), "mxq_gemm_w4a8": ("gemm.hip",), "mxq_gemm_bf16": ("gemm.hip",),
                "mxq_sqnr_w4a4": ("sqnr.hip",), "mxq_sqnr_w4a8": ("sqnr.hip",)}
    kinfo = {}
    for name, ms in per_kernel_ms.items():
        amount, unit, peak, bound = work[name]
        rate = amount / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        prof_name = "mxq_sqnr" if name.startswith("mxq_sqnr") else name
        t = samples[name]
        kinfo[name] = {"ms": round(ms, 4), "median_ms": round(float(np.median(t)), 4),
                       "std_ms": round(float(np.std(t)), 4), "cv": round(float(np.std(t) / ms), 4),
                       "achieved": round(rate, 2), "unit": unit, "peak": peak,
                       "frac": round(rate / peak, 4), "bound": bound,
                       "traffic": _traffic_from_profile(f"{prof_name}_{args.workload}", _src_hash(*src_keys[name]))}
    dominant = max(per_kernel_ms, key=per_kernel_ms.get)
    d = kinfo[dominant]
    roofline = {"kernel": dominant, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
                "unit": d["unit"], "frac": d["frac"], "traffic": d["traffic"]}

    res = {
        "metric": "W4A4/W4A8 GEMM TFLOP/s (% of MXFP4/FP8 peak); quantize GB/s (% of HBM)",
        "value": round(3 * flop / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4,fp8,bf16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": f"{args.workload}: A {M}x{K} bf16 ({wl.act}), W {N}x{K} bf16 N(0,{wl.w_std}); "
                               "quantize MXFP4 + FP8, W4A4 + W4A8 + bf16 GEMMs, 2x SQNR",
                   "M": M, "K": K, "N": N, "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": kinfo,
        "event_step_ms": round(step_ms, 4),
        "sqnr_db": {"w4a4": round(float(r44[2].item()), 4), "w4a8": round(float(r48[2].item()), 4)},
        "device": torch.cuda.get_device_name(0),
    }

    def time_fn(fn, n=10):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ---- outside the timed step: the MFMA ceiling on the step's own operand bits. A
    # register-only loop of each GEMM's MFMA instruction on fragments gathered from its
    # operands (no memory traffic) gives what the matrix cores sustain on this data at the
    # clock the chip holds under it; each GEMM's fraction of that ceiling beside it ----
    waves = 4096
    sink = torch.empty(waves * 64, dtype=torch.float32, device=dev)
    ceiling = {"what": "register-only loop of the GEMM's MFMA instruction on fragments of the step's operands"}
    for name, mode, ops, iters in (("mxq_gemm_w4a4", "w4a4", (ac, asc, wc, wsc), 1500),
                                   ("mxq_gemm_w4a8", "w4a8", (a8, None, wc, wsc), 1000),
                                   ("mxq_gemm_bf16", "bf16", (a, None, w, None), 3000)):
        ms_c = time_fn(lambda: mxq.mfma_ceiling(mode, *ops, waves=waves, iters=iters, sink=sink), n=3)
        rate_c = waves * iters * 16 * mxq.MFMA_FLOP[mode] / (ms_c * 1e-3) / 1e12
        peak = work[name][2]
        ceiling[name] = {"achieved": round(rate_c, 2), "unit": "TFLOP/s", "peak": peak,
                         "frac_of_peak": round(rate_c / peak, 4),
                         "gemm_frac_of_ceiling": round(kinfo[name]["achieved"] / rate_c, 4)}
    res["mfma_ceiling"] = ceiling
    del sink

    # ---- the UOS scale rule (quantize rate, W4A4 SQNR on the same workload, both operands
    # quantized with UOS) ----
    ms_uos = time_fn(lambda: mxq.quantize_into(a, ac, asc, rule="uos"))
    wc_u, wsc_u = mxq.quantize(w, rule="uos")
    mxq.quantize_into(a, ac, asc, rule="uos")
    mxq.gemm_w4a4(ac, asc, wc_u, wsc_u, out=o44)
    r_u = mxq.sqnr(ref, o44, workspace=ws1)
    q_amount = work["mxq_quantize"][0]
    # block-Hadamard rotation + MXFP4 of both operands (weights offline), n = 64 and 256
    hada = {}
    for n in (64, 256):
        ms_h = time_fn(lambda: mxq.quantize_hadamard(a, n))
        rwc, rwsc = mxq.quantize_hadamard(w, n)
        rac, rasc = mxq.quantize_hadamard(a, n)
        mxq.gemm_w4a4(rac, rasc, rwc, rwsc, out=o44)
        r_h = mxq.sqnr(ref, o44, workspace=ws1)
        rate = q_amount / (ms_h * 1e-3) / 1e9
        hada[f"n{n}"] = {"mxq_quantize_hadamard": {"ms": round(ms_h, 4), "achieved": round(rate, 2), "unit": "GB/s",
                                                   "peak": PEAK["hbm_GBps"], "frac": round(rate / PEAK["hbm_GBps"], 4)},
                         "sqnr_db_w4a4": round(float(r_h[2].item()), 4)}
        del rwc, rwsc, rac, rasc
    # W4A4 with the activation quantization fused into the GEMM (bf16 activations in),
    # against the separate quantize + W4A4 of the timed step, and checked bit for bit
    o_f = torch.empty_like(o44)
    ms_f = time_fn(lambda: mxq.gemm_w4a4_fused(a, wc, wsc, out=o_f))
    mxq.quantize_into(a, ac, asc)
    mxq.gemm_w4a4(ac, asc, wc, wsc, out=o44)
    torch.cuda.synchronize()
    fused_same = bool(torch.equal(o_f.view(torch.int16), o44.view(torch.int16)))
    del o_f
    rate_f = flop / (ms_f * 1e-3) / 1e12
    fused = {"mxq_gemm_w4a4_fused": {"ms": round(ms_f, 4), "achieved": round(rate_f, 2), "unit": "TFLOP/s",
                                     "peak": PEAK["fp4_TFLOPs"], "frac": round(rate_f / PEAK["fp4_TFLOPs"], 4)},
             "quantize_plus_w4a4_ms": round(per_kernel_ms["mxq_quantize"] + per_kernel_ms["mxq_gemm_w4a4"], 4),
             "bit_identical_to_quantize_then_w4a4": fused_same}
    # MXFP4 -> bf16 dequantization (the QDQ step) of the activation codes, into a bf16 buffer
    mxq.quantize_into(a, ac, asc)
    y_dq = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ms_dq = time_fn(lambda: mxq.dequantize(ac, asc, K, out=y_dq))
    del y_dq
    dq_rate = M * K * (0.5 + 1 / 32 + 2) / (ms_dq * 1e-3) / 1e9
    dequant = {"mxq_dequantize": {"ms": round(ms_dq, 4), "achieved": round(dq_rate, 2), "unit": "GB/s",
                                  "peak": PEAK["hbm_GBps"], "frac": round(dq_rate / PEAK["hbm_GBps"], 4)}}
    res["next"] = {
        "fused_activation_quant": fused,
        "dequantize": dequant,
        "hadamard_rotation": hada,
        "uos_scale_rule": {
            "mxq_quantize_uos": {"ms": round(ms_uos, 4), "achieved": round(q_amount / (ms_uos * 1e-3) / 1e9, 2),
                                 "unit": "GB/s", "peak": PEAK["hbm_GBps"],
                                 "frac": round(q_amount / (ms_uos * 1e-3) / 1e9 / PEAK["hbm_GBps"], 4)},
            "sqnr_db_w4a4": {"ocp": round(float(r44[2].item()), 4), "uos": round(float(r_u[2].item()), 4)},
        }
    }

    if not args.no_cpu_baseline:
        rows = min(args.cpu_rows, M)
        a_rows = a[:rows]
        a_host = (a_rows.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        w_bits = w.view(torch.int16).cpu().numpy().view(np.uint16)
        del a, ac, asc, a8, o44, o48, ref
        res["cpu_baseline"] = cpu_baseline(args.workload, rows, a_host, w_bits)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
