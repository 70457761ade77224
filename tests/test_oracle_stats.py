"""Statistical sanity of the oracle (CPU only; a cross-check, not a parity pin).

"Exp 2026-08-22 W4A4 Reference Model", section on error decomposition: with weights
and activations quantized independently, their output errors add in quadrature.  In
noise-power terms: N_both / S ~= N_A / S + N_W / S, i.e.
10^(-SQNR_both/10) ~= 10^(-SQNR_A/10) + 10^(-SQNR_W/10).
"""

import numpy as np
import torch

import oracle
import workloads


def test_weight_and_activation_errors_add_in_quadrature():
    a = workloads.activations(512, 1024, "student_t", seed=0, name="stats", dtype=torch.float32)
    w = workloads.weights(256, 1024, 0.015, seed=0, name="stats", dtype=torch.float32)
    a, w = a.double().numpy(), w.double().numpy()
    ca, sa = oracle.quantize_mxfp4(a)
    cw, sw = oracle.quantize_mxfp4(w)
    qa = oracle.dequantize_mxfp4(ca, sa, 1024)
    qw = oracle.dequantize_mxfp4(cw, sw, 1024)
    ref = a @ w.T
    s = np.sum(ref ** 2)
    r_a = np.sum((ref - qa @ w.T) ** 2) / s
    r_w = np.sum((ref - a @ qw.T) ** 2) / s
    r_b = np.sum((ref - qa @ qw.T) ** 2) / s
    assert 0.85 < r_b / (r_a + r_w) < 1.15, (r_a, r_w, r_b)
    # MXFP4 on both operands lands in the usual low-teens dB range for heavy tails
    assert 8.0 < -10 * np.log10(r_b) < 25.0
