"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only workload shapes and random-number recipes: none of the
quantization, GEMM or SQNR arithmetic lives here, so both the CPU oracle and the HIP
library can be fed from it without sharing any of the method's code.

The workloads stand in for the linear layers the pages measure on (FLUX.1-dev at
1024x768: 64x48 image tokens + 512 text tokens; batch 16; Wan2.2-14B 21x45x80 latent
tokens).  No model weights or datasets are used.  Weights are generated directly in the
N x K (nn.Linear) layout; with i.i.d. entries this is the same distribution as the
K x N matrix the shapes are quoted in.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class GemmShape:
    name: str
    M: int          # tokens (activation rows)
    K: int          # reduction length (multiple of 32)
    N: int          # output features (weight rows)
    modes: tuple    # subset of ("w4a4", "w4a8", "bf16")
    act: str        # "lognormal_channels" | "student_t" | "tiny_outliers"
    w_std: float


#: the five workloads (config 3 is two GEMMs); sizes are (M x K) @ (K x N)
WORKLOADS = {
    "tiny_w4a4": GemmShape("tiny_w4a4", 128, 256, 128, ("w4a4",), "tiny_outliers", 0.02),
    "flux_qkv_w4a4": GemmShape("flux_qkv_w4a4", 3584, 3072, 9216, ("w4a4",),
                               "lognormal_channels", 0.02),
    "flux_ffn_up_w4a4": GemmShape("flux_ffn_up_w4a4", 57344, 3072, 12288, ("w4a4",),
                                  "lognormal_channels", 0.02),
    "flux_ffn_down_w4a4": GemmShape("flux_ffn_down_w4a4", 57344, 12288, 3072, ("w4a4",),
                                    "lognormal_channels", 0.02),
    "wan_ffn_up_w4a8": GemmShape("wan_ffn_up_w4a8", 75600, 5120, 13824, ("w4a8",),
                                 "lognormal_channels", 0.015),
    "wan_ffn_down_sqnr": GemmShape("wan_ffn_down_sqnr", 75600, 13824, 5120,
                                   ("w4a4", "w4a8", "bf16"), "student_t", 0.015),
}

_TENSOR_ID = {"channel_scale": 0, "act": 1, "weight": 2, "act_aux": 3}


def _seed(seed: int, name: str, tensor: str) -> int:
    """Stable 63-bit seed per (seed, workload, tensor)."""
    ss = np.random.SeedSequence([seed, sum(ord(c) * 131 ** i for i, c in enumerate(name)) % (2 ** 31),
                                 _TENSOR_ID[tensor]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(2 ** 63 - 1))


def _gen(device, seed: int, name: str, tensor: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name, tensor))
    return g


def tiny_inputs(seed: int = 0):
    """Tiny W4A4 workload, float32 on the host.

    A = 128 x 256 ~ N(0, 1) with a Bernoulli(0.01) mask of entries multiplied by 20;
    W = 256 x 128 ~ N(0, 0.02) (K x N), returned transposed as N x K.
    Returns (A float32 [128, 256], W float32 [128, 256]).
    """
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((128, 256)).astype(np.float32)
    mask = rng.random((128, 256)) < 0.01
    a[mask] *= np.float32(20.0)
    w_kn = (rng.standard_normal((256, 128)) * 0.02).astype(np.float32)
    return a, np.ascontiguousarray(w_kn.T)


def activations(M: int, K: int, kind: str, seed: int = 0, name: str = "custom",
                device="cpu", dtype=torch.bfloat16, nu: float = 3.0) -> torch.Tensor:
    """Activation matrix [M, K] (rows = tokens, K contiguous).

    * "lognormal_channels": N(0, 1) * c_k with one c_k ~ LogNormal(0, 1) per K-channel
      (an outlier-channel activation model).
    * "normal": i.i.d. N(0, 1).
    * "student_t": i.i.d. Student-t with ``nu`` degrees of freedom (heavy tails),
      drawn as Z / sqrt(G / (nu/2)) with G ~ Gamma(nu/2, 1), so 2G ~ chi^2_nu.
    The float32 draw is rounded to ``dtype`` by torch (round to nearest even).
    """
    if kind == "normal":
        ga = _gen(device, seed, name, "act")
        x = torch.randn(M, K, generator=ga, device=device, dtype=torch.float32)
    elif kind == "lognormal_channels":
        gc = _gen(device, seed, name, "channel_scale")
        c = torch.exp(torch.randn(K, generator=gc, device=device, dtype=torch.float32))
        ga = _gen(device, seed, name, "act")
        x = torch.randn(M, K, generator=ga, device=device, dtype=torch.float32)
        x.mul_(c)
    elif kind == "student_t":
        ga = _gen(device, seed, name, "act")
        x = torch.randn(M, K, generator=ga, device=device, dtype=torch.float32)
        gg = _gen(device, seed, name, "act_aux")
        alpha = torch.full((M, K), nu / 2.0, device=device, dtype=torch.float32)
        g = torch._standard_gamma(alpha, generator=gg)
        del alpha
        g.div_(nu / 2.0).sqrt_()
        x.div_(g)
        del g
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    return x.to(dtype) if dtype != torch.float32 else x


def weights(N: int, K: int, std: float, seed: int = 0, name: str = "custom",
            device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """Weight matrix [N, K] ~ N(0, std), rounded to ``dtype`` by torch."""
    g = _gen(device, seed, name, "weight")
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32).mul_(std)
    return w.to(dtype) if dtype != torch.float32 else w


def workload_inputs(name: str, seed: int = 0, device="cpu",
                    M: Optional[int] = None):
    """(A, W) for a named workload as bf16 tensors on ``device``.

    ``M`` overrides the token count (for reduced-size parity runs of the same recipe).
    """
    w = WORKLOADS[name]
    m = w.M if M is None else M
    a = activations(m, w.K, w.act, seed=seed, name=name, device=device)
    wt = weights(w.N, w.K, w.w_std, seed=seed, name=name, device=device)
    return a, wt


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 view of a bf16 tensor, copied to host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
