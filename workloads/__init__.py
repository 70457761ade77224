"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only workload shapes and random-number recipes: none of the
quantization, GEMM or SQNR arithmetic lives here, so both the CPU oracle and the HIP
library can be fed from it without sharing any of the method's code.

Every tensor is drawn on the host with NumPy, row chunk by row chunk, each chunk from its
own stream default_rng(SeedSequence([seed, workload, tensor, chunk])), in float32, then
rounded to bf16 (round to nearest even): a seed names the same tensor on any device and
for any thread count.

The workloads stand in for the linear layers the pages measure on (FLUX.1-dev at
1024x768: 64x48 image tokens + 512 text tokens; batch 16; Wan2.2-14B 21x45x80 latent
tokens).  No model weights or datasets are used.  Weights are generated directly in the
N x K (nn.Linear) layout; with i.i.d. entries this is the same distribution as the
K x N matrix the shapes are quoted in.
"""

import functools
import os
import warnings
from concurrent.futures import ThreadPoolExecutor
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
ROWS_PER_CHUNK = 1024          # rows drawn from one random stream
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _name_id(name: str) -> int:
    return sum(ord(c) * 131 ** i for i, c in enumerate(name)) % (2 ** 31)


def _rng(seed: int, name: str, tensor: str, chunk: int) -> np.random.Generator:
    """One host stream per (seed, workload, tensor, row chunk):
    default_rng(SeedSequence([seed, workload id, tensor id, chunk]))."""
    return np.random.default_rng(np.random.SeedSequence([seed, _name_id(name), _TENSOR_ID[tensor], chunk]))


def _rows(M: int, K: int, draw) -> np.ndarray:
    """float32 [M, K] filled chunk by chunk: rows [c*ROWS_PER_CHUNK, ...) come from
    draw(c, rows) alone, so the result does not depend on the thread count."""
    out = np.empty((M, K), dtype=np.float32)
    chunks = range((M + ROWS_PER_CHUNK - 1) // ROWS_PER_CHUNK)

    def fill(c):
        r0 = c * ROWS_PER_CHUNK
        r1 = min(M, r0 + ROWS_PER_CHUNK)
        out[r0:r1] = draw(c, r1 - r0)

    if M * K < (1 << 22) or _THREADS == 1:
        for c in chunks:
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    return out


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even on the integer pattern (finite
    inputs): (u + 0x7FFF + ((u >> 16) & 1)) >> 16."""
    u = x.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _to_torch(x32: np.ndarray, device, dtype) -> torch.Tensor:
    if dtype == torch.float32:
        t = torch.from_numpy(x32)
    elif dtype == torch.bfloat16:
        t = torch.from_numpy(_bf16_bits(x32).view(np.int16)).view(torch.bfloat16)
    else:
        raise ValueError(f"unsupported dtype {dtype}")
    return t.to(device) if str(device) != "cpu" else t


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


def activations_f32(M: int, K: int, kind: str, seed: int = 0, name: str = "custom", nu: float = 3.0) -> np.ndarray:
    """Activation matrix [M, K] as float32 on the host (rows = tokens, K contiguous).

    * "lognormal_channels": N(0, 1) * c_k with one c_k ~ LogNormal(0, 1) per K-channel
      (an outlier-channel activation model); c comes from its own stream.
    * "normal": i.i.d. N(0, 1).
    * "student_t": i.i.d. Student-t with ``nu`` degrees of freedom (heavy tails), drawn
      as Z / sqrt(G / (nu/2)) with Z ~ N(0, 1), G ~ Gamma(nu/2, 1) (2G ~ chi^2_nu).
    """
    if kind == "normal":
        return _rows(M, K, lambda c, r: _rng(seed, name, "act", c).standard_normal((r, K), dtype=np.float32))
    if kind == "lognormal_channels":
        ch = np.exp(_rng(seed, name, "channel_scale", 0).standard_normal(K)).astype(np.float32)
        return _rows(M, K, lambda c, r: _rng(seed, name, "act", c).standard_normal((r, K), dtype=np.float32) * ch)
    if kind == "student_t":
        half = np.float32(nu / 2.0)

        def draw(c, r):
            g = _rng(seed, name, "act_aux", c).standard_gamma(nu / 2.0, (r, K), dtype=np.float32)
            z = _rng(seed, name, "act", c).standard_normal((r, K), dtype=np.float32)
            return z / np.sqrt(g / half)

        return _rows(M, K, draw)
    raise ValueError(f"unknown activation kind {kind!r}")


def activations(M: int, K: int, kind: str, seed: int = 0, name: str = "custom",
                device="cpu", dtype=torch.bfloat16, nu: float = 3.0) -> torch.Tensor:
    """``activations_f32`` rounded to ``dtype`` (bf16: round to nearest even) on ``device``.
    The draw is made on the host, so a seed gives the same tensor on every device."""
    return _to_torch(activations_f32(M, K, kind, seed, name, nu), device, dtype)


def weights(N: int, K: int, std: float, seed: int = 0, name: str = "custom",
            device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """Weight matrix [N, K] ~ N(0, std), drawn on the host, rounded to ``dtype``."""
    s = np.float32(std)
    w = _rows(N, K, lambda c, r: _rng(seed, name, "weight", c).standard_normal((r, K), dtype=np.float32) * s)
    return _to_torch(w, device, dtype)


@functools.lru_cache(maxsize=2)
def _workload_bits(name: str, seed: int, M: int):
    """Host bf16 bit patterns of a named workload's (A, W), kept for reuse: the full-size
    draws take seconds and several tests and the benchmark ask for the same ones."""
    w = WORKLOADS[name]
    a = _bf16_bits(activations_f32(M, w.K, w.act, seed=seed, name=name))
    s = np.float32(w.w_std)
    wt = _bf16_bits(_rows(w.N, w.K, lambda c, r: _rng(seed, name, "weight", c).standard_normal((r, w.K),
                                                                                            dtype=np.float32) * s))
    a.flags.writeable = False
    wt.flags.writeable = False
    return a, wt


def workload_inputs(name: str, seed: int = 0, device="cpu",
                    M: Optional[int] = None):
    """(A, W) for a named workload as bf16 tensors on ``device`` (fresh tensors; the host
    draw is cached).

    ``M`` overrides the token count (for reduced-size parity runs of the same recipe;
    the first M rows of the full workload's A, since rows are drawn chunk by chunk).
    """
    w = WORKLOADS[name]
    m = w.M if M is None else M
    a_bits, w_bits = _workload_bits(name, seed, m)

    def tensor(bits):
        with warnings.catch_warnings():      # read-only cache: the view is copied at once
            warnings.simplefilter("ignore", UserWarning)
            t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        return t.clone() if str(device) == "cpu" else t.to(device)

    return tensor(a_bits), tensor(w_bits)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 view of a bf16 tensor, copied to host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
