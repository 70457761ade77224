"""Small host-side helpers for the GPU parity tests (no method arithmetic here)."""

import numpy as np
import torch


def to_np_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def to_np_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_from_bits(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a bf16 is the high half of one)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def u8_to_gpu(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a fault can be attributed."""
    print(f"[gpu case] {msg}", flush=True)
