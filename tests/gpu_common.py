"""Helpers shared by the GPU parity tests (test side only)."""
import sys

import numpy as np
import torch

from helpers import bf16_bits

CANARY = 0xA5
GUARD = 4096


def say(*a):
    """Name the case on stdout before a GPU step (flushed, so a fault still
    leaves the case in the log)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy().view(np.uint8).reshape(-1)


def canary_buffer(n: int, device="cuda"):
    """A canary-filled byte buffer with a guard band; returns (view, whole)."""
    whole = torch.full((n + GUARD,), CANARY, dtype=torch.uint8, device=device)
    return whole[:n], whole


def guard_intact(whole: torch.Tensor, n: int) -> bool:
    return bool(torch.all(whole[n:] == CANARY).item())


def g_of(x: torch.Tensor) -> torch.Tensor:
    """fp32 encode scale 2688 / amax(x) (1 for an all-zero tensor), on x's device."""
    if x.numel() == 0:
        return torch.ones(1, dtype=torch.float32, device=x.device)
    a = x.float().abs().amax()
    return torch.where(a > 0, 2688.0 / a, torch.ones_like(a)).reshape(1)


def to_bits(x: torch.Tensor) -> np.ndarray:
    return bf16_bits(x)
