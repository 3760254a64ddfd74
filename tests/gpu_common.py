"""Helpers shared by the GPU parity tests (test side only)."""
import os
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


# Host threads for the oracle: the machine's CPU share for one GPU, at most 16.
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))


def par_map(fn, items):
    """fn over items on HOST_THREADS threads (the oracle's C calls release the
    GIL), results in order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(HOST_THREADS) as pool:
        return list(pool.map(fn, items))


def par_quantize(orc, fmt, layout, X, g=1.0):
    """The oracle's quantization of the bf16 bits X [rows, cols], in chunks of
    a multiple of 128 rows on host threads.  A swizzled scale matrix is whole
    128-row bands in row order, so the chunks' scale buffers concatenate to
    the whole tensor's (only the last chunk can hold padding rows)."""
    rows = X.shape[0]
    step = max(128, -(-rows // (4 * HOST_THREADS * 128)) * 128)
    parts = par_map(lambda r0: orc.quantize(fmt, layout, X[r0:r0 + step], g=g),
                    range(0, rows, step))
    if not parts:
        return orc.quantize(fmt, layout, X, g=g)
    return (np.concatenate([p for p, _ in parts]), np.concatenate([s for _, s in parts]))
