"""Seeded synthetic inputs for the quantization workloads.

This module holds no quantization arithmetic: it only draws bf16 tensors and
split sizes with the shapes, value distributions and structure of the MoE
workloads (expert weights, a routed token activation, the residual/RMSNorm
epilogue inputs).  The tests, the smoke check and the benchmark use it for
both the GPU path and the CPU oracle.

Recipes (every draw comes from a ``torch.Generator`` seeded as stated):
  * small grouped weights: 8 experts of bf16 [256, 512], values N(0,1) times a
    per-row log-normal(0,1) factor, each entry times 100 with probability 1e-3.
  * MoE layer weights (Qwen3-30B-A3B: gate_up [1536,2048], down [2048,768];
    Qwen3-235B-A22B: gate_up [3072,4096], down [4096,1536]): 128 experts per
    projection, N(0, std^2) (std 0.02 / 0.015), each entry times 50 with
    probability 1e-4; layer l of a model drawn from one generator seeded
    2000 + l (30B-A3B) or 5000 + l (235B-A22B).
  * routed activation: bf16 [8192, 7168] N(0,1) times a per-token
    log-normal(0, 0.5) factor; 256 experts, 10 of them forced empty, the other
    split sizes drawn multinomially (uniform routing) over the tokens.
  * epilogue inputs: x, residual ~ N(0,1) bf16 [T, 7168], gamma ~ N(1, 0.1^2).
"""
from __future__ import annotations

import torch

QWEN3_30B_A3B = {"gate_up": (1536, 2048), "down": (2048, 768)}
QWEN3_235B_A22B = {"gate_up": (3072, 4096), "down": (4096, 1536)}
N_EXPERTS = 128
GROUP = 16


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def small_grouped_experts(n_experts=8, rows=256, cols=512, seed=0, device="cpu"):
    """Row-scaled normal weights with rare x100 outliers, bf16."""
    g = _gen(seed)
    out = []
    for _ in range(n_experts):
        x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
        row_scale = torch.exp(torch.randn(rows, 1, generator=g, dtype=torch.float32))
        outlier = torch.rand(rows, cols, generator=g) < 1e-3
        x = x * row_scale
        x = torch.where(outlier, x * 100.0, x)
        out.append(x.to(torch.bfloat16).to(device))
    return out


def expert_stack(n, rows, cols, std, seed, device="cpu", outlier_p=1e-4, outlier_mul=50.0,
                 out=None, gen=None):
    """n same-shape expert weights as one bf16 [n, rows, cols] tensor.

    Drawn on `device` with a generator of that device (seeded `seed`, or
    `gen` when given), in float32, then rounded to bf16 (into `out` when
    given, so a stacking buffer is reused)."""
    g = _gen(seed, device) if gen is None else gen
    if out is None:
        out = torch.empty(n, rows, cols, dtype=torch.bfloat16, device=device)
    for i in range(n):
        x = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        m = torch.rand(rows, cols, generator=g, device=device) < outlier_p
        x = torch.where(m, x * outlier_mul, x)
        out[i].copy_(x)
    return out


def moe_layer(shapes, layer, base_seed, std, device="cpu", out=None):
    """One MoE layer's expert weights, {projection: bf16 [N_EXPERTS, rows,
    cols]} for the projections of `shapes` in order (gate_up, then down),
    all drawn from one generator seeded base_seed + layer on `device` (the
    Qwen3-235B-A22B layers use 5000 + l, std 0.015; the Qwen3-30B-A3B layers
    2000 + l, std 0.02).  `out`, a dict of the same shapes, is reused when
    given."""
    g = _gen(base_seed + layer, device)
    res = {}
    for p, (r, c) in shapes.items():
        res[p] = expert_stack(N_EXPERTS, r, c, std, None, device, out=None if out is None
                              else out[p], gen=g)
    return res


def routed_activation(T=8192, H=7168, n_experts=256, n_empty=10, seed=3000, device="cpu"):
    """Token activation plus per-expert split sizes (sum == T)."""
    g = _gen(seed)
    x = torch.randn(T, H, generator=g, dtype=torch.float32)
    x = x * torch.exp(0.5 * torch.randn(T, 1, generator=g, dtype=torch.float32))
    perm = torch.randperm(n_experts, generator=g)
    empty = set(perm[:n_empty].tolist())
    live = [e for e in range(n_experts) if e not in empty]
    picks = torch.multinomial(torch.ones(len(live)), T, replacement=True, generator=g)
    counts = torch.bincount(picks, minlength=len(live)).tolist()
    split = [0] * n_experts
    for e, c in zip(live, counts):
        split[e] = int(c)
    return x.to(torch.bfloat16).to(device), split


def epilogue_inputs(T, H=7168, seed=None, device="cpu"):
    """x, residual ~ N(0,1) [T, H]; gamma ~ N(1, 0.01) [H]; all bf16."""
    g = _gen(4000 + T if seed is None else seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    res = torch.randn(T, H, generator=g).to(torch.bfloat16)
    gamma = (1.0 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    return x.to(device), res.to(device), gamma.to(device)

