"""Calls allocate no device memory.

Every entry point writes only caller buffers: after one warm-up call (which
loads the code objects), further calls of each form, prepacked so that the
binding allocates nothing either, leave the device's free memory and torch's
allocator statistics exactly where they were.
"""
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from gpu_common import g_of, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _calls():
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=16, rows=384, cols=1024,
                                                             seed=5)]
    gs = torch.cat([g_of(x) for x in xs])
    act, split = workloads.routed_activation(T=1024, H=2048, n_experts=64, n_empty=3, seed=6)
    act = act.to(DEV)
    ga = g_of(act)
    x, r, gm = workloads.epilogue_inputs(300, 2048, seed=9, device=DEV)
    calls = [mxq.GroupedCall(f, l, xs, global_scales=gs if f else None)
             for f in (0, 1) for l in (0, 1)]
    calls += [mxq.GroupedAutoCall(l, xs) for l in (0, 1)]
    calls += [mxq.SplitCall(m, act, split, l, ga if m == "nvfp4" else None)
              for m in ("nvfp4", "nvfp4_row_scaled", "mxfp8") for l in (0, 1)]
    calls += [mxq.FusedCall(x, r, gm, 1e-6, f, l, ga) for f in (0, 1) for l in (0, 1)]
    return calls


def test_calls_allocate_nothing():
    calls = _calls()
    for c in calls:  # warm-up: code objects load on first use
        c()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    stats0 = torch.cuda.memory_stats()
    say("no-allocation check over", len(calls), "prepacked calls")
    for _ in range(3):
        for c in calls:
            c()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    stats1 = torch.cuda.memory_stats()
    assert free1 == free0
    for key in ("allocation.all.allocated", "segment.all.allocated", "allocated_bytes.all.allocated"):
        assert stats1.get(key, 0) == stats0.get(key, 0), key
