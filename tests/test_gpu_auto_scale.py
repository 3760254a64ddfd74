"""GPU parity of nvfp4_quant_grouped_auto (NVFP4 with encode scales from the
data in the same call) against the oracle's quantize_auto: ragged and
strided entries, gate/up pairs sharing a scale slot, zero and empty entries,
the full Qwen3-235B-A22B-shaped gate_up launch (sampled experts), capped
grids, repeated calls (the accumulators start from zero every call) and
graph replay.  Payload, scales, encode scales and amax byte for byte.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from helpers import bf16_bits
from gpu_common import canary_buffer, guard_intact, say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _experts(shapes, seed, scales=None):
    gen = torch.Generator().manual_seed(seed)
    out = []
    for k, (r, c) in enumerate(shapes):
        s = 1.0 if scales is None else scales[k]
        out.append((torch.randn(r, c, generator=gen) * s).to(torch.bfloat16))
    return out


def run_and_check(orc, layout, xs_cpu, slots=None, xs_dev=None, cols=None):
    xs = [x.to(DEV) for x in xs_cpu] if xs_dev is None else xs_dev
    cols = xs[0].shape[1] if cols is None else cols
    n_slots = len(xs) if slots is None else max(slots) + 1
    pays, scs = [], []
    wholes = []
    for x in xs:
        p, pw = canary_buffer(x.shape[0] * cols // 2)
        nb = mxq.scale_bytes(x.shape[0], cols, mxq.NVFP4, layout)
        s, sw = canary_buffer(nb)
        pays.append(p.view(x.shape[0], cols // 2))
        scs.append(s)
        wholes.append((pw, x.shape[0] * cols // 2, sw, nb))
    g = torch.full((n_slots + 8,), float("nan"), dtype=torch.float32, device=DEV)
    am = torch.full((n_slots + 8,), float("nan"), dtype=torch.float32, device=DEV)
    srcs = [x[:, :cols] for x in xs]
    mxq.nvfp4_quant_grouped_auto(layout, srcs, slots, pays, scs, g[:n_slots], am[:n_slots])
    torch.cuda.synchronize()
    for pw, n1, sw, n2 in wholes:
        assert guard_intact(pw, n1) and guard_intact(sw, n2)
    assert torch.all(torch.isnan(g[n_slots:])).item() and torch.all(torch.isnan(am[n_slots:])).item()
    op, os_, og, oa = orc.quantize_auto(layout, [bf16_bits(x) for x in xs_cpu], slots, cols)
    assert np.array_equal(am[:n_slots].cpu().numpy(), oa)
    assert np.array_equal(g[:n_slots].cpu().numpy(), og)
    for i in range(len(xs)):
        assert np.array_equal(u8(pays[i]), op[i].ravel()), i
        assert np.array_equal(u8(scs[i]), os_[i]), i
    return g[:n_slots], am[:n_slots]


@pytest.mark.parametrize("layout", [0, 1])
def test_auto_ragged_entries(orc, layout):
    shapes = [(1, 528), (37, 528), (128, 528), (129, 528), (300, 528)]
    xs = _experts(shapes, seed=1, scales=[1e-3, 1.0, 50.0, 1e4, 0.2])
    say("auto ragged, layout", layout)
    run_and_check(orc, layout, xs)


@pytest.mark.parametrize("layout", [0, 1])
def test_auto_strided_source(orc, layout):
    xs = _experts([(64, 1056), (70, 1056)], seed=2, scales=[3.0, 0.5])
    xs[0][:, 1024:] = 1e6  # past the quantized columns: must not reach the amax
    say("auto strided, layout", layout)
    run_and_check(orc, layout, xs, cols=1024)


@pytest.mark.parametrize("layout", [0, 1])
def test_auto_shared_gate_up_slots(orc, layout):
    shapes = [(96, 256)] * 8
    xs = _experts(shapes, seed=3, scales=[1.0, 4.0, 0.01, 0.02, 7.0, 7.0, 1e3, 1e-2])
    say("auto shared slots, layout", layout)
    run_and_check(orc, layout, xs, slots=[0, 0, 1, 1, 2, 2, 3, 3])
    run_and_check(orc, layout, xs, slots=[3, 0, 0, 1, 2, 0, 1, 3])


def test_auto_zero_and_empty(orc):
    xs = _experts([(32, 64), (0, 64), (40, 64)], seed=4)
    xs[2].zero_()
    say("auto zero and empty")
    g, am = run_and_check(orc, mxq.SWIZZLED, xs)
    assert g[1].item() == 1.0 and am[1].item() == 0.0
    assert g[2].item() == 1.0 and am[2].item() == 0.0
    # a slot with no entry at all still gets amax 0 and g 1
    g, am = run_and_check(orc, mxq.LINEAR, [xs[0]], slots=[1])
    assert g[0].item() == 1.0 and am[0].item() == 0.0


def test_auto_repeated_calls_restart_from_zero(orc):
    big = _experts([(64, 512)] * 3, seed=5, scales=[100.0] * 3)
    small = _experts([(64, 512)] * 3, seed=6, scales=[0.01] * 3)
    xs_big = [x.to(DEV) for x in big]
    xs_small = [x.to(DEV) for x in small]
    say("auto repeated calls")
    call_b = mxq.GroupedAutoCall(mxq.SWIZZLED, xs_big)
    call_s = mxq.GroupedAutoCall(mxq.SWIZZLED, xs_small, g_out=call_b.g, amax_out=call_b.amax)
    for _ in range(2):
        call_b()
        call_s()  # same accumulators: a stale amax from call_b would show
    torch.cuda.synchronize()
    op, os_, og, oa = orc.quantize_auto(mxq.SWIZZLED, [bf16_bits(x) for x in small])
    assert np.array_equal(call_s.amax.cpu().numpy(), oa)
    assert np.array_equal(call_s.g.cpu().numpy(), og)
    for i in range(3):
        assert np.array_equal(u8(call_s.payloads[i]), op[i].ravel())
        assert np.array_equal(u8(call_s.scales[i]), os_[i])


@pytest.mark.parametrize("layout", [0, 1])
def test_auto_grid_invariance(orc, layout):
    xs = _experts([(129, 1024), (64, 1024), (300, 1024)], seed=7, scales=[1.0, 30.0, 0.3])
    try:
        for cap in (1, 5):
            mxq.set_max_workgroups(cap)
            say("auto grid cap", cap, "layout", layout)
            run_and_check(orc, layout, xs, slots=[0, 1, 0])
    finally:
        mxq.set_max_workgroups(0)


def test_auto_qwen3_235b_gate_up_launch(orc):
    """One full launch: 16 experts bf16 [3072,4096]; every encode scale and
    amax exact; two experts compared byte for byte in full."""
    E = 16
    r, c = workloads.QWEN3_235B_A22B["gate_up"]
    stack = workloads.expert_stack(E, r, c, std=0.015, seed=5000, device=DEV)
    say("auto Qwen3-235B gate_up launch")
    call = mxq.GroupedAutoCall(mxq.SWIZZLED, [stack[i] for i in range(E)])
    pays, scs, g, am = call()
    torch.cuda.synchronize()
    want_am = stack.float().abs().amax(dim=(1, 2)).cpu().numpy()
    assert np.array_equal(am.cpu().numpy(), want_am)
    assert np.array_equal(g.cpu().numpy(),
                          np.array([orc.nvfp4_encode_scale(a) for a in want_am], np.float32))
    for i in (0, 11):
        p, s = orc.quantize(orc.NVFP4, orc.SWIZZLED, bf16_bits(stack[i]), g=float(g[i]))
        assert np.array_equal(u8(pays[i]), p.ravel())
        assert np.array_equal(u8(scs[i]), s)


def test_auto_graph_replay(orc):
    xs_cpu = _experts([(64, 256), (100, 256)], seed=8, scales=[2.0, 0.5])
    xs = [x.to(DEV) for x in xs_cpu]
    call = mxq.GroupedAutoCall(mxq.LINEAR, xs, slots=[0, 0])
    call()
    torch.cuda.synchronize()
    want = [u8(p).copy() for p in call.payloads] + [call.g.cpu().numpy().copy()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    say("auto graph capture")
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            call()
    for k in range(3):
        for p in call.payloads:
            p.fill_(0)
        call.g.fill_(-1.0)
        call.amax.fill_(-1.0)  # garbage in the accumulator: the graph must zero it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [u8(p) for p in call.payloads] + [call.g.cpu().numpy()]
        for a, b in zip(got, want):
            assert np.array_equal(a, b), k
