"""The library keeps no per-call state: calls replay from HIP graphs, run on
several streams at once, and come from several host threads, with the bytes
of eager single-stream calls.

Graph replays run several times with eager work and synchronizations in
between, and every replay is checked (the graphs hold kernel nodes only).
"""
import threading

import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from helpers import bf16_bits
from gpu_common import CANARY, g_of, say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def raw(t):
    """Bytes of a tensor of any dtype (bf16 included), as numpy uint8."""
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph there."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            fn()
    torch.cuda.synchronize()
    return graph


def _replay_and_check(graph, outs, want):
    for rep in range(3):
        for t in outs:
            t.fill_(CANARY) if t.dtype == torch.uint8 else t.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w in zip(outs, want):
            assert np.array_equal(raw(t), w), rep


@pytest.mark.parametrize("mode", ["nvfp4", "nvfp4_row_scaled", "mxfp8"])
@pytest.mark.parametrize("layout", [0, 1])
def test_split_graph_replay(mode, layout):
    x_cpu, split = workloads.routed_activation(T=2048, H=1024, seed=7)
    x = x_cpu.to(DEV)
    g = g_of(x)
    call = mxq.SplitCall(mode, x, split, layout, g if mode == "nvfp4" else None)
    say("split graph", mode, layout)
    eager = [raw(t).copy() for t in call()]
    graph = _capture(call)
    _replay_and_check(graph, list(call()), eager)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("T", [3, 3000])
def test_fused_graph_replay(fmt, T):
    x, r, gm = (t.to(DEV) for t in workloads.epilogue_inputs(T, 2048, seed=T))
    gs = torch.tensor([50.0], dtype=torch.float32, device=DEV)
    call = mxq.FusedCall(x, r, gm, 1e-6, fmt, mxq.SWIZZLED, gs)
    say("fused graph", fmt, T)
    eager = [raw(t).copy() for t in call()]
    graph = _capture(call)
    _replay_and_check(graph, list(call.out), eager)


def test_calls_on_two_streams_at_once():
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=16, rows=512, cols=2048,
                                                             seed=3)]
    gs = torch.cat([g_of(x) for x in xs])
    say("two streams")
    want = [u8(t).copy() for t in
            sum(mxq.mx_quant_grouped(mxq.NVFP4, mxq.SWIZZLED, xs, global_scales=gs), [])]
    calls = [mxq.GroupedCall(mxq.NVFP4, mxq.SWIZZLED, xs[k::2], global_scales=gs[k::2].contiguous())
             for k in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(5):
        for c, s in zip(calls, streams):
            with torch.cuda.stream(s):
                c()
    torch.cuda.synchronize()
    pays = [None] * 16
    scs = [None] * 16
    for k, c in enumerate(calls):
        for j, (p, sc) in enumerate(zip(c.payloads, c.scales)):
            pays[k + 2 * j], scs[k + 2 * j] = p, sc
    got = [u8(t) for t in pays + scs]
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_calls_from_several_host_threads(orc):
    """Each host thread drives its own stream; ctypes releases the GIL during
    the library call, so the calls overlap in the library."""
    n = 4
    inputs = [workloads.epilogue_inputs(64, 1024, seed=100 + k, device=DEV) for k in range(n)]
    gs = torch.tensor([80.0], dtype=torch.float32, device=DEV)
    calls = [mxq.FusedCall(*inputs[k], 1e-6, k % 2, mxq.SWIZZLED, gs) for k in range(n)]
    streams = [torch.cuda.Stream() for _ in range(n)]
    errors = []
    torch.cuda.synchronize()
    say("host threads")

    def work(k):
        try:
            with torch.cuda.stream(streams[k]):
                for _ in range(20):
                    calls[k]()
            streams[k].synchronize()
        except Exception as e:  # reported below
            errors.append(e)
    threads = [threading.Thread(target=work, args=(k,)) for k in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k in range(n):
        x, r, gm = (t.cpu() for t in inputs[k])
        oro, ono = orc.add_rmsnorm(bf16_bits(x), bf16_bits(r), bf16_bits(gm), 1e-6)
        ro, no_gpu, p, s = calls[k].out
        assert np.array_equal(bf16_bits(ro), oro)
        d = np.abs(bf16_bits(no_gpu).astype(np.int32) - ono.astype(np.int32))
        assert d.max() <= 1  # N(0,1) inputs: no sign changes near zero matter here
        qp, qs = orc.quantize(k % 2, mxq.SWIZZLED, bf16_bits(no_gpu), g=80.0)
        assert np.array_equal(u8(p), qp.ravel()) and np.array_equal(u8(s), qs)


def test_grouped_batch_chained(orc):
    """mx_quant_grouped_batch with MXQ_CHAIN (launches after the first
    dispatched any-order): the bytes equal the unchained call's and the
    oracle's, a late producer on the stream is seen by every launch, and a
    consumer queued after the call sees every output."""
    xs_cpu = workloads.small_grouped_experts(n_experts=40, rows=128, cols=512, seed=21)
    xs = [x.to(DEV) for x in xs_cpu]
    plain = mxq.GroupedCall(mxq.MXFP8, mxq.SWIZZLED, xs, max_per_launch=5)
    chained = mxq.GroupedCall(mxq.MXFP8, mxq.SWIZZLED, xs, max_per_launch=5, chain=True)
    say("grouped batch, chained launches")
    sp, ss = plain()
    want = [u8(t).copy() for t in sp + ss]
    late = [x.clone() for x in xs]
    for x in xs:
        x.zero_()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for rep in range(3):
            for t in chained.payloads + chained.scales:
                t.fill_(CANARY)
            torch.cuda._sleep(20_000_000)      # the producer is late ...
            for x, y in zip(xs, late):
                x.copy_(y)                     # ... and restores the inputs
            pays, scs = chained()
            copies = [t.clone() for t in pays + scs]  # a consumer queued after the call
            s.synchronize()
            assert all(np.array_equal(u8(a), b) for a, b in zip(copies, want)), rep
            for x in xs:
                x.zero_()
    for i in (0, 17, 39):
        p, sc = orc.quantize(orc.MXFP8, orc.SWIZZLED, bf16_bits(xs_cpu[i]))
        assert np.array_equal(want[i], p.ravel()) and np.array_equal(want[40 + i], sc)


def test_grouped_batch_chained_graph_replay(orc):
    """Captured into a graph, a chained batch falls back to ordinary
    launches; each replay gives the eager bytes."""
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=20, rows=64, cols=512,
                                                             seed=22)]
    gs = torch.cat([g_of(x) for x in xs])
    call = mxq.GroupedCall(mxq.NVFP4, mxq.LINEAR, xs, global_scales=gs, max_per_launch=7,
                           chain=True)
    say("chained batch graph replay")
    eager = [u8(t).copy() for t in sum(call(), [])]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            call()
    for rep in range(3):
        for t in call.payloads + call.scales:
            t.fill_(CANARY)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [u8(t) for t in call.payloads + call.scales]
        assert all(np.array_equal(a, b) for a, b in zip(eager, got)), rep


def test_grouped_issue_interleaved(orc):
    """issue_interleaved over two side streams: every launch sees a late
    producer on the current stream, a consumer queued after it sees every
    output, and the bytes equal the serial calls' and the oracle's.  The
    calls share one set of outputs, as a benchmark's layers do."""
    xs_cpu = [workloads.small_grouped_experts(n_experts=40, rows=128, cols=512, seed=31 + k)
              for k in range(3)]
    xs = [[x.to(DEV) for x in layer] for layer in xs_cpu]
    first = mxq.GroupedCall(mxq.MXFP8, mxq.SWIZZLED, xs[0], max_per_launch=5)
    calls = [first] + [mxq.GroupedCall(mxq.MXFP8, mxq.SWIZZLED, xs[k], first.payloads,
                                       first.scales, max_per_launch=5) for k in (1, 2)]
    say("grouped calls interleaved over two streams")
    calls[2]()  # the last call's bytes are what the shared outputs end with
    want = [u8(t).copy() for t in first.payloads + first.scales]
    late = [x.clone() for x in xs[2]]
    side = [torch.cuda.Stream(), torch.cuda.Stream()]
    with pytest.raises(ValueError):
        mxq.issue_interleaved(calls, [])
    for rep in range(3):
        for t in first.payloads + first.scales:
            t.fill_(CANARY)
        for x in xs[2]:
            x.zero_()
        torch.cuda._sleep(20_000_000)      # the producer is late ...
        for x, y in zip(xs[2], late):
            x.copy_(y)                     # ... and restores the last call's inputs
        mxq.issue_interleaved(calls, side)
        copies = [t.clone() for t in first.payloads + first.scales]  # a consumer after it
        torch.cuda.current_stream().synchronize()
        assert all(np.array_equal(u8(a), b) for a, b in zip(copies, want)), rep
    for i in (0, 13, 39):
        p, sc = orc.quantize(orc.MXFP8, orc.SWIZZLED, bf16_bits(xs_cpu[2][i]))
        assert np.array_equal(want[i], p.ravel()) and np.array_equal(want[40 + i], sc)
