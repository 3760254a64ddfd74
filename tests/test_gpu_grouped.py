"""GPU parity of mx_quant_grouped against the oracle, byte for byte.

Covers the small grouped workload (8 experts [256,512], MXFP8, linear), the
hand-worked blocks, MXFP8/NVFP4 x linear/swizzled on ragged shapes with
canary-filled outputs and guard bands, batched == per-expert, grid-shape
invariance, the Qwen3-30B-A3B layer shapes, sampled rows of the
Qwen3-235B-A22B layer shapes at full size, stream ordering and graph replay.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from helpers import bf16_bits, hand_blocks
from gpu_common import CANARY, canary_buffer, g_of, guard_intact, say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def oracle_entry(orc, fmt, layout, x_cpu, g=1.0):
    return orc.quantize(fmt, layout, bf16_bits(x_cpu), g=g)


def run_grouped(fmt, layout, xs, gs=None, canary=True):
    """Run one or more grouped calls on canary-filled outputs; returns numpy
    payloads/scales and checks the guard bands."""
    cols = xs[0].shape[1]
    pw = cols if fmt == mxq.MXFP8 else cols // 2
    pays, scs, wholes = [], [], []
    for x in xs:
        n_sc = mxq.scale_bytes(x.shape[0], cols, fmt, layout)
        p, pwhole = canary_buffer(x.shape[0] * pw)
        s, swhole = canary_buffer(n_sc)
        pays.append(p.view(x.shape[0], pw))
        scs.append(s)
        wholes.append((pwhole, x.shape[0] * pw, swhole, n_sc))
    mxq.mx_quant_grouped(fmt, layout, xs, pays, scs, gs)
    torch.cuda.synchronize()
    for pwhole, np_, swhole, ns in wholes:
        assert guard_intact(pwhole, np_) and guard_intact(swhole, ns), "write past the end"
    return [u8(p) for p in pays], [u8(s) for s in scs]


def test_small_grouped_mxfp8_linear(orc):
    say("small grouped 8x[256,512] MXFP8 linear")
    xs_cpu = workloads.small_grouped_experts(seed=0)
    xs = [x.to(DEV) for x in xs_cpu]
    pays, scs = run_grouped(mxq.MXFP8, mxq.LINEAR, xs)
    for i, x in enumerate(xs_cpu):
        p, s = oracle_entry(orc, orc.MXFP8, orc.LINEAR, x)
        assert np.array_equal(pays[i], p.ravel()), f"payload expert {i}"
        assert np.array_equal(scs[i], s), f"scales expert {i}"
        assert scs[i].size == 256 * 16
    # n = 8 in one launch equals eight n = 1 launches
    for i, x in enumerate(xs):
        p1, s1 = run_grouped(mxq.MXFP8, mxq.LINEAR, [x])
        assert np.array_equal(p1[0], pays[i]) and np.array_equal(s1[0], scs[i])


def test_hand_blocks_on_gpu(orc):
    """Every hand-worked block as its own single-block row (the squeezed
    single-block scale shape), compared with the hand-derived bytes."""
    cases = hand_blocks()
    for fmt_name, fmt in (("mxfp8", mxq.MXFP8), ("nvfp4", mxq.NVFP4)):
        cs = [c for c in cases if c["fmt"] == fmt_name]
        say("hand blocks", fmt_name, len(cs))
        xs = [torch.from_numpy(np.array(c["x"], np.uint16).view(np.int16)).view(torch.bfloat16)
              .reshape(1, -1).to(DEV) for c in cs]
        gs = torch.tensor([c["g"] for c in cs], dtype=torch.float32, device=DEV)
        for layout in (mxq.LINEAR, mxq.SWIZZLED):
            pays, scs = run_grouped(fmt, layout, xs, gs if fmt == mxq.NVFP4 else None)
            for c, p, s in zip(cs, pays, scs):
                assert list(p) == c["payload"], c["id"]
                assert s[0] == c["scale"], c["id"]
                assert np.all(s[1:] == 0), c["id"]  # swizzled padding


SHAPES = [(200, 768), (129, 64), (1, 32), (0, 512), (300, 1024), (64, 7168)]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_ragged_shapes_and_canaries(orc, fmt, layout):
    rng = torch.Generator().manual_seed(123 + 10 * fmt + layout)
    for rows, cols in SHAPES:
        if cols % (32 if fmt == 0 else 16):
            continue
        say("ragged", fmt, layout, rows, cols)
        xs_cpu = []
        for k in range(3):
            r = max(rows - 37 * k, 0) if rows else 0
            x = torch.randn(r, cols, generator=rng) * torch.exp(torch.randn(r, 1, generator=rng))
            xs_cpu.append(x.to(torch.bfloat16))
        xs = [x.to(DEV) for x in xs_cpu]
        gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
        pays, scs = run_grouped(fmt, layout, xs, gs)
        for i, x in enumerate(xs_cpu):
            g = float(gs[i]) if fmt == 1 else 1.0
            p, s = oracle_entry(orc, fmt, layout, x, g)
            assert np.array_equal(pays[i], p.ravel()), (rows, cols, i)
            assert np.array_equal(scs[i], s), (rows, cols, i)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_widest_rows(orc, fmt, layout):
    """The widest supported rows (32768 MXFP8, 16384 NVFP4 columns), and one
    block less, whose last 512-column chunk is ragged."""
    rng = torch.Generator().manual_seed(77 + 10 * fmt + layout)
    widest = 32768 if fmt == 0 else 16384
    block = 32 if fmt == 0 else 16
    for cols in (widest, widest - block):
        rows = 131
        say("widest", fmt, layout, rows, cols)
        xs_cpu = [(torch.randn(rows - 50 * k, cols, generator=rng) *
                   torch.exp(torch.randn(rows - 50 * k, 1, generator=rng))).to(torch.bfloat16)
                  for k in range(2)]
        xs = [x.to(DEV) for x in xs_cpu]
        gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
        pays, scs = run_grouped(fmt, layout, xs, gs)
        for i, x in enumerate(xs_cpu):
            p, s = oracle_entry(orc, fmt, layout, x, float(gs[i]) if fmt == 1 else 1.0)
            assert np.array_equal(pays[i], p.ravel()), (cols, i)
            assert np.array_equal(scs[i], s), (cols, i)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_narrowest_rows(orc, fmt, layout):
    """Rows of one block and of three (one 512-column chunk, mostly idle
    lanes; swizzled scale columns padded to a tile)."""
    rng = torch.Generator().manual_seed(91 + 10 * fmt + layout)
    block = 32 if fmt == 0 else 16
    for cols in (block, 3 * block):
        say("narrow rows", fmt, layout, cols)
        xs_cpu = [(torch.randn(r, cols, generator=rng) * 5).to(torch.bfloat16) for r in (1, 130, 300)]
        xs = [x.to(DEV) for x in xs_cpu]
        gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
        pays, scs = run_grouped(fmt, layout, xs, gs)
        for i, x in enumerate(xs_cpu):
            p, s = oracle_entry(orc, fmt, layout, x, float(gs[i]) if fmt == 1 else 1.0)
            assert np.array_equal(pays[i], p.ravel()) and np.array_equal(scs[i], s), (cols, i)


def test_empty_expert_with_zero_strides(orc):
    """A zero-row expert whose strides are (0, 0) (an empty array from numpy)
    is accepted among ordinary experts and changes none of their bytes."""
    empty = torch.from_numpy(np.zeros((0, 256), np.int16)).view(torch.bfloat16).to(DEV)
    assert empty.stride() == (0, 0) or empty.shape[0] == 0
    xs_cpu = [(torch.randn(r, 256) * 3).to(torch.bfloat16) for r in (70, 1)]
    xs = [xs_cpu[0].to(DEV), empty, xs_cpu[1].to(DEV)]
    gs = torch.cat([g_of(xs[0]), torch.ones(1, device=DEV), g_of(xs[2])])
    say("empty expert, zero strides")
    for fmt in (0, 1):
        pays, scs = run_grouped(fmt, mxq.SWIZZLED, xs, gs if fmt == 1 else None)
        assert pays[1].size == 0 and scs[1].size == 0
        for i, x in ((0, xs_cpu[0]), (2, xs_cpu[1])):
            p, s = oracle_entry(orc, fmt, orc.SWIZZLED, x, float(gs[i]) if fmt == 1 else 1.0)
            assert np.array_equal(pays[i], p.ravel()) and np.array_equal(scs[i], s), (fmt, i)
    pays, scs, g, am = mxq.nvfp4_quant_grouped_auto(mxq.SWIZZLED, xs)
    torch.cuda.synchronize()
    assert float(am[1]) == 0.0 and float(g[1]) == 1.0


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_scales_at_odd_offsets(orc, fmt):
    """Linear scale matrices may start at any byte.  Three experts' scales sit
    at byte offsets 1, 2 and 3 (mod 16) of one canary-filled buffer, so the
    rows that would leave as 16-byte stores leave byte by byte; the canary
    between the regions stays."""
    rng = torch.Generator().manual_seed(31 + fmt)
    cols = 1024
    xs_cpu = [(torch.randn(r, cols, generator=rng) * 3).to(torch.bfloat16) for r in (70, 33, 16)]
    xs = [x.to(DEV) for x in xs_cpu]
    gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
    n_sc = [mxq.scale_bytes(x.shape[0], cols, fmt, mxq.LINEAR) for x in xs]
    starts, pos = [], 0
    for k, n in enumerate(n_sc):
        pos = (pos + 15) // 16 * 16 + 16 + k + 1  # a canary gap, then offset k + 1
        starts.append(pos)
        pos += n
    total = pos + 16
    whole = torch.full((total,), CANARY, dtype=torch.uint8, device=DEV)
    scs = [whole[st:st + n] for st, n in zip(starts, n_sc)]
    pw = cols if fmt == 0 else cols // 2
    pays = [torch.empty(x.shape[0], pw, dtype=torch.uint8, device=DEV) for x in xs]
    say("odd linear scale offsets", fmt)
    mxq.mx_quant_grouped(fmt, mxq.LINEAR, xs, pays, scs, gs)
    torch.cuda.synchronize()
    w = u8(whole)
    outside = np.ones(total, bool)
    for st, n in zip(starts, n_sc):
        outside[st:st + n] = False
    assert np.all(w[outside] == CANARY)
    for i, x in enumerate(xs_cpu):
        p, sc = oracle_entry(orc, fmt, orc.LINEAR, x, float(gs[i]) if fmt == 1 else 1.0)
        assert np.array_equal(u8(pays[i]), p.ravel()) and np.array_equal(u8(scs[i]), sc), i


@pytest.mark.parametrize("fmt", [0, 1])
def test_strided_source_rows(orc, fmt):
    say("strided src", fmt)
    big = (torch.randn(96, 1024) * 3).to(torch.bfloat16)
    x_cpu = big[:, 128:128 + 512]
    x = big.to(DEV)[:, 128:128 + 512]
    gs = g_of(x) if fmt == 1 else None
    pays, scs = run_grouped(fmt, mxq.SWIZZLED, [x], gs)
    p, s = oracle_entry(orc, fmt, orc.SWIZZLED, x_cpu.contiguous(), float(gs[0]) if fmt else 1.0)
    assert np.array_equal(pays[0], p.ravel()) and np.array_equal(scs[0], s)


@pytest.mark.parametrize("fmt", [0, 1])
def test_grid_shape_invariance(orc, fmt):
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=5, rows=300, cols=768,
                                                             seed=5)]
    gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
    ref = run_grouped(fmt, mxq.SWIZZLED, xs, gs)
    try:
        for cap in (1, 3, 7, 64):
            say("grid cap", cap, "fmt", fmt)
            mxq.set_max_workgroups(cap)
            got = run_grouped(fmt, mxq.SWIZZLED, xs, gs)
            for a, b in zip(ref[0] + ref[1], got[0] + got[1]):
                assert np.array_equal(a, b), cap
    finally:
        mxq.set_max_workgroups(0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_batched_equals_per_expert_16_and_17(orc, fmt):
    """17 experts: the binding issues 16 + 1; each equals its n = 1 call."""
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=17, rows=64, cols=256,
                                                             seed=17)]
    gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
    say("17 experts", fmt)
    pays, scs = run_grouped(fmt, mxq.SWIZZLED, xs, gs)
    for i, x in enumerate(xs):
        p1, s1 = run_grouped(fmt, mxq.SWIZZLED, [x], gs[i:i + 1] if fmt == 1 else None)
        assert np.array_equal(p1[0], pays[i]) and np.array_equal(s1[0], scs[i]), i


@pytest.mark.parametrize("fmt", [0, 1])
def test_per_call_cap_keeps_bytes(fmt):
    """The binding's per-call cap (1, 5 or 16 experts per launch) changes the
    launches, never the bytes."""
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=11, rows=96, cols=512,
                                                             seed=11)]
    gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
    say("per-call cap", fmt)
    ref = None
    for cap in (16, 5, 1):
        pays, scs = mxq.mx_quant_grouped(fmt, mxq.LINEAR, xs, global_scales=gs,
                                         max_per_launch=cap)
        got = [u8(t) for t in pays + scs]
        if ref is None:
            ref = got
        assert all(np.array_equal(a, b) for a, b in zip(got, ref)), cap


@pytest.mark.parametrize("fmt", [0, 1])
def test_qwen3_30b_layer_shapes(orc, fmt):
    """Qwen3-30B-A3B layer shapes, 16 experts per launch (one launch per
    projection here), swizzled scales, byte-exact on every expert."""
    for proj, (rows, cols) in workloads.QWEN3_30B_A3B.items():
        say("qwen3-30b", proj, fmt)
        stack = workloads.expert_stack(16, rows, cols, std=0.02, seed=2000, device=DEV)
        xs = [stack[i] for i in range(16)]
        gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
        pays, scs = run_grouped(fmt, mxq.SWIZZLED, xs, gs, canary=False)
        for i in (0, 7, 15):
            g = float(gs[i]) if fmt == 1 else 1.0
            p, s = oracle_entry(orc, fmt, orc.SWIZZLED, xs[i].cpu(), g)
            assert np.array_equal(pays[i], p.ravel()), (proj, i)
            assert np.array_equal(scs[i], s), (proj, i)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_qwen3_235b_full_size_sampled_rows(orc, fmt, layout):
    """Full Qwen3-235B-A22B launch shapes (16 x [3072,4096] and 16 x
    [4096,1536]) in the benchmark's launch configuration; rows are
    independent, so sampled rows are checked against the oracle row by row,
    together with their scale bytes."""
    rng = np.random.default_rng(fmt * 2 + layout)
    for proj, (rows, cols) in workloads.QWEN3_235B_A22B.items():
        say("qwen3-235b", proj, "fmt", fmt, "layout", layout)
        stack = workloads.expert_stack(16, rows, cols, std=0.015, seed=5000, device=DEV)
        xs = [stack[i] for i in range(16)]
        gs = torch.cat([g_of(x) for x in xs]) if fmt == 1 else None
        pays, scs = run_grouped(fmt, layout, xs, gs, canary=False)
        C = cols // (32 if fmt == 0 else 16)
        pw = cols if fmt == 0 else cols // 2
        for i in (0, 5, 15):
            sample = np.sort(rng.choice(rows, 24, replace=False))
            sample[0], sample[-1] = 0, rows - 1
            xi = xs[i][torch.from_numpy(sample).to(DEV)].cpu()
            g = float(gs[i]) if fmt == 1 else 1.0
            p, s = orc.quantize(fmt, orc.LINEAR, bf16_bits(xi), g=g)
            got_p = pays[i].reshape(rows, pw)[sample]
            assert np.array_equal(got_p, p), (proj, i)
            offs = np.array([[orc.sf_offset(r, c, C, layout) for c in range(C)] for r in sample])
            assert np.array_equal(scs[i][offs], s.reshape(len(sample), C)), (proj, i)
        if layout == 1:  # no padding at these shapes: every scale byte is live
            assert scs[0].size == rows * C


def test_stream_order(orc):
    """Work is enqueued on the caller's current stream: a late producer on
    that stream is seen."""
    x_cpu = workloads.small_grouped_experts(n_experts=1, rows=256, cols=512, seed=3)[0]
    y_cpu = workloads.small_grouped_experts(n_experts=1, rows=256, cols=512, seed=4)[0]
    x = x_cpu.to(DEV)
    y = y_cpu.to(DEV)
    s = torch.cuda.Stream()
    say("stream order")
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)
        x.copy_(y)
        pays, scs = mxq.mx_quant_grouped(mxq.MXFP8, mxq.SWIZZLED, [x])
    s.synchronize()
    p, sc = oracle_entry(orc, orc.MXFP8, orc.SWIZZLED, y_cpu)
    assert np.array_equal(u8(pays[0]), p.ravel()) and np.array_equal(u8(scs[0]), sc)


def test_graph_replay(orc):
    """A captured grouped call replays to the eager bytes, replay after replay,
    with eager work and synchronizations in between."""
    xs = [x.to(DEV) for x in workloads.small_grouped_experts(n_experts=4, rows=256, cols=512,
                                                             seed=9)]
    gs = torch.cat([g_of(x) for x in xs])
    say("graph replay")
    eager = mxq.mx_quant_grouped(mxq.NVFP4, mxq.SWIZZLED, xs, global_scales=gs)
    eager = [u8(t) for t in eager[0] + eager[1]]
    outs_p = [torch.empty((x.shape[0], x.shape[1] // 2), dtype=torch.uint8, device=DEV) for x in xs]
    outs_s = [torch.empty(mxq.scale_bytes(x.shape[0], x.shape[1], mxq.NVFP4, mxq.SWIZZLED),
                          dtype=torch.uint8, device=DEV) for x in xs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        mxq.mx_quant_grouped(mxq.NVFP4, mxq.SWIZZLED, xs, outs_p, outs_s, gs)  # warm-up
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            mxq.mx_quant_grouped(mxq.NVFP4, mxq.SWIZZLED, xs, outs_p, outs_s, gs)
    for rep in range(3):
        for t in outs_p + outs_s:
            t.fill_(CANARY)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [u8(t) for t in outs_p + outs_s]
        for a, b in zip(eager, got):
            assert np.array_equal(a, b), rep
