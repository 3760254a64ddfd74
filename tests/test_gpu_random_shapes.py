"""Seeded random cases for every entry point against the oracle.

Each case draws its shape, format, layout, encode scale and value spread
from a fixed seed, so a failure names a reproducible case; every output byte
is compared (norm_out within 1 bf16 ulp).  Sizes stay small enough for the
oracle to finish the whole set in seconds.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from helpers import bf16_bits
from gpu_common import say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 48


def _values(gen, rows, cols):
    spread = float(torch.empty(1).uniform_(-3.0, 3.0, generator=gen))
    x = torch.randn(rows, cols, generator=gen) * torch.exp(
        spread * torch.randn(rows, 1, generator=gen))
    x = x * 10.0 ** float(torch.randint(-6, 6, (1,), generator=gen))
    bits = bf16_bits(x.to(torch.bfloat16)).copy()
    if rows > 2:
        bits[int(torch.randint(0, rows, (1,), generator=gen))] = 0x8000  # a -0 row
    return bits


def _to_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def _g_of(bits, orc):
    return np.float32(orc.nvfp4_encode_scale(float(np.abs((bits.astype(np.uint32) << 16)
                                                              .view(np.float32)).max())))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_grouped(orc, case):
    gen = torch.Generator().manual_seed(1000 + case)
    fmt = int(torch.randint(0, 2, (1,), generator=gen))
    layout = int(torch.randint(0, 2, (1,), generator=gen))
    block = 32 if fmt == mxq.MXFP8 else 16
    cols = block * int(torch.randint(1, 80, (1,), generator=gen))
    n = int(torch.randint(1, 18, (1,), generator=gen))
    srcs = [_values(gen, int(torch.randint(0, 300, (1,), generator=gen)), cols) for _ in range(n)]
    gs = [_g_of(b, orc) if b.size else np.float32(1.0) for b in srcs]
    say("random grouped", case, "fmt", fmt, "layout", layout, "cols", cols, "n", n)
    xs = [_to_dev(b) for b in srcs]
    g_dev = torch.tensor(gs, dtype=torch.float32, device=DEV)
    pays, scs = mxq.mx_quant_grouped(fmt, layout, xs, global_scales=g_dev if fmt else None)
    torch.cuda.synchronize()
    for b, gi, p, s in zip(srcs, gs, pays, scs):
        op, os_ = orc.quantize(fmt, layout, b.reshape(-1, cols), g=float(gi))
        assert np.array_equal(u8(p), op.ravel()) and np.array_equal(u8(s), os_)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_split(orc, case):
    gen = torch.Generator().manual_seed(2000 + case)
    mode = ("nvfp4", "nvfp4_row_scaled", "mxfp8")[int(torch.randint(0, 3, (1,), generator=gen))]
    fmt = mxq.MXFP8 if mode == "mxfp8" else mxq.NVFP4
    layout = int(torch.randint(0, 2, (1,), generator=gen))
    block = 32 if fmt == mxq.MXFP8 else 16
    cols = block * int(torch.randint(1, 100, (1,), generator=gen))
    n = int(torch.randint(1, 40, (1,), generator=gen))
    top = int(torch.randint(1, 400, (1,), generator=gen))
    split = [int(v) for v in torch.randint(0, top, (n,), generator=gen)]
    if sum(split) == 0:
        split[0] = 1
    bits = _values(gen, sum(split), cols)
    g = _g_of(bits, orc)
    say("random split", case, mode, "layout", layout, "cols", cols, "splits", n, "rows", sum(split))
    x = _to_dev(bits)
    g_dev = torch.tensor([g], dtype=torch.float32, device=DEV)
    p, s, a = mxq.SplitCall(mode, x, split, layout, g_dev if mode == "nvfp4" else None)()
    torch.cuda.synchronize()
    op, os_, oa = orc.split(fmt, bits, split, g=float(g), layout=layout,
                            row_scaled=mode == "nvfp4_row_scaled")
    assert np.array_equal(u8(p), op.ravel())
    assert np.array_equal(u8(s), os_)
    assert np.array_equal(a.cpu().numpy(), oa)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_fused(orc, case):
    gen = torch.Generator().manual_seed(3000 + case)
    fmt = int(torch.randint(0, 2, (1,), generator=gen))
    layout = int(torch.randint(0, 2, (1,), generator=gen))
    step = (128 if fmt == mxq.MXFP8 else 64) if layout == mxq.SWIZZLED else \
        (32 if fmt == mxq.MXFP8 else 16)
    H = step * int(torch.randint(1, max(2, 8192 // step), (1,), generator=gen))
    T = int(torch.randint(1, 2600, (1,), generator=gen)) if case % 3 else \
        int(torch.randint(1, 9, (1,), generator=gen))
    T = min(T, max(1, (1 << 22) // H))  # keep the oracle's work bounded
    x = _values(gen, T, H)
    r = _values(gen, T, H)
    gm = bf16_bits((1.0 + 0.1 * torch.randn(H, generator=gen)).to(torch.bfloat16))
    eps = float(10.0 ** float(torch.randint(-8, -2, (1,), generator=gen)))
    ro_o, no_o = orc.add_rmsnorm(x, r, gm, eps)
    g = _g_of(no_o, orc) if fmt else np.float32(1.0)
    say("random fused", case, "fmt", fmt, "layout", layout, "T", T, "H", H, "eps", eps)
    g_dev = torch.tensor([g], dtype=torch.float32, device=DEV)
    ro, no, p, s = mxq.rmsnorm_quant_fused(_to_dev(x), _to_dev(r), _to_dev(gm), eps, fmt, layout,
                                           g_dev)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(ro), ro_o)

    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    assert np.abs(key(bf16_bits(no)) - key(no_o)).max() <= 1
    op, os_ = orc.quantize(fmt, layout, bf16_bits(no), g=float(g))
    assert np.array_equal(u8(p), op.ravel()) and np.array_equal(u8(s), os_)


@pytest.mark.parametrize("case", range(24))
def test_random_auto_scale(orc, case):
    gen = torch.Generator().manual_seed(4000 + case)
    layout = int(torch.randint(0, 2, (1,), generator=gen))
    cols = 16 * int(torch.randint(1, 80, (1,), generator=gen))
    n = int(torch.randint(1, 17, (1,), generator=gen))
    n_slots = int(torch.randint(1, n + 1, (1,), generator=gen))
    slots = [int(v) for v in torch.randint(0, n_slots, (n,), generator=gen)]
    srcs = [_values(gen, int(torch.randint(0, 200, (1,), generator=gen)), cols) for _ in range(n)]
    say("random auto", case, "layout", layout, "cols", cols, "n", n, "slots", slots)
    xs = [_to_dev(b) for b in srcs]
    pays, scs, g, am = mxq.nvfp4_quant_grouped_auto(layout, xs, slots)
    torch.cuda.synchronize()
    op, os_, og, oa = orc.quantize_auto(layout, [b.reshape(-1, cols) for b in srcs], slots, cols)
    k = max(slots) + 1
    assert np.array_equal(am[:k].cpu().numpy(), oa) and np.array_equal(g[:k].cpu().numpy(), og)
    for i in range(n):
        assert np.array_equal(u8(pays[i]), op[i].ravel()) and np.array_equal(u8(scs[i]), os_[i])


@pytest.mark.parametrize("case", range(24))
def test_random_swizzle(orc, case):
    """scale_swizzle on random [rows, cols] matrices: ragged bands, any column
    count (word and byte loads), one to many 16-tile units per band."""
    gen = torch.Generator().manual_seed(5000 + case)
    rows = int(torch.randint(0, 3000, (1,), generator=gen))
    cols = int(torch.randint(1, 700, (1,), generator=gen))
    lin = torch.randint(0, 256, (rows, cols), generator=gen, dtype=torch.int32).to(torch.uint8)
    say("random swizzle", case, "rows", rows, "cols", cols)
    got = mxq.scale_swizzle(lin.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(u8(got), orc.scale_swizzle(lin.numpy()))
