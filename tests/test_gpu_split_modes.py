"""GPU parity of the row-scaled NVFP4 split and the MXFP8 split.

Row-scaled: the hand-worked rows of tests/golden/row_scaled_rows.txt at
several positions of a split; a hand split set whose rows span 2^-133 (capped
encode scale) to 2^127 with zero and negative-zero rows; the routed
activation at full size ([8192,7168], 256 experts, 10 empty); every row width
class the kernel instantiates; grid invariance.  MXFP8: the same hand split
set and the full routed activation, requantization isolation.  All outputs
byte for byte against the oracle, with canary-filled buffers and guard bands.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from helpers import bf16_bits, bits_to_bf16, row_scaled_rows
from gpu_common import CANARY, canary_buffer, guard_intact, say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(fmt, x, split, layout):
    """Run the row-scaled NVFP4 (fmt NVFP4) or MXFP8 split into canary buffers."""
    T, H = x.shape
    pw = H if fmt == mxq.MXFP8 else H // 2
    total = mxq.split_scale_offset(split, len(split), H, fmt, layout)
    p, pg = canary_buffer(T * pw)
    s, sg = canary_buffer(total)
    a = torch.full((T + 1024,), float("nan"), dtype=torch.float32, device=DEV)
    if fmt == mxq.MXFP8:
        mxq.mxfp8_quant_split(x, split, layout, p.view(T, pw), s, a[:T])
    else:
        mxq.nvfp4_quant_split_row_scaled(x, split, layout, p.view(T, pw), s, a[:T])
    torch.cuda.synchronize()
    assert guard_intact(pg, T * pw) and guard_intact(sg, total)
    assert torch.all(torch.isnan(a[T:])).item()
    return p, s, a[:T]


def check(orc, fmt, x_cpu, split, layout):
    x = x_cpu.to(DEV)
    p, s, a = run(fmt, x, split, layout)
    op, os_, oa = orc.split(fmt, bf16_bits(x_cpu), split, layout=layout,
                            row_scaled=fmt == mxq.NVFP4)
    assert np.array_equal(u8(p), op.ravel())
    assert np.array_equal(u8(s), os_)
    assert np.array_equal(a.cpu().numpy(), oa)
    return x, p, s, a


def extreme_rows(T, H, seed):
    """Rows N(0,1) * exp(N(0,2)) plus rows that reach the clamps and zeros."""
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=gen) * torch.exp(2.0 * torch.randn(T, 1, generator=gen))
    bits = bf16_bits(x.to(torch.bfloat16)).copy()
    bits[3] = 0x0000                       # zero row
    bits[5] = 0x8000                       # negative zeros
    bits[7] = (np.arange(H) % 3 + 1)       # subnormals 2^-133..3*2^-133: g capped at FLT_MAX*2^-9
    bits[11] = 0x7F00                      # 2^127 everywhere: g = 21*2^-120, below the table range edge
    bits[11, ::7] = 0x7B80                 # ... with 2^120 entries
    bits[13, :] = 0x3F80
    bits[13, min(17, H - 1)] = 0x7F7F      # bf16 max in one place
    return bits_to_bf16(bits)


HAND_SPLIT = [0, 1, 127, 128, 129, 0, 255, 256, 3, 31, 32, 33, 0]


@pytest.mark.parametrize("layout", [0, 1])
def test_row_scaled_hand_rows(orc, layout):
    cases = row_scaled_rows()
    x_bits = np.array([c["x"] for c in cases], np.uint16)
    x_cpu = bits_to_bf16(x_bits)
    for split in ([len(cases)], [2, 0, len(cases) - 2], [1] * len(cases)):
        say("row-scaled hand rows, layout", layout, "split", split)
        x, p, s, a = check(orc, mxq.NVFP4, x_cpu, split, layout)
        pay = u8(p).reshape(len(cases), 16)
        for r, c in enumerate(cases):
            assert list(pay[r]) == c["payload"], c["id"]
            assert float(a[r]) == orc.bf16_value(c["amax"]), c["id"]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_split_hand_set_extremes(orc, fmt, layout):
    T, H = sum(HAND_SPLIT), 7168
    say("split hand set with extreme rows, fmt", fmt, "layout", layout)
    check(orc, fmt, extreme_rows(T, H, seed=78), HAND_SPLIT, layout)


@pytest.mark.parametrize("H", [64, 528, 1040, 2048, 4096, 5136, 8192, 16384])
@pytest.mark.parametrize("fmt", [0, 1])
def test_split_row_widths(orc, fmt, H):
    """Every half-row step count the kernel instantiates (1, 2, 4, 7, 8, 16),
    with ragged tails inside a 512-column step."""
    if fmt == mxq.MXFP8 and H % 32:
        H += 16
    split = [3, 0, 40, 129]
    T = sum(split)
    for layout in (0, 1):
        say("split widths, fmt", fmt, "H", H, "layout", layout)
        check(orc, fmt, extreme_rows(T, H, seed=H), split, layout)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_split_routed_activation_full_size(orc, fmt, layout):
    x_cpu, split = workloads.routed_activation()
    assert sum(split) == 8192 and sum(1 for m in split if m == 0) >= 10
    say("split [8192,7168] x 256 experts, fmt", fmt, "layout", layout)
    x, p, s, a = check(orc, fmt, x_cpu, split, layout)
    # requantizing one expert into its own slice changes nothing else
    H = 7168
    pw = H if fmt == mxq.MXFP8 else H // 2
    i = max(range(len(split)), key=lambda k: split[k])
    o, m = sum(split[:i]), split[i]
    base = mxq.split_scale_offset(split, i, H, fmt, layout)
    size = mxq.split_scale_offset(split, i + 1, H, fmt, layout) - base
    before_p, before_s = u8(p).copy(), u8(s).copy()
    p[o * pw:(o + m) * pw].fill_(CANARY)
    s[base:base + size].fill_(CANARY)
    say("requantize expert", i, "rows", m)
    dst_p = p[o * pw:(o + m) * pw].view(m, pw)
    if fmt == mxq.MXFP8:
        mxq.mxfp8_quant_split(x[o:o + m], [m], layout, dst_p, s[base:base + size], a[o:o + m])
    else:
        mxq.nvfp4_quant_split_row_scaled(x[o:o + m], [m], layout, dst_p, s[base:base + size],
                                         a[o:o + m])
    torch.cuda.synchronize()
    assert np.array_equal(u8(p), before_p) and np.array_equal(u8(s), before_s)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_split_grid_invariance(orc, fmt, layout):
    """Capped grids make each workgroup loop over many units (the row-scaled
    form alternates its LDS exchange buffers across them): same bytes."""
    split = [0, 300, 1, 129, 0, 77]
    T, H = sum(split), 1536
    x_cpu = extreme_rows(T, H, seed=5)
    try:
        for cap in (1, 3, 7):
            mxq.set_max_workgroups(cap)
            say("split grid cap", cap, "fmt", fmt, "layout", layout)
            check(orc, fmt, x_cpu, split, layout)
    finally:
        mxq.set_max_workgroups(0)


def test_split_many_launches(orc):
    """More than 256 splits take several launches; offsets carry over."""
    gen = torch.Generator().manual_seed(11)
    split = torch.randint(0, 9, (600,), generator=gen).tolist()
    T, H = sum(split), 256
    x_cpu = extreme_rows(T, H, seed=12)
    for fmt in (0, 1):
        for layout in (0, 1):
            say("600 splits, fmt", fmt, "layout", layout)
            check(orc, fmt, x_cpu, split, layout)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_split_narrowest_rows(orc, fmt, layout):
    """Rows of one block and of three: most lanes of both waves of a row hold
    no column; swizzled scale columns are padded to a tile."""
    split = [0, 1, 130, 31, 0, 2]
    block = 32 if fmt == 0 else 16
    for H in (block, 3 * block):
        say("split narrow rows, fmt", fmt, "layout", layout, "H", H)
        check(orc, fmt, extreme_rows(sum(split), H, seed=70 + H), split, layout)


@pytest.mark.parametrize("mode", ["nvfp4", "mxfp8"])
def test_split_linear_scales_at_odd_offset(orc, mode):
    """Linear split scales may start at any byte: the bulk buffer at byte
    offsets 1..3 (mod 16) takes byte stores for rows that would leave as
    16-byte runs; the canary before and after stays."""
    fmt = mxq.MXFP8 if mode == "mxfp8" else mxq.NVFP4
    split = [0, 70, 33, 1, 0, 16]
    T, H = sum(split), 1024
    x_cpu = extreme_rows(T, H, seed=61)
    x = x_cpu.to(DEV)
    total = mxq.split_scale_offset(split, len(split), H, fmt, mxq.LINEAR)
    g = torch.tensor([37.0], dtype=torch.float32, device=DEV)
    op, os_, oa = orc.split(fmt, bf16_bits(x_cpu), split, g=37.0, layout=mxq.LINEAR)
    for off in (1, 2, 3):
        whole = torch.full((total + 32,), CANARY, dtype=torch.uint8, device=DEV)
        sc = whole[off:off + total]
        say("split odd linear scale offset", mode, off)
        call = mxq.SplitCall(mode, x, split, mxq.LINEAR, g if mode == "nvfp4" else None,
                             scales=sc)
        p, s, a = call()
        torch.cuda.synchronize()
        w = u8(whole)
        assert np.all(w[:off] == CANARY) and np.all(w[off + total:] == CANARY)
        assert np.array_equal(u8(p), op.ravel()) and np.array_equal(u8(s), os_)
        assert np.array_equal(a.cpu().numpy(), oa)


LONG_SPLITS = ([0, 300, 129, 0, 500], [128, 256, 1], [1000], [128, 128])


@pytest.mark.parametrize("mode", ["nvfp4", "nvfp4_row_scaled", "mxfp8"])
@pytest.mark.parametrize("layout", [0, 1])
def test_split_long_experts(orc, mode, layout):
    """Experts of 128 rows or more: whole 128-row bands, rows of one unit in
    two experts, bands with no padding unit: same bytes as the oracle, also
    with capped grids."""
    fmt = mxq.MXFP8 if mode == "mxfp8" else mxq.NVFP4
    for k, split in enumerate(LONG_SPLITS):
        T, H = sum(split), 1536
        x_cpu = extreme_rows(T, H, seed=40 + k)
        x = x_cpu.to(DEV)
        for cap in (0, 3):
            mxq.set_max_workgroups(cap)
            try:
                say("long experts", mode, "layout", layout, "split", split, "cap", cap)
                if mode == "nvfp4":
                    g = torch.tensor([37.0], dtype=torch.float32, device=DEV)
                    p, s, a = mxq.nvfp4_quant_split(x, split, g, layout)
                    torch.cuda.synchronize()
                    op, os_, oa = orc.split(fmt, bf16_bits(x_cpu), split, g=37.0, layout=layout)
                    assert np.array_equal(u8(p), op.ravel()) and np.array_equal(u8(s), os_)
                    assert np.array_equal(a.cpu().numpy(), oa)
                else:
                    check(orc, fmt, x_cpu, split, layout)
            finally:
                mxq.set_max_workgroups(0)
