"""GPU parity of nvfp4_quant_split, rmsnorm_quant_fused and scale_swizzle.

Split: the routed-activation workload at full size ([8192,7168], 256
experts, 10 empty) and a hand split set with uneven, empty and
128-multiple splits; canary-filled bulk buffers; requantizing one expert
leaves every other byte untouched.  Fused: T in {1,16,64,256,1024,4096} at
H = 7168: residual_out exact, norm_out within 1 bf16 ulp of the oracle,
payload and scales equal to the oracle's quantization of the GPU norm_out,
padded scale rows zero.  Swizzle: equals the oracle and the quantizer's own
swizzled output.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from helpers import bf16_bits
from gpu_common import CANARY, canary_buffer, g_of, guard_intact, say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_split(x, split, g, layout):
    T, H = x.shape
    total = mxq.split_scale_offset(split, len(split), H, mxq.NVFP4, layout)
    p, pw = canary_buffer(T * H // 2)
    s, sw = canary_buffer(total)
    a = torch.full((T + 1024,), float("nan"), dtype=torch.float32, device=DEV)
    mxq.nvfp4_quant_split(x, split, g, layout, p.view(T, H // 2), s, a[:T])
    torch.cuda.synchronize()
    assert guard_intact(pw, T * H // 2) and guard_intact(sw, total)
    assert torch.all(torch.isnan(a[T:])).item()
    return p, s, a[:T], total


@pytest.mark.parametrize("layout", [0, 1])
def test_split_hand_set(orc, layout):
    split = [0, 1, 127, 128, 129, 0, 255, 256, 3, 31, 32, 33, 0]
    T, H = sum(split), 7168
    gen = torch.Generator().manual_seed(77)
    x_cpu = (torch.randn(T, H, generator=gen) * 2).to(torch.bfloat16)
    x = x_cpu.to(DEV)
    g = g_of(x)
    say("split hand set, layout", layout)
    p, s, a, total = run_split(x, split, g, layout)
    op, os_, oa = orc.nvfp4_split(bf16_bits(x_cpu), split, float(g), layout)
    assert np.array_equal(u8(p), op.ravel())
    assert np.array_equal(u8(s), os_)
    assert np.array_equal(a.cpu().numpy(), oa)


@pytest.mark.parametrize("layout", [0, 1])
def test_split_routed_activation_full_size(orc, layout):
    x_cpu, split = workloads.routed_activation()
    assert sum(split) == 8192 and sum(1 for m in split if m == 0) >= 10
    x = x_cpu.to(DEV)
    g = g_of(x)
    say("split [8192,7168] x 256 experts, layout", layout)
    p, s, a, total = run_split(x, split, g, layout)
    op, os_, oa = orc.nvfp4_split(bf16_bits(x_cpu), split, float(g), layout)
    assert np.array_equal(u8(p), op.ravel())
    assert np.array_equal(u8(s), os_)
    assert np.array_equal(a.cpu().numpy(), oa)
    # requantizing one expert into its own slice changes nothing else
    i = max(range(len(split)), key=lambda k: split[k])
    o = sum(split[:i])
    m = split[i]
    base = mxq.split_scale_offset(split, i, 7168, mxq.NVFP4, layout)
    size = mxq.split_scale_offset(split, i + 1, 7168, mxq.NVFP4, layout) - base
    before_p, before_s = u8(p).copy(), u8(s).copy()
    p[o * 3584:(o + m) * 3584].fill_(CANARY)
    s[base:base + size].fill_(CANARY)
    say("requantize expert", i, "rows", m)
    mxq.nvfp4_quant_split(x[o:o + m], [m], g, layout, p[o * 3584:(o + m) * 3584].view(m, 3584),
                          s[base:base + size], a[o:o + m])
    torch.cuda.synchronize()
    assert np.array_equal(u8(p), before_p) and np.array_equal(u8(s), before_s)


def test_split_equals_grouped_per_expert(orc):
    """The split's per-expert storage equals quantizing each slice alone."""
    split = [5, 0, 130, 64, 1]
    T, H = sum(split), 1024
    x = (torch.randn(T, H) * 3).to(torch.bfloat16).to(DEV)
    g = g_of(x)
    say("split vs grouped")
    p, s, a, total = run_split(x, split, g, mxq.SWIZZLED)
    o = 0
    for i, m in enumerate(split):
        base = mxq.split_scale_offset(split, i, H)
        if m:
            gp, gs = mxq.mx_quant_grouped(mxq.NVFP4, mxq.SWIZZLED, [x[o:o + m]],
                                          global_scales=g)
            assert np.array_equal(u8(gp[0]), u8(p)[o * H // 2:(o + m) * H // 2])
            assert np.array_equal(u8(gs[0]), u8(s)[base:base + gs[0].numel()])
        o += m


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between bit patterns (sign-magnitude ordered)."""
    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))


@pytest.mark.parametrize("T", [1, 16, 64, 256, 1024, 4096])
def test_fused_epilogue(orc, T):
    H = 7168
    x_c, r_c, g_c = workloads.epilogue_inputs(T, H)
    x, r, gm = x_c.to(DEV), r_c.to(DEV), g_c.to(DEV)
    nb = mxq.scale_bytes(T, H, mxq.MXFP8, mxq.SWIZZLED)
    ro = torch.empty_like(x)
    no = torch.empty_like(x)
    pay, pw = canary_buffer(T * H)
    sc, sw = canary_buffer(nb)
    say("fused T =", T)
    mxq.rmsnorm_quant_fused(x, r, gm, 1e-6, mxq.MXFP8, mxq.SWIZZLED,
                            out=(ro, no, pay.view(T, H), sc))
    torch.cuda.synchronize()
    assert guard_intact(pw, T * H) and guard_intact(sw, nb)
    oro, ono = orc.add_rmsnorm(bf16_bits(x_c), bf16_bits(r_c), bf16_bits(g_c), 1e-6)
    assert np.array_equal(bf16_bits(ro), oro)
    d = bf16_ulp_diff(bf16_bits(no), ono)
    assert d.max() <= 1, d.max()
    # the quantized form is the quantization of the GPU's own norm_out
    qp, qs = orc.quantize(orc.MXFP8, orc.SWIZZLED, bf16_bits(no))
    assert np.array_equal(u8(pay), qp.ravel())
    assert np.array_equal(u8(sc), qs)
    # invented scale rows T..round_up(T,128) are zero
    C = H // 32
    rows_pad = -(-T // 128) * 128
    offs = [orc.sf_offset(rr, c, C, orc.SWIZZLED) for rr in range(T, rows_pad) for c in (0, C - 1)]
    assert np.all(u8(sc)[offs] == 0)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_fused_formats_layouts(orc, fmt, layout):
    T, H = 77, 1024
    x_c, r_c, g_c = workloads.epilogue_inputs(T, H, seed=31)
    x, r, gm = x_c.to(DEV), r_c.to(DEV), g_c.to(DEV)
    gs = torch.tensor([37.5], dtype=torch.float32, device=DEV)
    say("fused fmt/layout", fmt, layout)
    ro, no, pay, sc = mxq.rmsnorm_quant_fused(x, r, gm, 1e-5, fmt, layout, gs if fmt else None)
    torch.cuda.synchronize()
    oro, ono = orc.add_rmsnorm(bf16_bits(x_c), bf16_bits(r_c), bf16_bits(g_c), 1e-5)
    assert np.array_equal(bf16_bits(ro), oro)
    assert bf16_ulp_diff(bf16_bits(no), ono).max() <= 1
    qp, qs = orc.quantize(fmt, layout, bf16_bits(no), g=37.5)
    assert np.array_equal(u8(pay), qp.ravel()) and np.array_equal(u8(sc), qs)


@pytest.mark.parametrize("R,C", [(1, 1), (130, 8), (255, 7), (300, 17), (4096, 224), (3, 448)])
def test_scale_swizzle(orc, R, C):
    lin = torch.randint(1, 256, (R, C), dtype=torch.uint8)
    say("swizzle", R, C)
    n = (-(-R // 128) * 128) * (-(-C // 4) * 4)
    out, whole = canary_buffer(n)
    mxq.scale_swizzle(lin.to(DEV), out)
    torch.cuda.synchronize()
    assert guard_intact(whole, n)
    assert np.array_equal(u8(out), orc.scale_swizzle(lin.numpy()))


@pytest.mark.parametrize("off", [1, 2, 3])
def test_scale_swizzle_unaligned_linear(orc, off):
    """A linear matrix at a byte offset: 128 columns would take word loads,
    the misaligned base must take the byte path."""
    R, C = 300, 128
    host = torch.randint(0, 256, (R * C + 4,), dtype=torch.int32).to(torch.uint8)
    say("swizzle unaligned", off)
    lin = host.to(DEV)[off:off + R * C].view(R, C)
    got = mxq.scale_swizzle(lin)
    torch.cuda.synchronize()
    assert np.array_equal(u8(got), orc.scale_swizzle(host[off:off + R * C].view(R, C).numpy()))


def test_swizzle_of_linear_equals_swizzled_quant(orc):
    x = (torch.randn(300, 4096) * 0.02).to(torch.bfloat16).to(DEV)
    say("layouts agree")
    _, s_lin = mxq.mx_quant_grouped(mxq.MXFP8, mxq.LINEAR, [x])
    _, s_swz = mxq.mx_quant_grouped(mxq.MXFP8, mxq.SWIZZLED, [x])
    conv = mxq.scale_swizzle(s_lin[0].view(300, 128))
    torch.cuda.synchronize()
    assert torch.equal(conv, s_swz[0])


def _fused_check(orc, T, H, fmt, layout, seed, eps=1e-6, g=37.5, inputs=None):
    x_c, r_c, g_c = workloads.epilogue_inputs(T, H, seed=seed) if inputs is None else inputs
    x, r, gm = x_c.to(DEV), r_c.to(DEV), g_c.to(DEV)
    gs = torch.tensor([g], dtype=torch.float32, device=DEV)
    pw = H if fmt == mxq.MXFP8 else H // 2
    nb = mxq.scale_bytes(T, H, fmt, layout)
    pay, pwh = canary_buffer(T * pw)
    sc, swh = canary_buffer(nb)
    ro, no = torch.empty_like(x), torch.empty_like(x)
    mxq.rmsnorm_quant_fused(x, r, gm, eps, fmt, layout, gs, out=(ro, no, pay.view(T, pw), sc))
    torch.cuda.synchronize()
    assert guard_intact(pwh, T * pw) and guard_intact(swh, nb)
    oro, ono = orc.add_rmsnorm(bf16_bits(x_c), bf16_bits(r_c), bf16_bits(g_c), eps)
    assert np.array_equal(bf16_bits(ro), oro)
    assert bf16_ulp_diff(bf16_bits(no), ono).max() <= 1
    qp, qs = orc.quantize(fmt, layout, bf16_bits(no), g=g)
    assert np.array_equal(u8(pay), qp.ravel()) and np.array_equal(u8(sc), qs)


@pytest.mark.parametrize("eps", [1e-6, 2.0 ** -126])
@pytest.mark.parametrize("fmt", [0, 1])
def test_fused_row_magnitudes(orc, fmt, eps):
    """Rows far from unit scale, inside the range the header states: x and
    residual scaled by 2^53 (|r| up to about 2^56, squares summing to about
    2^120 at H = 7168) down to 2^-80 (squares subnormal or lost, where eps
    decides), with the smallest accepted eps too.  norm_out within 1 ulp,
    the quantized form exact."""
    T, H = 10, 7168
    x_c, r_c, g_c = workloads.epilogue_inputs(T, H, seed=6)
    k = torch.tensor([53.0, 40.0, 0.0, -20.0, -60.0, -63.0, -66.0, -70.0, -80.0, -10.0])
    scale = torch.pow(2.0, k).reshape(T, 1)
    xs = (x_c.float() * scale).to(torch.bfloat16)
    rs = (r_c.float() * scale).to(torch.bfloat16)
    for layout in (mxq.LINEAR, mxq.SWIZZLED):
        say("fused magnitudes, fmt", fmt, "eps", eps, "layout", layout)
        _fused_check(orc, T, H, fmt, layout, seed=0, eps=eps, inputs=(xs, rs, g_c))


@pytest.mark.parametrize("fmt", [0, 1])
def test_fused_narrowest_rows(orc, fmt):
    """The narrowest rows each layout accepts (linear: one or three blocks;
    swizzled: one tile of four scale columns), where most of a row's waves
    hold no column, with T on each side of the launcher's shape switches."""
    block = 32 if fmt == 0 else 16
    cases = [(mxq.LINEAR, block), (mxq.LINEAR, 3 * block), (mxq.SWIZZLED, 4 * block)]
    for T in (1, 3, 300, 2000):
        for layout, H in cases:
            say("fused narrow, fmt", fmt, "layout", layout, "T", T, "H", H)
            _fused_check(orc, T, H, fmt, layout, seed=T + H)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_fused_widths_both_row_splits(orc, fmt, layout):
    """Row widths with ragged 512-column tails, up to the 16384 maximum, on
    both sides of the launcher's switches from sixteen to four waves per row
    (T = 256 linear, 512 swizzled) and from four to two (T = 1536)."""
    for T, H in ((5, 128), (5, 640), (3, 16384), (130, 2176), (256, 640), (257, 2176),
                 (512, 640), (513, 16384), (1536, 640), (2100, 640), (1537, 2176)):
        say("fused widths, fmt", fmt, "layout", layout, "T", T, "H", H)
        _fused_check(orc, T, H, fmt, layout, seed=T + H)


@pytest.mark.parametrize("fmt", [0, 1])
def test_fused_swizzled_partial_bands(orc, fmt):
    """Swizzled one-row units are the live rows only: the live rows of a
    partial last band write its padding (a line's last live row carries the
    zeros of the slots after it; lines with no live row are zeroed by the
    band's units).  Every count of live rows around the line and band
    boundaries, both launch shapes of one-row units (sixteen waves up to
    T = 512, four above), and capped grids; every byte of the canary-filled
    scales against the oracle."""
    for T in (1, 2, 3, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 159, 160,
              161, 255, 256, 257, 300, 511, 512, 513, 600, 1023, 1025):
        say("fused partial band, fmt", fmt, "T", T)
        _fused_check(orc, T, 256, fmt, mxq.SWIZZLED, seed=900 + T)
    try:
        for T, cap in ((1, 1), (5, 2), (40, 3), (200, 7), (700, 8)):
            mxq.set_max_workgroups(cap)
            say("fused partial band, grid cap", cap, "T", T)
            _fused_check(orc, T, 256, fmt, mxq.SWIZZLED, seed=950 + T)
    finally:
        mxq.set_max_workgroups(0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_fused_few_rows_widths(orc, fmt):
    """The one-workgroup-per-row kernel (T = 1 and 17..31, swizzled, H up to
    16 x 512) at row widths of one tile, a partial last wave step (640, 2176),
    and exactly sixteen full steps (8192); 8320 runs the general kernel."""
    for T in (1, 20):
        for H in (128, 640, 2176, 8192, 8320):
            say("fused few rows, fmt", fmt, "T", T, "H", H)
            _fused_check(orc, T, H, fmt, mxq.SWIZZLED, seed=T * 7 + H)


@pytest.mark.parametrize("fmt", [0, 1])
def test_fused_grid_invariance(orc, fmt):
    try:
        for T in (100, 2100):
            for cap in (1, 7):
                mxq.set_max_workgroups(cap)
                say("fused grid cap", cap, "T", T, "fmt", fmt)
                _fused_check(orc, T, 1024, fmt, mxq.SWIZZLED, seed=T)
    finally:
        mxq.set_max_workgroups(0)


def test_empty_activations_through_the_binding():
    """T = 0 through every split form and the fused call: outputs are empty,
    nothing is launched, and no error is raised (a zero-row array from numpy
    has strides (0, 0); the binding must not care)."""
    for H in (256, 7168):
        x = torch.from_numpy(np.zeros((0, H), np.int16)).view(torch.bfloat16).to(DEV)
        g = torch.ones(1, dtype=torch.float32, device=DEV)
        say("empty activation", H)
        for p, s, a in (mxq.nvfp4_quant_split(x, [0, 0], g, mxq.SWIZZLED),
                        mxq.nvfp4_quant_split_row_scaled(x, [0], mxq.LINEAR),
                        mxq.mxfp8_quant_split(x, [0, 0, 0], mxq.SWIZZLED)):
            assert p.numel() == 0 and s.numel() == 0 and a.numel() == 0
        gm = torch.ones(H, dtype=torch.bfloat16, device=DEV)
        for fmt in (0, 1):
            ro, no, p, s = mxq.rmsnorm_quant_fused(x, x, gm, 1e-6, fmt, mxq.SWIZZLED, g)
            assert ro.numel() == no.numel() == p.numel() == s.numel() == 0
    torch.cuda.synchronize()


def test_binding_rejects_small_outputs():
    """Outputs smaller than the call writes are refused before any launch."""
    x = torch.zeros(64, 256, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(1, dtype=torch.float32, device=DEV)
    small = torch.empty(10, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        mxq.nvfp4_quant_split(x, [64], g, mxq.SWIZZLED, payload=small)
    with pytest.raises(ValueError):
        mxq.mxfp8_quant_split(x, [64], mxq.LINEAR, scales=small)
    with pytest.raises(ValueError):
        mxq.nvfp4_quant_split_row_scaled(x, [64], mxq.LINEAR,
                                         row_amax=torch.empty(3, device=DEV))
    r = torch.zeros_like(x)
    gm = torch.ones(256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        mxq.rmsnorm_quant_fused(x, r, gm, out=(torch.empty_like(x), torch.empty_like(x),
                                               small, small))
    with pytest.raises(ValueError):
        mxq.scale_swizzle(torch.zeros(64, 8, dtype=torch.uint8, device=DEV), small)
    with pytest.raises(ValueError):
        mxq.mx_quant_grouped(mxq.MXFP8, mxq.LINEAR, [x], payloads=[small])
    # encode-scale outputs: too small, not contiguous; no sources at all
    with pytest.raises(ValueError):
        mxq.nvfp4_quant_grouped_auto(mxq.SWIZZLED, [x, x], g_out=torch.empty(1, device=DEV))
    with pytest.raises(ValueError):
        mxq.nvfp4_quant_grouped_auto(mxq.SWIZZLED, [x, x],
                                     amax_out=torch.empty(4, device=DEV)[::2])
    with pytest.raises(ValueError):
        mxq.nvfp4_quant_grouped_auto(mxq.SWIZZLED, [])
    # outputs on the host
    with pytest.raises(ValueError):
        mxq.mxfp8_quant_split(x, [64], mxq.LINEAR, payload=torch.empty(64 * 256, dtype=torch.uint8))


# Caller encode scales outside the quotient-table range (g < 2^-117: the
# division path) and scales whose multipliers overflow (flushed), through the
# split and the fused epilogue.
ODD_G = [2.0 ** -149, 12337 * 2.0 ** -149, 2.0 ** -126,
         float(np.nextafter(np.float32(2.0 ** -117), np.float32(0))), 2.0 ** -117,
         2.0 ** 126, float(np.finfo(np.float32).max)]


@pytest.mark.parametrize("g", ODD_G, ids=[v.hex() for v in ODD_G])
def test_split_and_fused_odd_caller_scales(orc, g):
    T, H = 300, 1024
    gen = torch.Generator().manual_seed(91)
    # rows spread over 2^-120 .. 2^120 so that many block codes are met
    x_cpu = (torch.randn(T, H, generator=gen) *
             torch.exp2(torch.linspace(-120, 120, T))[:, None]).to(torch.bfloat16)
    gd = torch.tensor([g], dtype=torch.float32, device=DEV)
    split = [0, 7, 128, 0, 165]
    for layout in (0, 1):
        say("split with caller g", g.hex(), "layout", layout)
        p, s, a, total = run_split(x_cpu.to(DEV), split, gd, layout)
        op, os_, oa = orc.nvfp4_split(bf16_bits(x_cpu), split, float(np.float32(g)), layout)
        assert np.array_equal(u8(p), op.ravel()) and np.array_equal(u8(s), os_)
    xr, rr, gm = workloads.epilogue_inputs(64, H, seed=5)
    say("fused NVFP4 with caller g", g.hex())
    ro, no, fp, fs = mxq.rmsnorm_quant_fused(xr.to(DEV), rr.to(DEV), gm.to(DEV), 1e-6,
                                            mxq.NVFP4, mxq.SWIZZLED, gd)
    torch.cuda.synchronize()
    op, os_ = orc.quantize(orc.NVFP4, orc.SWIZZLED, bf16_bits(no), g=float(np.float32(g)))
    assert np.array_equal(u8(fp), op.ravel()) and np.array_equal(u8(fs), os_)
