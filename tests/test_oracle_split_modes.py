"""Pins of the oracle's split modes: row-scaled NVFP4 and MXFP8.

Hand-worked rows (tests/golden/row_scaled_rows.txt) fix the per-row encode
scale and the block arithmetic under it; a row-scaled tensor whose rows share
one amax reduces to the tensor-scaled split; in every row-scaled row the
largest element encodes as +-6 under the block scale 448; the MXFP8 split
reduces to the (pinned) per-tensor quantization of each slice, with the
per-expert scale padding sizes worked by hand.
"""
import numpy as np
import pytest
import torch

from helpers import bf16_bits, row_scaled_rows

ROWS = row_scaled_rows()


@pytest.mark.parametrize("case", ROWS, ids=[c["id"] for c in ROWS])
def test_row_scaled_hand_row(orc, case):
    x = np.array(case["x"], np.uint16).reshape(1, 32)
    amax_val = orc.bf16_value(case["amax"])
    assert orc.nvfp4_encode_scale(amax_val) == np.float32(case["g"])
    for layout in (orc.LINEAR, orc.SWIZZLED):
        payload, scales, amax = orc.split(orc.NVFP4, x, [1], layout=layout, row_scaled=True)
        assert list(payload[0]) == case["payload"]
        assert float(amax[0]) == amax_val
        got = [int(scales[orc.sf_offset(0, c, 2, layout)]) for c in range(2)]
        assert got == case["scales"]
        if layout == orc.SWIZZLED:
            assert scales.size == 128 * 4
            mask = np.ones(scales.size, bool)
            mask[[orc.sf_offset(0, c, 2, layout) for c in range(2)]] = False
            assert not scales[mask].any()  # padding rows and columns are zero


def test_row_encode_scale_special_values(orc):
    assert orc.nvfp4_encode_scale(0.0) == 1.0
    assert orc.nvfp4_encode_scale(2688.0) == 1.0
    assert orc.nvfp4_encode_scale(1.0) == 2688.0
    assert orc.nvfp4_encode_scale(7.0) == 384.0
    assert orc.nvfp4_encode_scale(3.0 * 2.0 ** 50) == np.float32(896.0 * 2.0 ** -50)
    # The cap: G = FLT_MAX * 2^-9, the largest g with G / 2^-9 finite.  Below
    # the smallest amax whose quotient 2688 / a (IEEE fp32 division, numpy)
    # stays <= G, every amax gets G, including those whose quotient overflows.
    f32 = np.float32
    fmax = np.finfo(np.float32).max
    G = f32(fmax) / f32(512)
    assert float(G) == float.fromhex("0x1.fffffep+118")
    assert np.isfinite(G / f32(2.0 ** -9))
    a = f32(2688.0 * 512.0 / float(fmax))
    while f32(2688.0) / a <= G:  # walk down to the first capped amax
        a = np.nextafter(a, f32(0))
    for v in (a, a / f32(3), f32(2.0 ** -120), f32(2.0 ** -133), f32(1e-45)):
        assert orc.nvfp4_encode_scale(float(v)) == G, v
    b = np.nextafter(a, f32(1))
    assert orc.nvfp4_encode_scale(float(b)) == f32(2688.0) / b < G
    # no lower bound: the largest bf16 and fp32 amax keep the plain quotient,
    # and the multiplier under it for the largest block scale is still normal
    for v in (f32(255.0 * 2.0 ** 120), f32(fmax)):
        g = orc.nvfp4_encode_scale(float(v))
        assert g == f32(2688.0) / v
        assert f32(g) / f32(448.0) >= np.finfo(np.float32).tiny


def _rows(T, H, seed, scale_spread=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g) * torch.exp(scale_spread * torch.randn(T, 1, generator=g))
    return x.to(torch.bfloat16)


def test_row_scaled_equal_amax_reduces_to_tensor_scaled(orc):
    """Rows that all have the amax A use g_r = fp32(2688 / A) for every row,
    which is the tensor-scaled split with that g."""
    T, H = 300, 96
    x = _rows(T, H, seed=3).float().clamp(-3.0, 3.0)
    x[torch.arange(T), torch.arange(T) % H] = torch.where(torch.arange(T) % 2 == 0, 3.5, -3.5)
    bits = bf16_bits(x.to(torch.bfloat16))
    split = [0, 40, 129, 0, 131]
    g = np.float32(2688.0) / np.float32(3.5)
    for layout in (orc.LINEAR, orc.SWIZZLED):
        pr, sr, ar = orc.split(orc.NVFP4, bits, split, layout=layout, row_scaled=True)
        pt, st, at = orc.split(orc.NVFP4, bits, split, g=g, layout=layout)
        assert np.array_equal(pr, pt) and np.array_equal(sr, st) and np.array_equal(ar, at)
        assert np.all(ar == 3.5)


def test_row_scaled_row_max_encodes_as_six(orc):
    """Under g_r the block holding the row's amax gets scale 448 and the amax
    element itself encodes as E2M1 +-6 (code 7 or 0xF): the scale product and
    the multiplier each carry only a few fp32 roundings, which move neither
    448 nor 6 to another code."""
    T, H = 64, 256
    x = _rows(T, H, seed=4, scale_spread=4.0)
    bits = bf16_bits(x)
    split = [64]
    payload, scales, amax = orc.split(orc.NVFP4, bits, split, layout=orc.LINEAR, row_scaled=True)
    xf = x.float().numpy()
    C = H // 16
    for r in range(T):
        j = int(np.argmax(np.abs(xf[r])))
        assert amax[r] == abs(xf[r, j])
        assert scales[r * C + j // 16] == 0x7E
        nib = (payload[r, j // 2] >> (4 * (j & 1))) & 0xF
        assert nib == (0xF if xf[r, j] < 0 else 0x7)
    assert scales.max() == 0x7E  # never saturated past 448 (no NaN code)


def test_row_scaled_rows_independent_of_split(orc):
    """Row scaling makes every row's payload independent of the split; only
    the scale placement depends on it."""
    T, H = 200, 64
    bits = bf16_bits(_rows(T, H, seed=5, scale_spread=2.0))
    p1, s1, a1 = orc.split(orc.NVFP4, bits, [200], layout=orc.LINEAR, row_scaled=True)
    p2, s2, a2 = orc.split(orc.NVFP4, bits, [7, 0, 150, 43], layout=orc.LINEAR, row_scaled=True)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2) and np.array_equal(a1, a2)


def test_mxfp8_split_sizes_by_hand(orc):
    # cols 64 -> 2 scale columns, padded to 4 when swizzled; rows padded to 128
    split = [0, 1, 129, 0, 3]
    assert [orc.split_scale_offset(split, i, 64, orc.MXFP8, orc.SWIZZLED) for i in range(6)] == \
        [0, 0, 512, 1536, 1536, 2048]
    assert [orc.split_scale_offset(split, i, 64, orc.MXFP8, orc.LINEAR) for i in range(6)] == \
        [0, 0, 2, 260, 260, 266]


def test_mxfp8_split_equals_per_expert(orc):
    split = [0, 1, 127, 128, 129, 0, 3]
    T, H = sum(split), 96
    bits = bf16_bits(_rows(T, H, seed=6))
    for layout in (orc.LINEAR, orc.SWIZZLED):
        payload, scales, amax = orc.split(orc.MXFP8, bits, split, layout=layout)
        o = 0
        for i, m in enumerate(split):
            base = orc.split_scale_offset(split, i, H, orc.MXFP8, layout)
            size = orc.sf_bytes(m, H // 32, layout)
            p_i, s_i = orc.quantize(orc.MXFP8, layout, bits[o:o + m])
            assert np.array_equal(payload[o:o + m], p_i)
            assert np.array_equal(scales[base:base + size], s_i)
            o += m
        assert scales.size == orc.split_scale_offset(split, len(split), H, orc.MXFP8, layout)
        assert np.array_equal(amax, np.abs(bits_f32(bits)).max(axis=1))


def bits_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_split_rejects_bad_modes(orc):
    bits = np.zeros((4, 64), np.uint16)
    with pytest.raises(ValueError):
        orc.split(orc.MXFP8, bits, [4], row_scaled=True)  # row scaling is NVFP4 only
    with pytest.raises(ValueError):
        orc.split(orc.MXFP8, bits[:, :48], [4])  # 48 % 32 != 0
    with pytest.raises(ValueError):
        orc.split(orc.NVFP4, bits, [3])  # rows do not add up
