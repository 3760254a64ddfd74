"""Pins of the oracle's grouped NVFP4 with encode scales from the data.

The tensor amax against numpy's max over the decoded values (strided rows
included); auto-scaled quantization against the pinned per-tensor
quantization under g = 2688 / amax formed with numpy's fp32 division; a
shared scale slot (gate and up of one expert) takes the larger amax; the
element at the slot's amax encodes as +-6 under the block scale 448.
"""
import numpy as np
import torch

from helpers import bf16_bits


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _tensor(rows, cols, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return bf16_bits((torch.randn(rows, cols, generator=g) * scale).to(torch.bfloat16))


def test_tensor_amax_matches_numpy(orc):
    for seed, (r, c) in enumerate([(1, 16), (7, 48), (130, 96)]):
        x = _tensor(r, c, seed, scale=10.0 ** (seed - 1))
        assert orc.tensor_amax(x) == np.abs(_f32(x)).max()
    x = _tensor(9, 64, 5)
    x[:, 48:] = 0x7F00  # huge values past the first 48 columns are not read
    assert orc.tensor_amax(x, cols=48) == np.abs(_f32(x[:, :48])).max()
    assert orc.tensor_amax(np.zeros((3, 32), np.uint16)) == 0.0
    assert orc.tensor_amax(np.full((3, 32), 0x8000, np.uint16)) == 0.0


def test_auto_equals_per_tensor_with_numpy_scale(orc):
    xs = [_tensor(64, 96, 10 + i, scale=3.0 ** i) for i in range(4)]
    for layout in (orc.LINEAR, orc.SWIZZLED):
        pays, scs, g, amax = orc.quantize_auto(layout, xs)
        for i, x in enumerate(xs):
            a = np.abs(_f32(x)).max()
            gi = np.float32(2688.0) / np.float32(a)
            assert amax[i] == a and g[i] == gi
            p, s = orc.quantize(orc.NVFP4, layout, x, g=float(gi))
            assert np.array_equal(pays[i], p) and np.array_equal(scs[i], s)


def test_shared_slot_takes_the_larger_amax(orc):
    gate, up = _tensor(32, 64, 20, scale=1.0), _tensor(32, 64, 21, scale=5.0)
    down = _tensor(64, 32, 22, scale=0.1)
    pays, scs, g, amax = orc.quantize_auto(orc.LINEAR, [gate, up, down], slots=[0, 0, 1])
    a01 = max(np.abs(_f32(gate)).max(), np.abs(_f32(up)).max())
    assert amax[0] == a01 and amax[1] == np.abs(_f32(down)).max()
    assert g[0] == np.float32(2688.0) / np.float32(a01)
    p, s = orc.quantize(orc.NVFP4, orc.LINEAR, gate, g=float(g[0]))
    assert np.array_equal(pays[0], p) and np.array_equal(scs[0], s)


def test_slot_amax_element_encodes_as_six(orc):
    xs = [_tensor(40, 128, 30 + i, scale=10.0 ** (i - 2)) for i in range(5)]
    pays, scs, g, amax = orc.quantize_auto(orc.LINEAR, xs)
    for i, x in enumerate(xs):
        xf = _f32(x)
        r, j = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
        assert scs[i][r * 8 + j // 16] == 0x7E
        nib = (pays[i][r, j // 2] >> (4 * (j & 1))) & 0xF
        assert nib == (0xF if xf[r, j] < 0 else 0x7)
        assert scs[i].max() == 0x7E
