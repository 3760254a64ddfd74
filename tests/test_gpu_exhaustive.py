"""Exhaustive GPU enumerations against the oracle.

* MXFP8: every finite bf16 element x with every scale code c it can meet in
  a block (|x| <= 448 * 2^(c-127)), codes 1..247, plus all-subnormal blocks
  (code 0, the flush-to-zero case).
* NVFP4: every finite non-negative bf16 block maximum, under several encode
  scales g, with the block's other elements drawn below it: this enumerates
  the scale arithmetic (amax/6, times g, E4M3, g/s_q) for every amax.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from gpu_common import say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits_to_dev(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(
        torch.bfloat16).to(DEV)


def _finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def test_mxfp8_all_elements_all_codes(orc):
    xb = _finite_bf16()
    mag = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().abs().numpy()
    blocks = []
    for c in range(1, 248):
        lim = 448.0 * 2.0 ** (c - 127)
        # block maximum with code c: 1.75 * 2^(c-119) is a bf16 value (mantissa 0x60)
        e = c - 119 + 127
        amax = (e << 7) | 0x60 if e <= 254 else 0x7F7F
        xs = xb[mag <= lim]
        n = -(-len(xs) // 31) * 31
        xs = np.concatenate([xs, np.zeros(n - len(xs), np.uint16)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((len(xs), 1), amax, np.uint16), xs], axis=1))
    sub = xb[((xb >> 7) & 0xFF) == 0]  # every subnormal and zero: scale code 0
    n = -(-len(sub) // 32) * 32
    blocks.append(np.concatenate([sub, np.zeros(n - len(sub), np.uint16)]).reshape(-1, 32))
    B = np.concatenate(blocks)
    B = np.concatenate([B, np.zeros((-len(B) % 16, 32), np.uint16)])
    X = B.reshape(-1, 32 * 16)  # 16 blocks per row
    say("mxfp8 exhaustive rows", X.shape)
    x = _bits_to_dev(X)
    pays, scs = mxq.mx_quant_grouped(mxq.MXFP8, mxq.LINEAR, [x])
    torch.cuda.synchronize()
    p, s = orc.quantize(orc.MXFP8, orc.LINEAR, X)
    assert np.array_equal(u8(scs[0]), s)
    assert np.array_equal(u8(pays[0]), p.ravel())
    codes = set(np.unique(s).tolist())
    assert set(range(0, 248)) <= codes


@pytest.mark.parametrize("g", [1.0, 384.0, 2688.0 / 7.3, 1.0 / 3.0, 1e-3, 5e4])
def test_nvfp4_all_block_maxima(orc, g):
    amax = np.arange(0, 0x7F80, dtype=np.uint16)  # every finite non-negative bf16
    rng = np.random.default_rng(int(g * 1000) % 2**31)
    a = torch.from_numpy(amax.view(np.int16)).view(torch.bfloat16).float()
    frac = torch.from_numpy(rng.uniform(-1, 1, (len(amax), 15)).astype(np.float32))
    rest = (a[:, None] * frac).to(torch.bfloat16)
    blk = torch.cat([a[:, None].to(torch.bfloat16), rest], dim=1)
    X = blk.reshape(-1, 16 * 8).contiguous()  # 8 blocks per row
    Xb = X.view(torch.int16).numpy().view(np.uint16)
    say("nvfp4 exhaustive amax, g =", g)
    x = X.to(DEV)
    gs = torch.tensor([g], dtype=torch.float32, device=DEV)
    for layout in (mxq.LINEAR, mxq.SWIZZLED):
        pays, scs = mxq.mx_quant_grouped(mxq.NVFP4, layout, [x], global_scales=gs)
        torch.cuda.synchronize()
        p, s = orc.quantize(orc.NVFP4, layout, Xb, g=float(np.float32(g)))
        assert np.array_equal(u8(scs[0]), s), layout
        assert np.array_equal(u8(pays[0]), p.ravel()), layout
