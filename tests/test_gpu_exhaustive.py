"""Exhaustive GPU enumerations against the oracle.

* The two hardware conversions of the NVFP4 path (fp32 -> E2M1 elements,
  fp32 -> E4M3 block scale), each over every non-negative fp32 bit pattern
  (zero, every subnormal, every normal, +inf) with the sign mirrored, through
  the test-only probe in tests/hw_probe: the step patterns it records must be
  the oracle's.
* MXFP8: every finite bf16 element x with every scale code c it can meet in
  a block (|x| <= 448 * 2^(c-127)), codes 1..247, plus all-subnormal blocks
  (code 0, the flush-to-zero case).
* NVFP4 through the library: for each encode scale g of a set that spans the
  quotient-table range, its edges and the division path below it, and for
  every E4M3 block-scale code the g can reach, every finite bf16 element the
  block can hold (both signs, subnormals and signed zeros included), so every
  fp32 product x * m the element step meets at those multipliers; every
  finite bf16 block maximum under 256 more encode scales drawn over the whole
  positive finite fp32 range; and blocks whose elements sit at, and one bf16
  step either side of, each E2M1 rounding boundary.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from gpu_common import HOST_THREADS, par_map, par_quantize, say, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"
HERE = os.path.dirname(os.path.abspath(__file__))

F32 = np.float32
FLT_MAX = float(np.finfo(np.float32).max)
G_CAP = float.fromhex("0x1.fffffep+118")   # the encode-scale cap, FLT_MAX * 2^-9
TABLE_MIN = 2.0 ** -117                     # smallest g of the quotient-table path


def _bits_to_dev(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(
        torch.bfloat16).to(DEV)


def _finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def _bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).double().numpy()


# ---- the hardware conversions, through the probe ---------------------------
def _probe():
    so = os.path.join(HERE, "hw_probe", "libcvtprobe.so")
    if not os.path.exists(so):  # normally built by __graft_entry__.build()
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "hw_probe_build", os.path.join(HERE, "hw_probe", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    L = ctypes.CDLL(so)
    for fn in (L.probe_fp4_steps, L.probe_fp8_steps):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return L


def _oracle_steps(enc, last_code):
    """Smallest non-negative fp32 pattern whose code is >= c, for c = 1 ..
    last_code (the oracle's encoders are non-decreasing in the value)."""
    steps = []
    for c in range(1, last_code + 1):
        lo, hi = 0, 0x7F800000
        while lo < hi:
            mid = (lo + hi) // 2
            if enc(np.array([mid], np.uint32).view(np.float32))[0] >= c:
                hi = mid
            else:
                lo = mid + 1
        steps.append((lo, c, c - 1))
    return steps


def _run_probe(fn, cap=512):
    out = torch.zeros(4 + 2 * cap, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert fn(out.data_ptr(), cap, stream) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32)
    n = int(o[0])
    assert n <= cap
    steps = sorted((int(o[4 + 2 * k]), int(o[5 + 2 * k]) & 0xFF, int(o[5 + 2 * k]) >> 8)
                   for k in range(n))
    return steps, int(o[1]), int(o[2])


def test_e2m1_conversion_every_fp32(orc):
    say("probe: fp32 -> E2M1 over every non-negative fp32 pattern")
    steps, sign_bad, slot_bad = _run_probe(_probe().probe_fp4_steps)
    assert steps == _oracle_steps(orc.e2m1_encode_f32, 7)
    assert sign_bad == 0 and slot_bad == 0
    # the saturation end: +inf and the largest finite value encode as 6
    assert orc.e2m1_encode(FLT_MAX) == 7


def test_e4m3_scale_conversion_every_fp32(orc):
    say("probe: fp32 -> E4M3 (min(s, 448)) over every non-negative fp32 pattern")
    steps, _, _ = _run_probe(_probe().probe_fp8_steps)
    assert steps == _oracle_steps(orc.e4m3_encode_f32, 0x7E)


# ---- MXFP8 -------------------------------------------------------------------
def test_mxfp8_all_elements_all_codes(orc):
    xb = _finite_bf16()
    mag = np.abs(_bf16_values(xb))
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
    p, s = par_quantize(orc, orc.MXFP8, orc.LINEAR, X)
    assert np.array_equal(u8(scs[0]), s)
    assert np.array_equal(u8(pays[0]), p.ravel())
    codes = set(np.unique(s).tolist())
    assert set(range(0, 248)) <= codes


# ---- NVFP4 -------------------------------------------------------------------
def _nvfp4_check(orc, X, gs, layouts=(mxq.LINEAR,), what=""):
    """Quantize the bf16 bits X_i [rows_i, 128] under encode scales gs (one
    grouped entry each, up to 16 per call) and compare every byte with the
    oracle, in every layout given.  Returns the oracle's scale bytes."""
    out_scales = []
    for layout in layouts:
        for b in range(0, len(X), 16):
            xs = [_bits_to_dev(x) for x in X[b:b + 16]]
            g = torch.tensor(gs[b:b + 16], dtype=torch.float32, device=DEV)
            pays, scs = mxq.mx_quant_grouped(mxq.NVFP4, layout, xs, global_scales=g)
            torch.cuda.synchronize()
            want = par_map(lambda i: orc.quantize(orc.NVFP4, layout, X[i], g=float(gs[i])),
                           range(b, min(b + 16, len(X))))
            for j, (p, s) in enumerate(want):
                i = b + j
                assert np.array_equal(u8(scs[j]), s), (what, "scales", layout, gs[i].hex())
                assert np.array_equal(u8(pays[j]), p.ravel()), (what, "payload", layout,
                                                                 gs[i].hex())
                if layout == layouts[0]:
                    out_scales.append(s)
    return out_scales


def _rows128(blocks):
    """[n, 16] blocks -> [ceil(n / 8), 128] rows (8 blocks per row, zero padded)."""
    blocks = np.concatenate([blocks, np.zeros((-len(blocks) % 8, 16), np.uint16)])
    return np.ascontiguousarray(blocks.reshape(-1, 128))


def _bf16_near(v):
    """Nearest bf16 bits to the positive float64 values v (0 where none)."""
    t = torch.from_numpy(np.asarray(v, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


E4M3_POS = np.array([float(np.ldexp(m, -9)) if e == 0 else float(np.ldexp(8 + m, e - 10))
                     for e in range(16) for m in range(8)])[:0x7F]  # codes 0 .. 0x7E


def _every_code_blocks(g):
    """For every E4M3 code k >= 1 whose block maximum 6 * dec(k) / g is a
    finite bf16 value a_k, and for the largest bf16 value: blocks [a, then 15
    of the finite bf16 values x with |x| <= a, both signs], covering all of
    them.  Returns the blocks and the codes whose a_k is a normal bf16 (those
    must all be reached)."""
    xb = _finite_bf16()
    mag = np.abs(_bf16_values(xb))
    blocks, must, seen = [], set(), set()
    for k in range(1, 0x80):
        if k == 0x7F:  # the largest bf16 block maximum, whatever code it gets
            a_bits = np.uint16(0x7F7F)
        else:
            target = 6.0 * E4M3_POS[k] / g
            if not (0.0 < target < 3.3e38):
                continue
            a_bits = _bf16_near([target])[0]
        a = _bf16_values(np.array([a_bits], np.uint16))[0]
        if a == 0.0 or not np.isfinite(a) or int(a_bits) in seen:
            continue
        seen.add(int(a_bits))
        if a >= 2.0 ** -126 and k < 0x7F:
            must.add(k)
        xs = xb[mag <= a]
        n = -(-len(xs) // 15) * 15
        xs = np.concatenate([xs, np.zeros(n - len(xs), np.uint16)]).reshape(-1, 15)
        blocks.append(np.concatenate([np.full((len(xs), 1), a_bits, np.uint16), xs], axis=1))
    return np.concatenate(blocks), must


EVERY_G = {
    "one": 1.0,
    "384": 384.0,
    "2688_over_7.3": float(F32(2688.0 / 7.3)),
    "third": float(F32(1.0 / 3.0)),
    "2^-100": 2.0 ** -100,
    "2^100": 2.0 ** 100,
    "table_min_2^-117": TABLE_MIN,
    "g_of_bf16_max": float(F32(2688.0) / F32(255.0 * 2.0 ** 120)),
    "g_of_2^127": float(F32(2688.0) / F32(2.0 ** 127)),
    "cap": G_CAP,
    "below_table_min": float(np.nextafter(F32(TABLE_MIN), F32(0))),
    "flt_min": 2.0 ** -126,
    "subnormal_12337x2^-149": 12337 * 2.0 ** -149,
    "2^126": 2.0 ** 126,
    "flt_max": FLT_MAX,
}


@pytest.mark.parametrize("gname", list(EVERY_G))
def test_nvfp4_every_element_every_code(orc, gname):
    g = EVERY_G[gname]
    blocks, must = _every_code_blocks(g)
    X = _rows128(blocks)
    say("nvfp4 every element x every code, g =", gname, g.hex(), X.shape)
    layouts = (mxq.LINEAR, mxq.SWIZZLED) if gname in ("one", "cap") else (mxq.LINEAR,)
    (s,) = _nvfp4_check(orc, [X], np.array([g], np.float32), layouts, gname)
    assert must <= set(np.unique(s).tolist())


def _many_g(n, seed):
    """n encode scales: bit patterns drawn uniformly over the positive finite
    fp32 range (every binade and the subnormals alike), plus the edges."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(1, 0x7F7FFFFF, n - 8, dtype=np.uint32, endpoint=True)
    edges = [1, 0x00800000, float_bits(TABLE_MIN) - 1, float_bits(TABLE_MIN),
             float_bits(G_CAP), float_bits(G_CAP) + 1, 0x7F7FFFFF, float_bits(1.0)]
    return np.concatenate([bits, np.array(edges, np.uint32)]).view(np.float32)


def float_bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def test_nvfp4_all_block_maxima_256_scales(orc):
    """Every finite non-negative bf16 block maximum, each block with 15
    elements drawn below it, under 256 encode scales over the whole positive
    finite fp32 range (the table path, the division path, subnormal g, and
    scales whose multipliers overflow)."""
    gs = _many_g(256, seed=11)
    amax = np.arange(0, 0x7F80, dtype=np.uint16)
    a = torch.from_numpy(amax.view(np.int16)).view(torch.bfloat16).float()
    X = []
    for i in range(len(gs)):
        gen = torch.Generator().manual_seed(100 + i)
        frac = torch.rand(len(amax), 15, generator=gen) * 2 - 1
        rest = (a[:, None] * frac).to(torch.bfloat16)
        blk = torch.cat([a[:, None].to(torch.bfloat16), rest], dim=1)
        X.append(_rows128(blk.view(torch.int16).numpy().view(np.uint16)))
    say("nvfp4 all amax under", len(gs), "encode scales, host threads", HOST_THREADS)
    _nvfp4_check(orc, X, gs, (mxq.LINEAR,), "many-g")


@pytest.mark.parametrize("seed", [0, 1])
def test_nvfp4_e2m1_boundaries(orc, seed):
    """For every finite bf16 block maximum, blocks whose elements are the
    bf16 values nearest to t / m (and one bf16 step below and above) for each
    E2M1 rounding boundary t in 0.25 .. 5, both signs, where m is the block's
    multiplier: products at, and next to, every boundary, under 16 encode
    scales (table path; the multiplier is computed here in fp32 from the
    formats, as input preparation)."""
    gs = _many_g(24, seed=50 + seed)
    gs = gs[(gs >= TABLE_MIN) & (gs <= 2.0 ** 100)][:16]
    thresholds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    av = _bf16_values(amax_bits)
    X = []
    for g in gs:
        with np.errstate(over="ignore"):  # s overflows to inf where a * g is huge
            s = F32(F32(av.astype(np.float32)) / F32(6.0)) * F32(g)  # numpy fp32 roundings
        code = orc.e4m3_encode_f32(np.minimum(s, F32(448.0)))
        sq = E4M3_POS[code].astype(np.float32)
        with np.errstate(divide="ignore", over="ignore"):
            m = np.where(sq > 0, F32(g) / np.where(sq > 0, sq, F32(1)), F32(0))
        live = (m > 0) & np.isfinite(m)
        rows = []
        for off in (-1, 0, 1):  # bf16 steps around the nearest value
            xt = _bf16_near(np.outer(1.0 / m[live].astype(np.float64), thresholds))
            xt = np.where(xt == 0, 0, xt.astype(np.int32) + off).astype(np.uint16)
            xt = np.minimum(xt & 0x7FFF, 0x7F7F)
            # keep every element at or below its block maximum
            xt = np.minimum(xt, amax_bits[live][:, None])
            am = amax_bits[live][:, None]
            rows.append(np.concatenate([am, xt, xt | 0x8000, am | 0x8000], axis=1))
        X.append(_rows128(np.concatenate(rows)))
    say("nvfp4 E2M1 boundaries under", len(gs), "encode scales")
    _nvfp4_check(orc, X, np.array(gs, np.float32), (mxq.LINEAR,), "boundaries")
