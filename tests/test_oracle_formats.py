"""Pins of the oracle's element codecs against things other than itself.

* torch's CPU float8_e4m3fn / bfloat16 conversions (round to nearest even,
  sign of zero kept) on the range where they agree with a saturating
  encoder (|v| < 464 for E4M3),
* brute-force nearest-code searches over the code tables (a different
  formulation from the oracle's binade-spacing rounding),
* closed forms for the E8M0 exponent rule.
"""
import numpy as np
import pytest
import torch

from helpers import e4m3_table

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nearest_code(a, mags, maxcode):
    """Brute force: index of the nearest magnitude, ties to the even index,
    saturating at the largest magnitude."""
    a = np.asarray(a, dtype=np.float64)
    idx = np.searchsorted(mags, a, side="left")  # mags[idx-1] < a <= mags[idx]
    hi = np.clip(idx, 0, maxcode)
    lo = np.clip(idx - 1, 0, maxcode)
    dlo = np.abs(a - mags[lo])
    dhi = np.abs(mags[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= mags[maxcode], maxcode, pick)
    return pick.astype(np.uint8)


def brute_e4m3(v):
    mags = e4m3_table()[:127]  # codes 0..126: 0 .. 448, increasing
    assert np.all(np.diff(mags) > 0)
    v = np.asarray(v, dtype=np.float64)
    code = nearest_code(np.abs(v), mags, 126)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def brute_e2m1(v):
    v = np.asarray(v, dtype=np.float64)
    code = nearest_code(np.abs(v), E2M1_MAG, 7)
    return code | np.where(np.signbit(v), 0x8, 0).astype(np.uint8)


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (b >> 7) & 0xFF
    return b[e != 0xFF]


def test_bf16_decode_all_codes(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([orc.bf16_value(b) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    assert np.array_equal(ref[~np.isnan(ref)], mine[~np.isnan(mine)])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(mine[fin]))


def test_bf16_round_matches_torch_rne(orc):
    rng = np.random.default_rng(1)
    # fp32 values (exact in double): torch's fp32 -> bf16 rounding is RNE.
    # Random bit patterns, plus exact midpoints and their neighbours.
    raw = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    base = (rng.integers(0, 0x7F7F, 3000, dtype=np.uint32) << 16)
    mids = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base | 0x18000])
    u = np.concatenate([raw, mids, mids | 0x80000000]).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([orc.bf16_round(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(ref, mine)


def test_e4m3_decode_all_codes(orc):
    ref = e4m3_table()
    mine = np.array([orc.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert mine[0x7E] == 448.0 and mine[0x08] == 2.0**-6 and mine[0x01] == 2.0**-9
    # encode(decode(k)) == k for every non-NaN code
    for k in range(256):
        if not np.isnan(mine[k]):
            assert orc.e4m3_encode(mine[k]) == k


def _e4m3_inputs():
    rng = np.random.default_rng(2)
    mags = e4m3_table()[:127]
    mids = (mags[:-1] + mags[1:]) / 2  # every tie
    pts = np.concatenate([mags, mids])
    f32 = pts.astype(np.float32)
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(-np.inf))
    rnd = np.exp(rng.uniform(np.log(1e-4), np.log(463.0), 200000)).astype(np.float32)
    tiny = rng.uniform(0, 2.0**-8, 20000).astype(np.float32)
    v = np.concatenate([f32, up, dn, rnd, tiny, [0.0, 2.0**-10, 463.99997]]).astype(np.float32)
    v = v[np.abs(v) < 464.0]
    return np.concatenate([v, -v])


def test_e4m3_encode_matches_torch_cast(orc):
    v = _e4m3_inputs()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = orc.e4m3_encode_f32(v)
    assert np.array_equal(ref, mine)


def test_e4m3_encode_matches_brute_force(orc):
    v = _e4m3_inputs()
    big = np.array([448.0, 463.9, 464.0, 500.0, 1e6, 3e38], np.float32)
    v = np.concatenate([v, big, -big])
    assert np.array_equal(brute_e4m3(v), orc.e4m3_encode_f32(v))
    assert orc.e4m3_encode(float("inf")) == 0x7E
    assert orc.e4m3_encode(float("-inf")) == 0xFE


def test_e2m1_codec(orc):
    for c in range(16):
        v = orc.e2m1_value(c)
        assert abs(v) == E2M1_MAG[c & 7] and (c >= 8) == (np.signbit(v))
        assert orc.e2m1_encode(v) == c
    # ties of the pages' packers' format: 0.25->0, 0.75->1, 1.25->1, 1.75->2,
    # 2.5->2, 3.5->4, 5->4; saturation beyond 6
    expect = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.5: 7, 100.0: 7}
    for v, code in expect.items():
        assert orc.e2m1_encode(v) == code
        assert orc.e2m1_encode(-v) == code | 8


def test_e2m1_encode_matches_brute_force(orc):
    rng = np.random.default_rng(3)
    # every fp32 whose top 16 bits fall in [2^-3, 2^4), with the low mantissa
    # half at ties and their neighbours, plus random values and zeros
    hi = np.arange(0x3E00, 0x4180, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    v = u.view(np.float32)
    rnd = rng.uniform(0, 8, 300000).astype(np.float32)
    tiny = np.array([0.0, 1e-45, 1e-38, 0.2499999, 0.25, 0.2500001], np.float32)
    v = np.concatenate([v, rnd, tiny])
    v = np.concatenate([v, -v])
    assert np.array_equal(brute_e2m1(v), orc.e2m1_encode_f32(v))


def test_e8m0_value(orc):
    assert orc.e8m0_value(127) == 1.0
    assert orc.e8m0_value(0) == 2.0**-127
    assert orc.e8m0_value(254) == 2.0**127
    assert np.isnan(orc.e8m0_value(255))


def test_mxfp8_scale_rule_closed_form_all_bf16(orc):
    """Smallest c with amax <= 448 * 2^(c-127), for every finite non-negative
    bf16 amax: equals the integer rule on the bf16 fields, E - 8 + [M > 0x60]
    clamped to [0, 254] (0 for zero and subnormals), and a brute-force
    search written with numpy."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    mine = orc.mxfp8_scale_code_bf16(bits)
    E = (bits >> 7).astype(np.int64)
    M = (bits & 0x7F).astype(np.int64)
    closed = np.where(E == 0, 0, np.clip(E - 8 + (M > 0x60), 0, 254)).astype(np.uint8)
    assert np.array_equal(mine, closed)
    a = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    cs = np.arange(255)
    bound = 448.0 * np.ldexp(1.0, cs - 127)
    brute = np.argmax(a[:, None] <= bound[None, :], axis=1).astype(np.uint8)
    assert np.array_equal(mine, brute)


def test_mxfp8_multiplier_ftz(orc):
    assert orc.mxfp8_multiplier(0) == 0.0  # scale 2^-127 is subnormal in fp32
    assert orc.mxfp8_multiplier(254) == 0.0  # reciprocal 2^-127 is subnormal
    for c in range(1, 254):
        assert orc.mxfp8_multiplier(c) == 2.0 ** (127 - c)


@pytest.mark.slow
def test_mxfp8_element_step_all_bf16_all_codes(orc):
    """For every finite bf16 x and every scale code c reachable with x in the
    block (|x| * 2^(127-c) <= 448): the element byte equals torch's E4M3 cast
    of x * 2^(127-c) (exact in fp32 whenever it is >= 2^-126; below that the
    code is a signed zero either way)."""
    xb = all_finite_bf16()
    xv = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for c in range(1, 254):
        m = 2.0 ** (127 - c)
        y = xv * m
        ok = np.abs(y) <= 448.0
        mine = orc.mxfp8_elements(xb[ok], c)
        ref = torch.from_numpy(y[ok].astype(np.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(mine, ref.view(torch.uint8).numpy()), c
