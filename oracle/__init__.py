"""ctypes front end of the CPU oracle (oracle/mxq_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are its only users.  The GPU package never
imports this module, and this module imports nothing from the GPU package.

bf16 tensors are passed as numpy ``uint16`` bit patterns; payloads and scales
come back as numpy ``uint8`` arrays.
"""
import ctypes
import os

import numpy as np

MXFP8, NVFP4 = 0, 1
LINEAR, SWIZZLED = 0, 1
BLOCK = {MXFP8: 32, NVFP4: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load(path):
    L = ctypes.CDLL(path)
    sig = {
        "orc_bf16_value": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_bf16_round": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_double]),
        "orc_e2m1_value": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_e2m1_encode": (ctypes.c_uint8, [ctypes.c_double]),
        "orc_e8m0_value": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_mxfp8_scale_code": (ctypes.c_uint8, [ctypes.c_double]),
        "orc_mxfp8_multiplier": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_mxfp8_block": (None, [_u16p, ctypes.c_int, _u8p, _u8p]),
        "orc_nvfp4_block": (None, [_u16p, ctypes.c_int, ctypes.c_float, _u8p, _u8p]),
        "orc_sf_cols": (_i64, [_i64, ctypes.c_int]),
        "orc_sf_bytes": (_i64, [_i64, _i64, ctypes.c_int]),
        "orc_sf_offset": (_i64, [_i64, _i64, _i64, ctypes.c_int]),
        "orc_quantize": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _u16p, _i64, _i64, _i64,
                                        ctypes.c_float, _u8p, _u8p]),
        "orc_split_scale_offset": (_i64, [_i64p, ctypes.c_int, ctypes.c_int, _i64,
                                          ctypes.c_int, ctypes.c_int]),
        "orc_nvfp4_split": (ctypes.c_int, [_u16p, _i64, _i64, _i64p, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_int, _u8p, _u8p, _f32p]),
        "orc_split": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _u16p, _i64, _i64, _i64p,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_int, _u8p, _u8p,
                                     _f32p]),
        "orc_nvfp4_encode_scale": (ctypes.c_float, [ctypes.c_float]),
        "orc_tensor_amax": (ctypes.c_float, [_u16p, _i64, _i64, _i64]),
        "orc_add_rmsnorm": (ctypes.c_int, [_u16p, _u16p, _u16p, ctypes.c_float, _i64, _i64,
                                           _u16p, _u16p]),
        "orc_scale_swizzle": (ctypes.c_int, [_u8p, _i64, _i64, _u8p]),
        "orc_e4m3_encode_f32": (None, [_f32p, _i64, _u8p]),
        "orc_e2m1_encode_f32": (None, [_f32p, _i64, _u8p]),
        "orc_mxfp8_scale_code_bf16": (None, [_u16p, _i64, _u8p]),
        "orc_mxfp8_elements": (None, [_u16p, _i64, ctypes.c_uint8, _u8p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = _load(_LIB_PATH)
    return _lib


class using:
    """Context manager: route every call of this module to another build of
    the oracle source (the mutation tests use it to check that the pins
    reject planted mistakes)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        lib()
        self.saved = _lib
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


# ---- scalar rules --------------------------------------------------------
def bf16_value(bits):
    return lib().orc_bf16_value(int(bits))


def bf16_round(v):
    return lib().orc_bf16_round(float(v))


def e4m3_value(code):
    return lib().orc_e4m3_value(int(code))


def e4m3_encode(v):
    return lib().orc_e4m3_encode(float(v))


def e2m1_value(code):
    return lib().orc_e2m1_value(int(code))


def e2m1_encode(v):
    return lib().orc_e2m1_encode(float(v))


def e8m0_value(code):
    return lib().orc_e8m0_value(int(code))


def mxfp8_scale_code(amax):
    return lib().orc_mxfp8_scale_code(float(amax))


def mxfp8_multiplier(code):
    return lib().orc_mxfp8_multiplier(int(code))


def mxfp8_block(x_bits):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.zeros(len(x), np.uint8)
    s = np.zeros(1, np.uint8)
    lib().orc_mxfp8_block(_ptr(x, _u16p), len(x), _ptr(q, _u8p), _ptr(s, _u8p))
    return int(s[0]), q


def nvfp4_block(x_bits, g):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.zeros(len(x) // 2, np.uint8)
    s = np.zeros(1, np.uint8)
    lib().orc_nvfp4_block(_ptr(x, _u16p), len(x), float(g), _ptr(q, _u8p), _ptr(s, _u8p))
    return int(s[0]), q


# ---- layouts -------------------------------------------------------------
def sf_cols(cols, fmt):
    return lib().orc_sf_cols(cols, fmt)


def sf_bytes(rows, n_sf_cols, layout):
    return lib().orc_sf_bytes(rows, n_sf_cols, layout)


def sf_offset(r, c, n_sf_cols, layout):
    return lib().orc_sf_offset(r, c, n_sf_cols, layout)


# ---- whole tensors -------------------------------------------------------
def quantize(fmt, layout, src_bits, cols=None, g=1.0):
    """Quantize one bf16 tensor [rows, ld] (first `cols` columns of each row).

    Returns (payload uint8 [rows, cols or cols/2], scales uint8 [sf_bytes])."""
    src = np.ascontiguousarray(src_bits, dtype=np.uint16)
    rows, ld = src.shape
    cols = ld if cols is None else cols
    C = sf_cols(cols, fmt)
    payload = np.zeros((rows, cols if fmt == MXFP8 else cols // 2), np.uint8)
    scales = np.zeros(sf_bytes(rows, C, layout), np.uint8)
    rc = lib().orc_quantize(fmt, layout, _ptr(src, _u16p), rows, cols, ld, float(g),
                            _ptr(payload, _u8p), _ptr(scales, _u8p))
    if rc != 0:
        raise ValueError("oracle quantize: invalid arguments")
    return payload, scales


def split_scale_offset(split_rows, i, cols, fmt, layout):
    sr = np.ascontiguousarray(split_rows, dtype=np.int64)
    return lib().orc_split_scale_offset(_ptr(sr, _i64p), len(sr), i, cols, fmt, layout)


def nvfp4_split(src_bits, split_rows, g, layout):
    """Returns (payload [T, cols/2], bulk scales, row_amax fp32 [T])."""
    src = np.ascontiguousarray(src_bits, dtype=np.uint16)
    T, cols = src.shape
    sr = np.ascontiguousarray(split_rows, dtype=np.int64)
    total_sf = split_scale_offset(sr, len(sr), cols, NVFP4, layout)
    payload = np.zeros((T, cols // 2), np.uint8)
    scales = np.zeros(total_sf, np.uint8)
    amax = np.zeros(T, np.float32)
    rc = lib().orc_nvfp4_split(_ptr(src, _u16p), T, cols, _ptr(sr, _i64p), len(sr), float(g),
                               layout, _ptr(payload, _u8p), _ptr(scales, _u8p), _ptr(amax, _f32p))
    if rc != 0:
        raise ValueError("oracle split: invalid arguments")
    return payload, scales, amax


def split(fmt, src_bits, split_rows, g=1.0, layout=LINEAR, row_scaled=False):
    """Split quantization in any mode: MXFP8 (g ignored), NVFP4 under one
    encode scale g, or row-scaled NVFP4 (each row under
    nvfp4_encode_scale of its own amax).

    Returns (payload [T, cols or cols/2], bulk scales, row_amax fp32 [T])."""
    src = np.ascontiguousarray(src_bits, dtype=np.uint16)
    T, cols = src.shape
    sr = np.ascontiguousarray(split_rows, dtype=np.int64)
    total_sf = split_scale_offset(sr, len(sr), cols, fmt, layout)
    payload = np.zeros((T, cols if fmt == MXFP8 else cols // 2), np.uint8)
    scales = np.zeros(total_sf, np.uint8)
    amax = np.zeros(T, np.float32)
    rc = lib().orc_split(fmt, int(bool(row_scaled)), _ptr(src, _u16p), T, cols, _ptr(sr, _i64p),
                         len(sr), float(g), layout, _ptr(payload, _u8p), _ptr(scales, _u8p),
                         _ptr(amax, _f32p))
    if rc != 0:
        raise ValueError("oracle split: invalid arguments")
    return payload, scales, amax


def nvfp4_encode_scale(amax):
    return lib().orc_nvfp4_encode_scale(float(amax))


def tensor_amax(src_bits, cols=None):
    src = np.ascontiguousarray(src_bits, dtype=np.uint16)
    rows, ld = src.shape
    return lib().orc_tensor_amax(_ptr(src, _u16p), rows, ld if cols is None else cols, ld)


def quantize_auto(layout, srcs, slots=None, cols=None):
    """Grouped NVFP4 with encode scales from the data: entry i belongs to
    scale slot slots[i] (default: its own); a slot's amax is the max over its
    entries, its encode scale nvfp4_encode_scale(amax), and every entry is
    quantized under its slot's scale.

    Returns (payloads, scales, g [n_slots] fp32, amax [n_slots] fp32)."""
    slots = list(range(len(srcs))) if slots is None else list(slots)
    n_slots = max(slots) + 1
    amax = np.zeros(n_slots, np.float32)
    for s, x in zip(slots, srcs):
        amax[s] = max(amax[s], tensor_amax(x, cols))
    g = np.array([nvfp4_encode_scale(a) for a in amax], np.float32)
    outs = [quantize(NVFP4, layout, x, cols, float(g[s])) for s, x in zip(slots, srcs)]
    return [o[0] for o in outs], [o[1] for o in outs], g, amax


def add_rmsnorm(x_bits, res_bits, gamma_bits, eps):
    """Returns (residual_out, norm_out) as bf16 bit patterns [T, H]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    r = np.ascontiguousarray(res_bits, dtype=np.uint16)
    gm = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
    T, H = x.shape
    ro = np.zeros((T, H), np.uint16)
    no = np.zeros((T, H), np.uint16)
    rc = lib().orc_add_rmsnorm(_ptr(x, _u16p), _ptr(r, _u16p), _ptr(gm, _u16p), float(eps), T, H,
                               _ptr(ro, _u16p), _ptr(no, _u16p))
    if rc != 0:
        raise ValueError("oracle rmsnorm: invalid arguments")
    return ro, no


def scale_swizzle(linear):
    lin = np.ascontiguousarray(linear, dtype=np.uint8)
    rows, C = lin.shape
    out = np.zeros(sf_bytes(rows, C, SWIZZLED), np.uint8)
    if lib().orc_scale_swizzle(_ptr(lin, _u8p), rows, C, _ptr(out, _u8p)) != 0:
        raise ValueError("oracle swizzle: invalid arguments")
    return out


# ---- elementwise helpers ------------------------------------------------
def e4m3_encode_f32(v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib().orc_e4m3_encode_f32(_ptr(v, _f32p), v.size, _ptr(out, _u8p))
    return out


def e2m1_encode_f32(v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib().orc_e2m1_encode_f32(_ptr(v, _f32p), v.size, _ptr(out, _u8p))
    return out


def mxfp8_scale_code_bf16(amax_bits):
    a = np.ascontiguousarray(amax_bits, dtype=np.uint16)
    out = np.zeros(a.shape, np.uint8)
    lib().orc_mxfp8_scale_code_bf16(_ptr(a, _u16p), a.size, _ptr(out, _u8p))
    return out


def mxfp8_elements(x_bits, code):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.zeros(x.shape, np.uint8)
    lib().orc_mxfp8_elements(_ptr(x, _u16p), x.size, int(code), _ptr(out, _u8p))
    return out
