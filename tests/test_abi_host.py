"""Host-only checks of the C ABI (no GPU needed, no kernel launched).

* libmxq.so loads and exports every function include/mxq.h declares;
* the size helpers agree with the oracle's layout sizes;
* argument validation returns the documented status before any HIP call
  (every case here fails validation, or is a documented no-op).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import _Entry

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")
OK, EINVAL, ESHAPE, EUNSUP, ELAUNCH = 0, 1, 2, 3, 4

pytestmark = pytest.mark.skipif(not os.path.exists(mxq.library_path()),
                                reason="libmxq.so not built")

A = 0x10000  # a 16-byte-aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"mx_quant_grouped", "nvfp4_quant_split", "nvfp4_quant_split_row_scaled",
            "mxfp8_quant_split", "rmsnorm_quant_fused", "scale_swizzle"} <= set(names)
    L = ctypes.CDLL(mxq.library_path())
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = mxq.lib()
    for s in range(5):
        assert len(L.mxq_status_str(s)) > 0
    assert L.mxq_status_str(99) == b"unknown status"


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [0, 1])
def test_scale_bytes_match_oracle(orc, fmt, layout):
    for rows in [0, 1, 31, 32, 127, 128, 129, 3072, 4096]:
        for cols in [32, 64, 96, 512, 768, 1536, 4096, 7168]:
            if cols % (32 if fmt == 0 else 16):
                continue
            C = orc.sf_cols(cols, fmt)
            assert mxq.scale_bytes(rows, cols, fmt, layout) == orc.sf_bytes(rows, C, layout)
    assert mxq.lib().mxq_scale_bytes(4, 48, 0, 0) == -1  # 48 % 32
    assert mxq.lib().mxq_scale_bytes(-1, 64, 0, 0) == -1
    assert mxq.lib().mxq_scale_bytes(4, 64, 2, 0) == -1


@pytest.mark.parametrize("layout", [0, 1])
def test_split_offsets_match_oracle(orc, layout):
    split = [0, 1, 127, 128, 129, 0, 255, 256, 3]
    for i in range(len(split) + 1):
        assert mxq.split_scale_offset(split, i, 7168, 1, layout) == \
            orc.split_scale_offset(split, i, 7168, orc.NVFP4, layout)
    arr = (ctypes.c_int64 * 2)(3, -1)
    assert mxq.lib().mxq_split_scale_offset(arr, 2, 1, 64, 1, 0) == -1


def _grouped(fmt, layout, cols, ents):
    n = len(ents)
    arr = (_Entry * max(n, 1))(*ents)
    return mxq.lib().mx_quant_grouped(fmt, layout, cols, arr, n, None)


def _ent(rows=4, ld=None, src=A, pay=A, sc=A, g=A, cols=64):
    return _Entry(src, pay, sc, g, rows, cols if ld is None else ld)


def test_grouped_validation():
    L = mxq.lib()
    assert L.mx_quant_grouped(0, 0, 64, None, 1, None) == EINVAL
    assert _grouped(0, 0, 64, []) == EINVAL                       # n = 0
    assert _grouped(0, 0, 64, [_ent()] * 17) == EINVAL            # n > 16
    assert _grouped(2, 0, 64, [_ent()]) == EINVAL                 # bad format
    assert _grouped(0, 5, 64, [_ent()]) == EINVAL                 # bad layout
    assert _grouped(0, 0, 48, [_ent(cols=48)]) == ESHAPE          # 48 % 32
    assert _grouped(1, 0, 40, [_ent(cols=40)]) == ESHAPE          # 40 % 16
    assert _grouped(0, 0, 0, [_ent(cols=0)]) == ESHAPE
    assert _grouped(0, 0, 65536, [_ent(cols=65536)]) == ESHAPE    # too wide
    assert _grouped(0, 0, 64, [_ent(rows=-1)]) == EINVAL
    assert _grouped(0, 1, 64, [_ent(rows=(1 << 31) - 127)]) == EINVAL  # padded rows overflow
    assert _grouped(0, 0, 64, [_ent(src=0)]) == EINVAL            # null src
    assert _grouped(0, 0, 64, [_ent(pay=0)]) == EINVAL
    assert _grouped(0, 0, 64, [_ent(sc=0)]) == EINVAL
    assert _grouped(1, 0, 64, [_ent(g=0)]) == EINVAL              # NVFP4 needs g
    assert _grouped(0, 0, 64, [_ent(ld=32)]) == ESHAPE            # ld < cols
    assert _grouped(0, 0, 64, [_ent(ld=68)]) == ESHAPE            # ld % 8
    assert _grouped(0, 0, 64, [_ent(src=A + 2)]) == ESHAPE        # misaligned
    assert _grouped(0, 0, 64, [_ent(pay=A + 8)]) == ESHAPE
    assert _grouped(0, 1, 64, [_ent(sc=A + 4)]) == ESHAPE         # swizzled scales
    assert _grouped(0, 0, 64, [_ent(), _ent(src=0)]) == EINVAL    # any bad entry
    # entries with no rows are a no-op (nothing launched)
    assert _grouped(0, 1, 64, [_ent(rows=0, src=0, pay=0, sc=0)]) == OK


def _batch(ents, per=16, flags=0, fmt=0, layout=1, cols=64):
    arr = (_Entry * max(len(ents), 1))(*ents)
    return mxq.lib().mx_quant_grouped_batch(fmt, layout, cols, arr, len(ents), per, flags, None)


def test_grouped_batch_validation():
    """Every batch of a multi-launch call is checked before the first launch:
    a bad entry in the last batch is refused with no launch (on this machine
    a launch could only fail, so EINVAL shows the check came first)."""
    ents = [_ent() for _ in range(40)]
    assert _batch([]) == EINVAL                                   # no entries
    assert _batch(ents, per=0) == EINVAL
    assert _batch(ents, per=17) == EINVAL
    assert _batch(ents, flags=2) == EINVAL                        # unknown flag
    assert _batch(ents, flags=3) == EINVAL
    assert _batch(ents, fmt=2) == EINVAL
    assert _batch(ents[:39] + [_ent(src=0)]) == EINVAL            # last batch
    assert _batch(ents[:33] + [_ent(ld=60)] + ents[34:], per=5) == ESHAPE
    assert _batch([_ent(rows=0, src=0, pay=0, sc=0)] * 20, flags=1) == OK  # no rows: no launch
    assert mxq.lib().mx_quant_grouped_batch(0, 1, 64, None, 3, 16, 0, None) == EINVAL


def _split(split, T=None, cols=64, src=A, g=A, pay=A, sc=A, amax=A, layout=1):
    T = sum(split) if T is None else T
    arr = (ctypes.c_int64 * max(len(split), 1))(*split)
    return mxq.lib().nvfp4_quant_split(src, T, cols, arr, len(split), g, pay, sc, amax, layout,
                                       None)


def test_split_validation():
    assert _split([3, 4], T=8) == EINVAL           # sum != rows
    assert _split([3, -1, 4], T=6) == EINVAL       # negative split
    assert _split([]) == OK                         # no splits, no rows: no launch
    assert _split([], T=3) == EINVAL                # no splits cannot hold rows
    L = mxq.lib()
    assert L.nvfp4_quant_split(A, 0, 64, None, 0, A, A, A, A, 1, None) == OK
    assert L.nvfp4_quant_split(A, 0, 64, None, 2, A, A, A, A, 1, None) == EINVAL
    assert L.mxq_split_scale_offset(None, 0, 0, 64, 1, 1) == 0
    assert L.mxq_split_scale_offset(None, 1, 0, 64, 1, 1) == -1
    assert _split([4], cols=40) == ESHAPE
    assert _split([4], cols=32768) == ESHAPE
    assert _split([4], layout=3) == EINVAL
    assert _split([4], src=0) == EINVAL
    assert _split([4], g=0) == EINVAL
    assert _split([4], src=A + 4) == ESHAPE
    assert _split([4], sc=A + 1, layout=1) == ESHAPE
    assert _split([0, 0, 0], src=0, pay=0, sc=0, g=0) == OK   # all empty: no launch


def _split_rows(split, T=None, cols=64, src=A, pay=A, sc=A, amax=A, layout=1):
    T = sum(split) if T is None else T
    arr = (ctypes.c_int64 * max(len(split), 1))(*split)
    return mxq.lib().nvfp4_quant_split_row_scaled(src, T, cols, arr, len(split), pay, sc, amax,
                                                  layout, None)


def _split_mx(split, T=None, cols=64, src=A, pay=A, sc=A, amax=A, layout=1):
    T = sum(split) if T is None else T
    arr = (ctypes.c_int64 * max(len(split), 1))(*split)
    return mxq.lib().mxfp8_quant_split(src, T, cols, arr, len(split), pay, sc, amax, layout, None)


def test_split_modes_validation():
    for f in (_split_rows, _split_mx):
        assert f([3, 4], T=8) == EINVAL
        assert f([3, -1, 4], T=6) == EINVAL
        assert f([]) == OK
        assert f([], T=2) == EINVAL
        assert f([4], layout=2) == EINVAL
        assert f([4], cols=32768) == ESHAPE
        assert f([4], src=0) == EINVAL
        assert f([4], pay=0) == EINVAL
        assert f([4], pay=A + 4) == ESHAPE
        assert f([4], sc=A + 2) == ESHAPE
        assert f([0, 0], src=0, pay=0, sc=0, amax=0) == OK
    assert _split_rows([4], cols=40) == ESHAPE       # 40 % 16
    assert _split_rows([4], cols=48, amax=0) == EINVAL  # row amax is required
    assert _split_mx([4], cols=48) == ESHAPE          # 48 % 32
    assert _split_mx([4], amax=0, src=0) == EINVAL    # row amax optional, src is not


@pytest.mark.parametrize("layout", [0, 1])
def test_mxfp8_split_offsets_match_oracle(orc, layout):
    split = [0, 1, 127, 128, 129, 0, 255, 3]
    for i in range(len(split) + 1):
        assert mxq.split_scale_offset(split, i, 7168, 0, layout) == \
            orc.split_scale_offset(split, i, 7168, orc.MXFP8, layout)


def _fused(fmt=0, layout=1, T=4, H=256, eps=1e-6, x=A, g=0):
    return mxq.lib().rmsnorm_quant_fused(fmt, layout, x, A, A, eps, T, H, g, A, A, A, A, None)


def test_fused_validation():
    assert _fused(eps=0.0) == EINVAL
    assert _fused(eps=-1.0) == EINVAL
    assert _fused(eps=float("nan")) == EINVAL
    assert _fused(eps=float("inf")) == EINVAL
    assert _fused(eps=2.0 ** -127) == EINVAL        # subnormal eps
    assert _fused(eps=2.0 ** -126, T=0) == OK       # the smallest normal is accepted
    assert _fused(T=-1) == EINVAL
    assert _fused(T=(1 << 31) - 127) == EINVAL      # padded rows must index as int32
    assert _fused(fmt=3) == EINVAL
    assert _fused(H=96) == ESHAPE                   # MXFP8 swizzled: 3 scale cols pad
    assert _fused(H=48) == ESHAPE                   # 48 % 32
    assert _fused(fmt=1, H=96) == ESHAPE            # NVFP4 swizzled: 6 scale cols pad
    assert _fused(H=32768) == ESHAPE
    assert _fused(x=0) == EINVAL
    assert _fused(fmt=1, H=128, g=0) == EINVAL      # NVFP4 needs g
    assert _fused(x=A + 8) == ESHAPE
    assert _fused(T=0, x=0) == OK                   # no rows: no launch


def test_swizzle_validation():
    L = mxq.lib()
    assert L.scale_swizzle(A, 4, 0, A, None) == EINVAL
    assert L.scale_swizzle(A, -1, 4, A, None) == EINVAL
    assert L.scale_swizzle(0, 4, 4, A, None) == EINVAL
    assert L.scale_swizzle(A, 4, 4, A + 4, None) == ESHAPE
    assert L.scale_swizzle(0, 0, 4, 0, None) == OK
    assert L.scale_swizzle(A, 1 << 40, 4, A, None) == EINVAL     # rows < 2^40
    assert L.scale_swizzle(A, 4, 1 << 31, A, None) == EINVAL     # sf_cols < 2^31


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mxq.mx_quant_grouped(mxq.MXFP8, mxq.LINEAR, [x])
    with pytest.raises(ValueError):
        mxq.scale_swizzle(torch.zeros(4, 4, dtype=torch.uint8))


def _auto(ents, slots=None, n_slots=None, g=A, am=A, layout=1, cols=64):
    n = len(ents)
    arr = (_Entry * max(n, 1))(*ents)
    sl = None if slots is None else (ctypes.c_int * len(slots))(*slots)
    ns = n if n_slots is None else n_slots
    return mxq.lib().nvfp4_quant_grouped_auto(layout, cols, arr, n, sl, ns, g, am, None)


def test_grouped_auto_validation():
    e = _ent(g=0)  # entries' own global_scale is not used
    assert _auto([e], n_slots=0) == EINVAL
    assert _auto([e] * 2, n_slots=17, slots=[0, 0]) == EINVAL
    assert _auto([e] * 3, n_slots=2) == EINVAL             # no slot map: one slot per entry
    assert _auto([e] * 2, slots=[0, 2], n_slots=2) == EINVAL  # slot out of range
    assert _auto([e] * 2, slots=[0, -1], n_slots=2) == EINVAL
    assert _auto([e], g=0) == EINVAL
    assert _auto([e], am=0) == EINVAL
    assert _auto([e], g=A + 2) == ESHAPE
    assert _auto([e], am=A + 1) == ESHAPE
    assert _auto([e], cols=40) == ESHAPE                   # 40 % 16
    assert _auto([e] * 17, n_slots=16, slots=[0] * 17) == EINVAL
    assert _auto([_ent(src=0)]) == EINVAL


def test_header_compiles_as_c99_and_links(tmp_path):
    """include/mxq.h is a C header: a C99 client compiled with gcc links the
    library and sees the documented sizes and statuses."""
    import subprocess
    src = os.path.join(ROOT, "tests", "abi_c", "check_abi.c")
    exe = str(tmp_path / "check_abi")
    libdir = os.path.dirname(mxq.library_path())
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"), src, "-o", exe,
                    "-L", libdir, "-l:libmxq.so", "-Wl,-rpath," + libdir], check=True)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = libdir + ":/opt/rocm/lib:" + env.get("LD_LIBRARY_PATH", "")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "ok: 0 failed" in p.stdout


def test_binding_per_call_cap():
    """The per-call expert cap: values outside 1..16 raise before any tensor is
    looked at (0 and negatives included); 1 is the one-launch-per-expert path."""
    for bad in (0, -1, 17):
        with pytest.raises(ValueError):
            mxq.mx_quant_grouped(0, 0, [], max_per_launch=bad)
        with pytest.raises(ValueError):
            mxq.GroupedCall(0, 0, [], max_per_launch=bad)
    assert mxq.mx_quant_grouped(0, 0, [], max_per_launch=1) == ([], [])
