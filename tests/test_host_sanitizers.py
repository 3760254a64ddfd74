"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised in a child Python process that preloads its
compiler's ASan runtime (it must come before every other library):
  * the oracle (plain C) with -fsanitize=address,undefined, running every
    entry point on small ragged shapes; its outputs must equal those of the
    normal build;
  * the C library with the sanitizers on its host code only (argument
    validation, size and offset arithmetic; device code is built as usual);
    the validation tests of test_abi_host.py run against it.  No kernel is
    launched.
A report from either sanitizer aborts the child with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN = _runtime("libasan.so")
# hipcc is clang: its instrumented host code needs clang's own runtime
CLANG_ASAN = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
if not os.path.exists(CLANG_ASAN):
    r = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    CLANG_ASAN = r.stdout.strip()


def _child(script, runtime):
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    return subprocess.run([sys.executable, "-c", script], env=env, capture_output=True,
                          text=True, timeout=600)


ORACLE_SCRIPT = r"""
import hashlib
import numpy as np
import oracle

def digest():
    h = hashlib.sha256()
    rng = np.random.default_rng(7)
    def bits(r, c):
        x = (rng.standard_normal((r, c)) * np.exp(rng.standard_normal((r, 1)))).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    for fmt, cols in ((0, 96), (1, 48), (1, 16), (0, 32)):
        for layout in (0, 1):
            for rows in (1, 5, 130):
                p, s = oracle.quantize(fmt, layout, bits(rows, cols), g=37.5)
                h.update(p.tobytes()); h.update(s.tobytes())
    for fmt, rs in ((1, False), (1, True), (0, False)):
        for layout in (0, 1):
            split = [0, 3, 1, 0, 140, 2]
            p, s, a = oracle.split(fmt, bits(sum(split), 64), split, g=11.0, layout=layout,
                                   row_scaled=rs)
            h.update(p.tobytes()); h.update(s.tobytes()); h.update(a.tobytes())
    srcs = [bits(r, 32) for r in (3, 0, 129)]
    p, s, g, am = oracle.quantize_auto(1, srcs, [0, 1, 0], 32)
    for t in list(p) + list(s) + [g, am]:
        h.update(np.ascontiguousarray(t).tobytes())
    ro, no = oracle.add_rmsnorm(bits(3, 128), bits(3, 128), bits(1, 128).ravel(), 1e-6)
    h.update(ro.tobytes()); h.update(no.tobytes())
    h.update(oracle.scale_swizzle(np.arange(5 * 7, dtype=np.uint8).reshape(5, 7)).tobytes())
    h.update(repr(float(oracle.tensor_amax(bits(4, 64)))).encode())
    return h.hexdigest()

plain = digest()
with oracle.using(SAN_LIB):
    sanitized = digest()
print("digests", plain, sanitized)
assert plain == sanitized
"""


@pytest.mark.skipif(ASAN is None, reason="gcc's ASan runtime is not installed")
def test_oracle_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    lib = obuild.build(str(tmp_path / "liboracle_san.so"), extra=SAN)
    r = _child(f"SAN_LIB = {lib!r}\n" + ORACLE_SCRIPT, ASAN)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "digests" in r.stdout


ABI_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, ROOT + "/tests")
import nvfp4_quantization_moe_amd as mxq
mxq._LIB_PATH = SAN_LIB
mxq._lib = None
L = mxq.lib()
import test_abi_host as t
for name in ("test_grouped_validation", "test_split_validation", "test_split_modes_validation",
             "test_fused_validation", "test_swizzle_validation", "test_grouped_auto_validation",
             "test_status_strings"):
    getattr(t, name)()
# size and offset arithmetic over many shapes, edge values included
for fmt in (0, 1):
    for layout in (0, 1):
        for rows in (0, 1, 127, 128, 129, 1 << 20):
            for cols in (16, 32, 48, 64, 7168, 16384, 1 << 30):
                L.mxq_scale_bytes(rows, cols, fmt, layout)
        split = [0, 1, 127, 128, 129, 0, 255, 3]
        arr = (ctypes.c_int64 * len(split))(*split)
        for i in range(-1, len(split) + 2):
            L.mxq_split_scale_offset(arr, len(split), i, 7168, fmt, layout)
for s in range(-2, 8):
    L.mxq_status_str(s)
print("abi ok")
"""


@pytest.mark.skipif(not os.path.exists(CLANG_ASAN), reason="clang's ASan runtime is not installed")
def test_abi_host_code_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from nvfp4_quantization_moe_amd import build as B
    out = str(tmp_path / "libmxq_host_san.so")
    # every sanitizer flag is scoped to the host compilation
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    B.build(out, extra=host_san + ["-shared-libsan"])
    r = _child(f"ROOT = {ROOT!r}\nSAN_LIB = {out!r}\n" + ABI_SCRIPT, CLANG_ASAN)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "abi ok" in r.stdout
