"""The C ABI driven from C on the GPU: tests/abi_c/gpu_client.c allocates with
the HIP runtime, calls the library directly and compares every output byte
with the oracle (grouped, row-scaled split, fused epilogue)."""
import os
import subprocess

import pytest

from gpu_common import say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_client_on_gpu():
    exe = os.path.join(HERE, "abi_c", "gpu_client")
    if not os.path.exists(exe):  # normally built by __graft_entry__.build()
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "abi_c_build", os.path.join(HERE, "abi_c", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    say("C client")
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "ok:" in p.stdout and ", 0 failed" in p.stdout, p.stdout
