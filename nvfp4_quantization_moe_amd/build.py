"""Build the HIP library libmxq.so in-tree for gfx950 with hipcc.

    python -m nvfp4_quantization_moe_amd.build        # or build() from Python
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmxq.so")
SOURCES = ["mxq_grouped.hip", "mxq_split.hip", "mxq_fused.hip", "mxq_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # exact arithmetic: IEEE fp32 division/sqrt, denormals kept, no contraction
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def build(out: str = LIB, extra=(), verbose=False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
