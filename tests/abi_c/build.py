"""Build the C99 GPU client of the C ABI (gpu_client.c) with gcc.

It links the HIP library (nvfp4_quantization_moe_amd/libmxq.so), the oracle
(oracle/liboracle.so; test infrastructure) and the HIP runtime; both in-tree
libraries are found relative to the executable, so the tree can move.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "gpu_client.c")
OUT = os.path.join(HERE, "gpu_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = OUT) -> str:
    rpath = "$ORIGIN/../../nvfp4_quantization_moe_amd:$ORIGIN/../../oracle:" + ROCM + "/lib"
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           "-I", os.path.join(ROCM, "include"), SRC, "-o", out + ".tmp",
           "-L", os.path.join(ROOT, "nvfp4_quantization_moe_amd"), "-l:libmxq.so",
           "-L", os.path.join(ROOT, "oracle"), "-l:liboracle.so",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + rpath]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
