"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the GPU library never links or loads this file's output.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxq_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

# Strict IEEE arithmetic: no fast-math, no FMA contraction, SSE binary32/64.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror"]


def build(out: str = OUT, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
