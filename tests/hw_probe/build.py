"""Build the test-only conversion probe (cvt_probe.hip) into libcvtprobe.so
with the library's own device flags.  Test infrastructure: the library never
loads it."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "cvt_probe.hip")
OUT = os.path.join(HERE, "libcvtprobe.so")


def build(out: str = OUT) -> str:
    sys.path.insert(0, ROOT)
    from nvfp4_quantization_moe_amd.build import FLAGS, HIPCC
    subprocess.run([HIPCC, *FLAGS, SRC, "-o", out + ".tmp"], check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
