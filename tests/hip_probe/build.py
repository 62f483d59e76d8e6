"""Build the cast-math test probe (libcastprobe.so) with the library's own hipcc flags.

Test infrastructure: the probe runs the device functions of the FP8 casts
(fp8_block_scaled_e4m3_amd/csrc/dg_cast_math.h) over large input sets on the GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "cast_math_probe.hip")
LIB = os.path.join(HERE, "libcastprobe.so")


def build() -> str:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from fp8_block_scaled_e4m3_amd.build import HIPCC_FLAGS, hipcc
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([hipcc(), *HIPCC_FLAGS, "-shared", SRC, "-o", tmp], check=True, stdout=subprocess.PIPE,
                   stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
