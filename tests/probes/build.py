"""Build the matrix-core probe library (libprobe.so) next to this file:

    python tests/probes/build.py
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8_mfma_probe.hip")
LIB = os.path.join(HERE, "libprobe.so")


def build() -> str:
    tmp = LIB + ".tmp"
    r = subprocess.run(["hipcc", "-O2", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the probe:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
