"""Sanitizer builds of the host code, for tests/test_host_sanitizers.py:

- abi_check: tests/host_check/abi_driver.cpp linked with the library's host
  code (sage_api.hip) built with AddressSanitizer and UndefinedBehaviorSanitizer
  for the host only, and the kernel objects of the normal build;
- liboracle_san.so: oracle/oracle.c with both sanitizers (gcc).

Outputs go to tests/host_check/_build/.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
PKG = os.path.join(ROOT, "bit_quantized_attention_02_amd")
CSRC = os.path.join(PKG, "csrc")
# the sanitizers instrument host code only (each flag behind -Xarch_host)
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"


def _package_build():
    spec = importlib.util.spec_from_file_location("_sage_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def build_abi_check() -> str:
    os.makedirs(OUT, exist_ok=True)
    pb = _package_build()
    objs = []
    for src in ("prep.hip", "attn_fwd.hip", "attn_decode.hip"):
        obj = os.path.join(pb.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(CSRC, src)):
            obj = pb._compile(src)
        objs.append(obj)
    exe = os.path.join(OUT, "abi_check")
    flags = ["-O1", "-g", "-std=c++17", f"--offload-arch={pb.ARCH}", *HOST_SAN.split(),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    steps = []
    for src, obj in ((os.path.join(HERE, "abi_driver.cpp"), "abi_driver.o"),
                     (os.path.join(CSRC, "sage_api.hip"), "sage_api_san.o")):
        steps.append(["hipcc", *flags, "-x", "hip", "-c", src, "-o", os.path.join(OUT, obj)])
    steps.append(["hipcc", f"--offload-arch={pb.ARCH}", *HOST_SAN.split(), os.path.join(OUT, "abi_driver.o"),
                  os.path.join(OUT, "sage_api_san.o"), *objs, "-o", exe])
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("sanitizer build of the host code failed:\n" + r.stderr[-4000:])
    return exe


def build_oracle_san() -> str:
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"]
    subprocess.check_call(cmd)
    return lib


if __name__ == "__main__":
    print(build_abi_check())
    print(build_oracle_san())
